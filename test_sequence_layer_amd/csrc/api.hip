// C ABI of libttt.so: argument validation and kernel dispatch.
// The entry points and their contracts are documented in include/ttt.h.
#include <limits.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "../../include/ttt.h"
#include "ttt_internal.h"

// Scratch of ttt_linear_fwd_chunked_noalloc (chunk maps and start states):
// one copy per GPU the library runs on, held until the process ends.  In host
// code this name stands for a host-side shadow, not device memory: host code
// uses only the per-device address scratch_address() looks up.
__device__ __align__(256) unsigned char scratch[TTT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of each GPU's `scratch` (nullptr: not looked up yet)

// The device address of `scratch` on the GPU that owns `stream`, looked up once
// per device (hipGetSymbolAddress with that device current) and kept.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlaps(Range a, Range b) {
  if (a.bytes <= 0 || b.bytes <= 0 || a.p == nullptr || b.p == nullptr) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// a*b*c*... <= limit without overflow (all factors >= 0)
bool mul_ok(int64_t& acc, int64_t f, int64_t limit = (int64_t(1) << 46)) {
  if (f < 0) return false;
  if (f != 0 && acc > limit / f) return false;
  acc *= f;
  return true;
}

int64_t dtype_size(int32_t dt) { return dt == TTT_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == TTT_F32 || dt == TTT_BF16; }

// element extent of eta (last index + 1) for B, H, T >= 1
int64_t eta_extent(int64_t B, int64_t H, int64_t T, int64_t sb, int64_t sh, int64_t st) {
  return (B - 1) * sb + (H - 1) * sh + (T - 1) * st + 1;
}

enum Kernel { K_NONE, K_GENERIC, K_MFMA, K_MFMA32, K_PRIMAL };

constexpr uint32_t kRowFlags = TTT_FLAG_ROWS1 | TTT_FLAG_ROWS2 | TTT_FLAG_ROWS4;

Kernel pick_linear(const ttt::LinearArgs& a, uint32_t flags) {
  if (flags & TTT_FLAG_PRIMAL) return ttt::linear_primal_supported(a.d) ? K_PRIMAL : K_NONE;
  if (flags & TTT_FLAG_GENERIC) return ttt::linear_generic_supported(a.d, a.b) ? K_GENERIC : K_NONE;
  if (ttt::linear_mfma_supported(a)) return K_MFMA;
  if (flags & kRowFlags) return K_NONE;  // row blocks exist only in the bf16 matrix-core kernel
  if (ttt::linear_mfma_f32_supported(a)) return K_MFMA32;
  if (ttt::linear_generic_supported(a.d, a.b)) return K_GENERIC;
  return K_NONE;
}

// Row blocks per (sequence, head, chunk) of the matrix-core forward: the
// flag's count, else 1 (see TTT_FLAG_ROWS1 in ttt.h for why).
int row_blocks(uint32_t flags) {
  if (flags & TTT_FLAG_ROWS4) return 4;
  if (flags & TTT_FLAG_ROWS2) return 2;
  return 1;
}

ttt::LinearArgs make_linear_args(const ttt_linear_desc* d, const void* Q, const void* K, const void* V,
                                 const float* W0, const float* eta, const void* Z, const float* Wf) {
  ttt::LinearArgs a;
  a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.b = d->b;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.Q = Q; a.K = K; a.V = V; a.W0 = W0; a.w0_bstride = d->w0_batch_stride;
  a.eta = eta; a.esb = d->eta_stride_b; a.esh = d->eta_stride_h; a.est = d->eta_stride_t;
  a.Z = const_cast<void*>(Z); a.Wf = const_cast<float*>(Wf);
  a.nchunk = 1; a.mb1 = d->T / 16; a.Wstart = nullptr; a.maps = nullptr;
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f;
  a.Esave = nullptr;
  a.rb = row_blocks(d->flags);
  return a;
}

ttt_status validate_linear(const ttt_linear_desc* d, const void* Q, const void* K, const void* V,
                           const float* W0, const float* eta, const void* Z, const float* Wf,
                           Kernel* which) {
  if (which) *which = K_NONE;
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (d->T % d->b != 0) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if (d->flags & ~(static_cast<uint32_t>(TTT_FLAG_GENERIC | TTT_FLAG_PRIMAL) | kRowFlags)) return TTT_ERR_FLAGS;
  if ((d->flags & TTT_FLAG_GENERIC) && (d->flags & TTT_FLAG_PRIMAL)) return TTT_ERR_FLAGS;
  {
    const uint32_t rows = d->flags & kRowFlags;
    if (rows & (rows - 1)) return TTT_ERR_FLAGS;  // more than one row-block count
    if (rows && (d->flags & (TTT_FLAG_GENERIC | TTT_FLAG_PRIMAL))) return TTT_ERR_FLAGS;
  }
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  if (chains * row_blocks(d->flags) > INT_MAX) return TTT_ERR_SHAPE;  // workgroups of one launch
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->d)) return TTT_ERR_SHAPE;
  const int64_t hdd = static_cast<int64_t>(d->H) * d->d * d->d;
  if (d->w0_batch_stride != 0 && d->w0_batch_stride != hdd) return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;

  ttt::LinearArgs a = make_linear_args(d, Q, K, V, W0, eta, Z, Wf);
  const Kernel k = pick_linear(a, d->flags);
  if (k == K_NONE) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) {
    if (which) *which = k;
    return TTT_OK;
  }

  // pointers
  if (!W0 || !Wf) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !V || !Z || !eta)) return TTT_ERR_NULL;
  if (!aligned(W0, 16) || !aligned(Wf, 16)) return TTT_ERR_ALIGN;
  if (tok > 0 && (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Z, 16) || !aligned(eta, 4)))
    return TTT_ERR_ALIGN;

  // extents and aliasing
  const int64_t in_b = tok * dtype_size(d->in_dtype);
  const int64_t z_b = tok * dtype_size(d->out_dtype);
  const int64_t wf_b = wel * 4;
  const int64_t w0_b = (d->w0_batch_stride == 0 ? hdd : wel) * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range rq{Q, in_b}, rk{K, in_b}, rv{V, in_b}, re{eta, eta_b}, rw0{W0, w0_b};
  const Range rz{Z, z_b}, rwf{Wf, wf_b};
  for (Range in : {rq, rk, rv, re, rw0})
    if (overlaps(rz, in)) return TTT_ERR_ALIAS;
  if (overlaps(rz, rwf)) return TTT_ERR_ALIAS;
  for (Range in : {rq, rk, rv, re})
    if (overlaps(rwf, in)) return TTT_ERR_ALIAS;
  if (overlaps(rwf, rw0)) {
    const bool inplace = static_cast<const void*>(Wf) == static_cast<const void*>(W0) && d->w0_batch_stride == hdd;
    if (!inplace) return TTT_ERR_ALIAS;
  }
  if (which) *which = k;
  return TTT_OK;
}

ttt::PrimalArgs make_primal_args_fwd(const ttt_linear_desc* d, const void* Q, const void* K, const void* V,
                                     const float* W0, const float* eta, void* Z, float* Wf) {
  ttt::PrimalArgs a;
  a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.b = d->b;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.W_in = W0; a.Wb_in = W0; a.w_in_bstride = d->w0_batch_stride;
  a.eta = eta; a.esb = d->eta_stride_b; a.esh = d->eta_stride_h; a.est = d->eta_stride_t;
  a.Z = Z; a.W_out = Wf; a.Wb_out = nullptr; a.pos = 0;
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f;
  return a;
}

ttt_status validate_decode(const ttt_linear_desc* d, const void* Q, const void* K, const void* V, const float* eta,
                           const void* Z, const float* W, const float* Wb, int64_t pos) {
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if (d->flags != 0) return TTT_ERR_FLAGS;
  if (pos < 0) return TTT_ERR_POS;
  if (d->w0_batch_stride != 0) return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->d)) return TTT_ERR_SHAPE;
  if (!ttt::linear_primal_supported(d->d)) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) return TTT_OK;
  if (!W || !Wb) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !V || !Z || !eta)) return TTT_ERR_NULL;
  if (!aligned(W, 16) || !aligned(Wb, 16)) return TTT_ERR_ALIGN;
  if (tok > 0 && (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Z, 16) || !aligned(eta, 4)))
    return TTT_ERR_ALIGN;
  const int64_t in_b = tok * dtype_size(d->in_dtype);
  const int64_t z_b = tok * dtype_size(d->out_dtype);
  const int64_t w_b = wel * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range rq{Q, in_b}, rk{K, in_b}, rv{V, in_b}, re{eta, eta_b}, rz{Z, z_b}, rw{W, w_b}, rwb{Wb, w_b};
  for (Range out : {rz, rw, rwb})
    for (Range in : {rq, rk, rv, re})
      if (overlaps(out, in)) return TTT_ERR_ALIAS;
  if (overlaps(rz, rw) || overlaps(rz, rwb) || overlaps(rw, rwb)) return TTT_ERR_ALIAS;
  return TTT_OK;
}

// Layer-norm parameters: finite eps >= 0, gamma and beta [H, d] fp32, non-NULL,
// 4-byte aligned, overlapping none of the outputs.
ttt_status check_ln(int64_t chains, int64_t H, int64_t d, const float* gamma, const float* beta, float eps,
                    std::initializer_list<Range> outs) {
  if (!(eps >= 0.f) || eps > 1e30f) return TTT_ERR_SHAPE;
  if (chains == 0) return TTT_OK;
  if (!gamma || !beta) return TTT_ERR_NULL;
  if (!aligned(gamma, 4) || !aligned(beta, 4)) return TTT_ERR_ALIGN;
  const int64_t hd_b = H * d * 4;
  for (Range out : outs)
    for (Range in : {Range{gamma, hd_b}, Range{beta, hd_b}})
      if (overlaps(out, in)) return TTT_ERR_ALIAS;
  return TTT_OK;
}

ttt_status check_ln_params(const ttt_linear_desc* d, const float* gamma, const float* beta, float eps,
                           std::initializer_list<Range> outs) {
  return check_ln(static_cast<int64_t>(d->B) * d->H, d->H, d->d, gamma, beta, eps, outs);
}

ttt_status validate_ln_decode(const ttt_linear_desc* d, const void* Q, const void* K, const void* V,
                              const float* eta, const float* gamma, const float* beta, float eps, const void* Z,
                              const float* W, const float* Wb, int64_t pos) {
  const ttt_status st = validate_decode(d, Q, K, V, eta, Z, W, Wb, pos);
  if (st != TTT_OK) return st;
  const int64_t chains = static_cast<int64_t>(d->B) * d->H;
  const int64_t w_b = chains * d->d * d->d * 4;
  return check_ln_params(d, gamma, beta, eps,
                         {Range{Z, chains * d->T * d->d * dtype_size(d->out_dtype)}, Range{W, w_b}, Range{Wb, w_b}});
}

ttt::PrimalArgs make_decode_args(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                 const float* eta, void* Z, float* W, float* Wb, int64_t pos) {
  ttt::PrimalArgs a;
  a.B = desc->B; a.H = desc->H; a.T = desc->T; a.d = desc->d; a.b = desc->b;
  a.in_dtype = desc->in_dtype; a.out_dtype = desc->out_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.W_in = W; a.Wb_in = Wb; a.w_in_bstride = static_cast<int64_t>(desc->H) * desc->d * desc->d;
  a.eta = eta; a.esb = desc->eta_stride_b; a.esh = desc->eta_stride_h; a.est = desc->eta_stride_t;
  a.Z = Z; a.W_out = W; a.Wb_out = Wb; a.pos = pos;
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f;
  return a;
}

// ----------------------------------------------------------- backward --

enum BwdKernel { KB_NONE, KB_GENERIC, KB_MFMA };

ttt::BwdArgs make_bwd_args(const ttt_linear_desc* d, const void* Q, const void* K, const float* eta,
                           const float* Wf, const float* E, const void* dZ, const float* dWf, void* dQ, void* dK,
                           void* dV, float* deta, float* dW0) {
  ttt::BwdArgs a;
  a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.b = d->b;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.Q = Q; a.K = K;
  a.eta = eta; a.esb = d->eta_stride_b; a.esh = d->eta_stride_h; a.est = d->eta_stride_t;
  a.Wf = Wf; a.E = E; a.dZ = dZ; a.dWf = dWf;
  a.dQ = dQ; a.dK = dK; a.dV = dV; a.deta = deta; a.dW0 = dW0;
  a.V = nullptr; a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f; a.dgamma = nullptr; a.dbeta = nullptr;
  return a;
}

BwdKernel pick_bwd(const ttt::BwdArgs& a, uint32_t flags) {
  if (!(flags & TTT_FLAG_GENERIC) && ttt::linear_bwd_mfma_supported(a)) return KB_MFMA;
  if (ttt::linear_bwd_generic_supported(a.d, a.b)) return KB_GENERIC;
  return KB_NONE;
}

ttt_status validate_bwd(const ttt_linear_desc* d, const void* Q, const void* K, const float* eta, const float* Wf,
                        const float* E, const void* dZ, const float* dWf, const void* dQ, const void* dK,
                        const void* dV, const float* deta, const float* dW0, BwdKernel* which) {
  if (which) *which = KB_NONE;
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (d->T % d->b != 0) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if (d->flags & ~static_cast<uint32_t>(TTT_FLAG_GENERIC)) return TTT_ERR_FLAGS;
  if (d->w0_batch_stride != 0 && d->w0_batch_stride != static_cast<int64_t>(d->H) * d->d * d->d)
    return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->d)) return TTT_ERR_SHAPE;
  const ttt::BwdArgs a = make_bwd_args(d, Q, K, eta, Wf, E, dZ, dWf, nullptr, nullptr, nullptr, nullptr, nullptr);
  const BwdKernel k = pick_bwd(a, d->flags);
  if (k == KB_NONE) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) {
    if (which) *which = k;
    return TTT_OK;
  }
  if (!Wf || !dW0) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !eta || !E || !dZ || !dQ || !dK || !dV || !deta)) return TTT_ERR_NULL;
  if (!aligned(Wf, 16) || !aligned(dW0, 16) || (dWf && !aligned(dWf, 16))) return TTT_ERR_ALIGN;
  if (tok > 0) {
    for (const void* p : {Q, K, static_cast<const void*>(E), dZ, dQ, dK, dV})
      if (!aligned(p, 16)) return TTT_ERR_ALIGN;
    if (!aligned(eta, 4) || !aligned(deta, 4)) return TTT_ERR_ALIGN;
  }
  const int64_t in_b = tok * dtype_size(d->in_dtype);
  const int64_t g_b = tok * dtype_size(d->out_dtype);
  const int64_t w_b = wel * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const int64_t deta_b = tok > 0 ? chains * d->T * 4 : 0;
  const Range ins[] = {{Q, in_b}, {K, in_b}, {eta, eta_b}, {Wf, w_b}, {E, tok * 4}, {dZ, g_b}, {dWf, w_b}};
  const Range outs[] = {{dQ, g_b}, {dK, g_b}, {dV, g_b}, {deta, deta_b}, {dW0, w_b}};
  for (int i = 0; i < 5; ++i) {
    for (const Range& in : ins)
      if (overlaps(outs[i], in)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
  }
  if (which) *which = k;
  return TTT_OK;
}

// ---------------------------------------------------------------- MLP --

ttt::MlpArgs make_mlp_args(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V, const float* W1,
                           const float* W2, const float* eta, const void* Z, const float* W1f, const float* W2f) {
  ttt::MlpArgs a;
  a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.dh = d->dh; a.b = d->b;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.Q = Q; a.K = K; a.V = V; a.W1 = W1; a.W2 = W2; a.w_bstride = d->w_batch_stride;
  a.eta = eta; a.esb = d->eta_stride_b; a.esh = d->eta_stride_h; a.est = d->eta_stride_t;
  a.Z = const_cast<void*>(Z); a.W1f = const_cast<float*>(W1f); a.W2f = const_cast<float*>(W2f);
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f;
  a.ckpt = nullptr;
  return a;
}

ttt_status validate_mlp(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V, const float* W1,
                        const float* W2, const float* eta, const void* Z, const float* W1f, const float* W2f,
                        bool* ok_kernel) {
  if (ok_kernel) *ok_kernel = false;
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->dh < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (d->T % d->b != 0) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if ((d->flags & ~static_cast<uint32_t>(TTT_FLAG_PRIMAL)) != 0 || d->reserved != 0) return TTT_ERR_FLAGS;
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->dh)) return TTT_ERR_SHAPE;
  const int64_t hw = static_cast<int64_t>(d->H) * d->d * d->dh;
  if (d->w_batch_stride != 0 && d->w_batch_stride != hw) return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;
  ttt::MlpArgs a = make_mlp_args(d, Q, K, V, W1, W2, eta, Z, W1f, W2f);
  const bool supported =
      (d->flags & TTT_FLAG_PRIMAL) ? ttt::mlp_primal_supported(d->d, d->dh) : ttt::mlp_supported(a);
  if (!supported) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) {
    if (ok_kernel) *ok_kernel = true;
    return TTT_OK;
  }
  if (!W1 || !W2 || !W1f || !W2f) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !V || !Z || !eta)) return TTT_ERR_NULL;
  for (const void* p : {static_cast<const void*>(W1), static_cast<const void*>(W2),
                        static_cast<const void*>(W1f), static_cast<const void*>(W2f)})
    if (!aligned(p, 16)) return TTT_ERR_ALIGN;
  if (tok > 0 && (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Z, 16) || !aligned(eta, 4)))
    return TTT_ERR_ALIGN;
  const int64_t in_b = tok * dtype_size(d->in_dtype);
  const int64_t z_b = tok * dtype_size(d->out_dtype);
  const int64_t wf_b = wel * 4;
  const int64_t w0_b = (d->w_batch_stride == 0 ? hw : wel) * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range rq{Q, in_b}, rk{K, in_b}, rv{V, in_b}, re{eta, eta_b}, rw1{W1, w0_b}, rw2{W2, w0_b};
  const Range rz{Z, z_b}, rf1{W1f, wf_b}, rf2{W2f, wf_b};
  for (Range out : {rz, rf1, rf2}) {
    for (Range in : {rq, rk, rv, re})
      if (overlaps(out, in)) return TTT_ERR_ALIAS;
  }
  if (overlaps(rz, rf1) || overlaps(rz, rf2) || overlaps(rf1, rf2)) return TTT_ERR_ALIAS;
  if (overlaps(rz, rw1) || overlaps(rz, rw2)) return TTT_ERR_ALIAS;
  const bool per_seq = d->w_batch_stride == hw;
  if (overlaps(rf1, rw1) && !(per_seq && static_cast<const void*>(W1f) == static_cast<const void*>(W1)))
    return TTT_ERR_ALIAS;
  if (overlaps(rf2, rw2) && !(per_seq && static_cast<const void*>(W2f) == static_cast<const void*>(W2)))
    return TTT_ERR_ALIAS;
  if (overlaps(rf1, rw2) || overlaps(rf2, rw1)) return TTT_ERR_ALIAS;
  if (ok_kernel) *ok_kernel = true;
  return TTT_OK;
}

}  // namespace

extern "C" {

int ttt_abi_version(void) { return TTT_ABI_VERSION; }

const char* ttt_status_str(int s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_NULL: return "a required pointer is NULL";
    case TTT_ERR_SHAPE: return "invalid shape (negative size, b < 1, T % b != 0 or size overflow)";
    case TTT_ERR_DTYPE: return "invalid dtype code";
    case TTT_ERR_UNSUPPORTED: return "no kernel is built for this (d, b, dtype) combination";
    case TTT_ERR_ALIAS: return "an output overlaps an input";
    case TTT_ERR_ALIGN: return "a pointer is misaligned (16 bytes for tensors, 4 for eta)";
    case TTT_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case TTT_ERR_STRIDE: return "invalid stride";
    case TTT_ERR_FLAGS: return "unknown flag or non-zero reserved field";
    case TTT_ERR_POS: return "negative decode position";
    case TTT_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TTT_ERR_SCRATCH:
      return "the call needs more than the library's static scratch (TTT_NOALLOC_SCRATCH_BYTES); "
             "use ttt_linear_fwd_chunked with a workspace, or fewer chunks";
    default: return "unknown status";
  }
}

ttt_status ttt_linear_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                               const float* W0, const float* eta, const void* Z, const float* W_final) {
  return validate_linear(desc, Q, K, V, W0, eta, Z, W_final, nullptr);
}

const char* ttt_linear_kernel_name(const ttt_linear_desc* d) {
  if (!d) return nullptr;
  ttt::LinearArgs a = make_linear_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  switch (pick_linear(a, d->flags)) {
    case K_MFMA: return ttt::linear_mfma_name(a);
    case K_MFMA32: return "ttt_linear_mfma_f32_d64b16";
    case K_GENERIC: return ttt::linear_generic_name(a.d);
    case K_PRIMAL: return ttt::linear_primal_name(a.d);
    default: return nullptr;
  }
}

ttt_status ttt_linear_fwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W0, const float* eta, void* Z, float* W_final, void* stream) {
  Kernel k;
  const ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (k == K_MFMA)
    e = ttt::launch_linear_mfma(a, s);
  else if (k == K_MFMA32)
    e = ttt::launch_linear_mfma_f32(a, s);
  else if (k == K_PRIMAL)
    e = ttt::launch_linear_primal(make_primal_args_fwd(desc, Q, K, V, W0, eta, Z, W_final), s);
  else
    e = ttt::launch_linear_generic(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

namespace {

// Checks of a forward's saved-for-backward buffer (fp32, one value per token
// and output): non-NULL, 16-byte aligned, overlapping no input or output.
ttt_status check_saved(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V, const float* W0,
                       const float* eta, const void* Z, const float* W_final, const float* saved) {
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  const int64_t tok = chains * desc->T * desc->d;
  if (tok == 0) return TTT_OK;
  if (!saved) return TTT_ERR_NULL;
  if (!aligned(saved, 16)) return TTT_ERR_ALIGN;
  const int64_t in_b = tok * dtype_size(desc->in_dtype), z_b = tok * dtype_size(desc->out_dtype);
  const int64_t hdd = static_cast<int64_t>(desc->H) * desc->d * desc->d;
  const int64_t w0_b = (desc->w0_batch_stride == 0 ? hdd : chains * desc->d * desc->d) * 4;
  const int64_t eta_b =
      eta_extent(desc->B, desc->H, desc->T, desc->eta_stride_b, desc->eta_stride_h, desc->eta_stride_t) * 4;
  const Range re{saved, tok * 4};
  for (Range r : {Range{Q, in_b}, Range{K, in_b}, Range{V, in_b}, Range{eta, eta_b}, Range{W0, w0_b},
                  Range{Z, z_b}, Range{W_final, chains * desc->d * desc->d * 4}})
    if (overlaps(re, r)) return TTT_ERR_ALIAS;
  return TTT_OK;
}

}  // namespace

ttt_status ttt_linear_fwd_save(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                               const float* W0, const float* eta, void* Z, float* W_final, float* E_saved,
                               void* stream) {
  Kernel k;
  ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (desc->flags & TTT_FLAG_PRIMAL) return TTT_ERR_FLAGS;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  st = check_saved(desc, Q, K, V, W0, eta, Z, W_final, E_saved);
  if (st != TTT_OK) return st;
  const int64_t tok = chains * desc->T * desc->d;
  ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  a.Esave = tok > 0 ? E_saved : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = k == K_MFMA ? ttt::launch_linear_mfma(a, s) : ttt::launch_linear_generic(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_linear_bwd_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const float* eta,
                                   const float* W_final, const float* E_saved, const void* dZ,
                                   const float* dW_final, const void* dQ, const void* dK, const void* dV,
                                   const float* deta, const float* dW0) {
  return validate_bwd(desc, Q, K, eta, W_final, E_saved, dZ, dW_final, dQ, dK, dV, deta, dW0, nullptr);
}

const char* ttt_linear_bwd_kernel_name(const ttt_linear_desc* d) {
  if (!d) return nullptr;
  const ttt::BwdArgs a = make_bwd_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr);
  switch (pick_bwd(a, d->flags)) {
    case KB_MFMA: return "ttt_linear_bwd_d64b16";
    case KB_GENERIC: return ttt::linear_bwd_generic_name(a.d);
    default: return nullptr;
  }
}

ttt_status ttt_linear_bwd(const ttt_linear_desc* desc, const void* Q, const void* K, const float* eta,
                          const float* W_final, const float* E_saved, const void* dZ, const float* dW_final,
                          void* dQ, void* dK, void* dV, float* deta, float* dW0, void* stream) {
  BwdKernel k;
  const ttt_status st =
      validate_bwd(desc, Q, K, eta, W_final, E_saved, dZ, dW_final, dQ, dK, dV, deta, dW0, &k);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const ttt::BwdArgs a = make_bwd_args(desc, Q, K, eta, W_final, E_saved, dZ, dW_final, dQ, dK, dV, deta, dW0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = k == KB_MFMA ? ttt::launch_linear_bwd_mfma(a, s) : ttt::launch_linear_bwd_generic(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

namespace {

// Every check of the layer-norm forward (the plain forward's, then its own).
ttt_status validate_ln(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V, const float* W0,
                       const float* gamma, const float* beta, float eps, const float* eta, const void* Z,
                       const float* W_final) {
  Kernel k;
  const ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  const bool ok = (desc->flags == 0 && k == K_MFMA) || (desc->flags == TTT_FLAG_PRIMAL && k == K_PRIMAL);
  if (!ok) return TTT_ERR_UNSUPPORTED;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  const int64_t z_b = chains * desc->T * desc->d * dtype_size(desc->out_dtype);
  return check_ln_params(desc, gamma, beta, eps, {Range{Z, z_b}, Range{W_final, chains * desc->d * desc->d * 4}});
}

hipError_t launch_ln(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V, const float* W0,
                     const float* gamma, const float* beta, float eps, const float* eta, void* Z, float* W_final,
                     float* saved, void* stream) {
  if (desc->flags & TTT_FLAG_PRIMAL) {
    ttt::PrimalArgs p = make_primal_args_fwd(desc, Q, K, V, W0, eta, Z, W_final);
    p.gamma = gamma; p.beta = beta; p.eps = eps;
    return ttt::launch_linear_primal(p, static_cast<hipStream_t>(stream));
  }
  ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.rb = 1;
  a.Esave = saved;
  return ttt::launch_linear_mfma(a, static_cast<hipStream_t>(stream));
}

}  // namespace

const char* ttt_linear_ln_kernel_name(const ttt_linear_desc* d) {
  if (!d) return nullptr;
  ttt::LinearArgs a = make_linear_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  const Kernel k = pick_linear(a, d->flags);
  if (d->flags == 0 && k == K_MFMA) return "ttt_linear_mfma_d64b16 (layer norm)";
  if (d->flags == TTT_FLAG_PRIMAL && k == K_PRIMAL) return ttt::linear_primal_name(a.d, true);
  return nullptr;
}

ttt_status ttt_linear_ln_fwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* W0, const float* gamma, const float* beta, float eps, const float* eta,
                             void* Z, float* W_final, void* stream) {
  const ttt_status st = validate_ln(desc, Q, K, V, W0, gamma, beta, eps, eta, Z, W_final);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const hipError_t e = launch_ln(desc, Q, K, V, W0, gamma, beta, eps, eta, Z, W_final, nullptr, stream);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_linear_ln_fwd_save(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                  const float* W0, const float* gamma, const float* beta, float eps,
                                  const float* eta, void* Z, float* W_final, float* G_saved, void* stream) {
  ttt_status st = validate_ln(desc, Q, K, V, W0, gamma, beta, eps, eta, Z, W_final);
  if (st != TTT_OK) return st;
  if (desc->flags != 0) return TTT_ERR_UNSUPPORTED;  // the primal kernel saves nothing
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  st = check_saved(desc, Q, K, V, W0, eta, Z, W_final, G_saved);
  if (st != TTT_OK) return st;
  const int64_t hd_b = static_cast<int64_t>(desc->H) * desc->d * 4;
  const Range rd{G_saved, chains * desc->T * desc->d * 4};
  if (overlaps(rd, Range{gamma, hd_b}) || overlaps(rd, Range{beta, hd_b})) return TTT_ERR_ALIAS;
  const bool any = chains * desc->T > 0;
  const hipError_t e =
      launch_ln(desc, Q, K, V, W0, gamma, beta, eps, eta, Z, W_final, any ? G_saved : nullptr, stream);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

namespace {

// Every check of the layer-norm backward: the plain backward's (with the saved
// delta in E's place), then V, gamma, beta, eps and the two extra outputs.
ttt_status validate_ln_bwd(const ttt_linear_desc* d, const void* Q, const void* K, const void* V, const float* eta,
                           const float* gamma, const float* beta, float eps, const float* Wf, const float* Ds,
                           const void* dZ, const float* dWf, const void* dQ, const void* dK, const void* dV,
                           const float* deta, const float* dW0, const float* dgamma, const float* dbeta) {
  BwdKernel k;
  const ttt_status st = validate_bwd(d, Q, K, eta, Wf, Ds, dZ, dWf, dQ, dK, dV, deta, dW0, &k);
  if (st != TTT_OK) return st;
  ttt::BwdArgs a = make_bwd_args(d, Q, K, eta, Wf, Ds, dZ, dWf, nullptr, nullptr, nullptr, nullptr, nullptr);
  if ((d->flags & ~static_cast<uint32_t>(TTT_FLAG_GENERIC)) != 0 || !ttt::linear_ln_bwd_supported(a))
    return TTT_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps > 1e30f) return TTT_ERR_SHAPE;
  const int64_t chains = static_cast<int64_t>(d->B) * d->H;
  if (chains == 0) return TTT_OK;
  const int64_t tok = chains * d->T * d->d;
  if (!gamma || !beta || !dgamma || !dbeta || (tok > 0 && !V)) return TTT_ERR_NULL;
  if (!aligned(gamma, 4) || !aligned(beta, 4) || !aligned(dgamma, 4) || !aligned(dbeta, 4)) return TTT_ERR_ALIGN;
  if (tok > 0 && !aligned(V, 16)) return TTT_ERR_ALIGN;
  const int64_t in_b = tok * dtype_size(d->in_dtype), g_b = tok * dtype_size(d->out_dtype);
  const int64_t hd_b = static_cast<int64_t>(d->H) * d->d * 4, cd_b = chains * d->d * 4;
  const int64_t w_b = chains * d->d * d->d * 4;
  const int64_t eta_b = tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range ins[] = {{Q, in_b}, {K, in_b}, {V, in_b}, {eta, eta_b}, {gamma, hd_b}, {beta, hd_b}, {Wf, w_b},
                       {Ds, tok * 4}, {dZ, g_b}, {dWf, w_b}};
  const Range outs[] = {{dQ, g_b}, {dK, g_b}, {dV, g_b}, {deta, tok > 0 ? chains * d->T * 4 : 0}, {dW0, w_b},
                        {dgamma, cd_b}, {dbeta, cd_b}};
  for (int i = 0; i < 7; ++i) {
    for (const Range& in : ins)
      if (overlaps(outs[i], in)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
  }
  return TTT_OK;
}

}  // namespace

ttt_status ttt_linear_ln_bwd_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const float* gamma, const float* beta, float eps,
                                      const float* W_final, const float* G_saved, const void* dZ,
                                      const float* dW_final, const void* dQ, const void* dK, const void* dV,
                                      const float* deta, const float* dW0, const float* dgamma,
                                      const float* dbeta) {
  return validate_ln_bwd(desc, Q, K, V, eta, gamma, beta, eps, W_final, G_saved, dZ, dW_final, dQ, dK, dV,
                         deta, dW0, dgamma, dbeta);
}

const char* ttt_linear_ln_bwd_kernel_name(const ttt_linear_desc* d) {
  if (!d || (d->flags & ~static_cast<uint32_t>(TTT_FLAG_GENERIC)) != 0) return nullptr;
  const ttt::BwdArgs a = make_bwd_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr);
  if (!ttt::linear_ln_bwd_supported(a)) return nullptr;
  return (d->flags & TTT_FLAG_GENERIC) ? "ttt_linear_ln_bwd_fp32" : "ttt_linear_ln_bwd_d64b16";
}

ttt_status ttt_linear_ln_bwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, const float* gamma, const float* beta, float eps,
                             const float* W_final, const float* G_saved, const void* dZ, const float* dW_final,
                             void* dQ, void* dK, void* dV, float* deta, float* dW0, float* dgamma, float* dbeta,
                             void* stream) {
  const ttt_status st = validate_ln_bwd(desc, Q, K, V, eta, gamma, beta, eps, W_final, G_saved, dZ, dW_final,
                                        dQ, dK, dV, deta, dW0, dgamma, dbeta);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  ttt::BwdArgs a =
      make_bwd_args(desc, Q, K, eta, W_final, G_saved, dZ, dW_final, dQ, dK, dV, deta, dW0);
  a.V = V;
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.dgamma = dgamma;
  a.dbeta = dbeta;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      (desc->flags & TTT_FLAG_GENERIC) ? ttt::launch_linear_ln_bwd(a, s) : ttt::launch_linear_ln_bwd_mfma(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int64_t ttt_linear_chunked_workspace_bytes(const ttt_linear_desc* desc, int32_t nchunks) {
  if (!desc || nchunks < 1 || desc->B < 0 || desc->H < 0 || desc->d < 1) return -1;
  if (nchunks == 1) return 0;
  // maps (P, R) of chunks 1 .. n-2 and start states of chunks 1 .. n-1
  const int64_t per_chain = (static_cast<int64_t>(nchunks - 2) * 2 + (nchunks - 1)) * desc->d * desc->d * 4;
  return static_cast<int64_t>(desc->B) * desc->H * per_chain;
}

namespace {

// Argument checks of the chunked forward (everything but the workspace).
ttt_status validate_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K,
                            const void* V, const float* W0, const float* eta, const void* Z, const float* W_final) {
  Kernel k;
  ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (nchunks < 1 || nchunks > desc->T / 16) {  // every chunk holds at least one mini-batch
    if (!(nchunks == 1 && desc->T == 0)) return TTT_ERR_SHAPE;
  }
  if ((desc->flags & ~kRowFlags) != 0 || k != K_MFMA) return TTT_ERR_UNSUPPORTED;
  // workgroups of the launches (nchunks - 1 units per chain, row blocks in the last)
  if (static_cast<int64_t>(desc->B) * desc->H * nchunks * row_blocks(desc->flags) > INT_MAX)
    return TTT_ERR_SHAPE;
  return TTT_OK;
}

// Mini-batches of chunk 0 of a chunked forward.  Its workgroup runs the plain
// forward in the first launch while the others compute two maps each, which
// measured ~10% slower per mini-batch on MI355X (219 against 198 us for 410
// mini-batches), so with maps in that launch chunk 0 gets ~1.1 shares of the
// sequence and the other chunks one each; every chunk keeps at least one.
int64_t chunk0_minibatches(int64_t nb, int32_t nchunks) {
  const double share = nchunks > 2 ? 1.1 : 1.0;
  int64_t mb1 = static_cast<int64_t>(static_cast<double>(nb) * share / (nchunks - 1 + share) + 0.5);
  if (mb1 < 1) mb1 = 1;
  if (mb1 > nb - (nchunks - 1)) mb1 = nb - (nchunks - 1);
  return mb1;
}

// The chunked forward's launches, after validate_chunked, nchunks > 1 and
// B*H > 0, with a workspace of at least the bytes it needs.
ttt_status run_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K, const void* V,
                       const float* W0, const float* eta, void* Z, float* W_final, void* workspace,
                       void* stream);

}  // namespace

ttt_status ttt_linear_fwd_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K,
                                  const void* V, const float* W0, const float* eta, void* Z, float* W_final,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  ttt_status st = validate_chunked(desc, nchunks, Q, K, V, W0, eta, Z, W_final);
  if (st != TTT_OK) return st;
  if (nchunks == 1) return ttt_linear_fwd(desc, Q, K, V, W0, eta, Z, W_final, stream);
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  const int64_t need = ttt_linear_chunked_workspace_bytes(desc, nchunks);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return TTT_ERR_WORKSPACE;
  {
    const int64_t tok = chains * desc->T * desc->d;
    const int64_t in_b = tok * dtype_size(desc->in_dtype), z_b = tok * dtype_size(desc->out_dtype);
    const int64_t hdd = static_cast<int64_t>(desc->H) * desc->d * desc->d;
    const int64_t w0_b = (desc->w0_batch_stride == 0 ? hdd : chains * desc->d * desc->d) * 4;
    const int64_t eta_b = tok > 0 ? eta_extent(desc->B, desc->H, desc->T, desc->eta_stride_b, desc->eta_stride_h,
                                               desc->eta_stride_t) * 4 : 0;
    const Range rw{workspace, need};
    for (Range r : {Range{Q, in_b}, Range{K, in_b}, Range{V, in_b}, Range{eta, eta_b}, Range{W0, w0_b},
                    Range{Z, z_b}, Range{W_final, chains * desc->d * desc->d * 4}})
      if (overlaps(rw, r)) return TTT_ERR_ALIAS;
  }
  return run_chunked(desc, nchunks, Q, K, V, W0, eta, Z, W_final, workspace, stream);
}

ttt_status ttt_linear_fwd_chunked_noalloc(const ttt_linear_desc* desc, int32_t nchunks, const void* Q,
                                          const void* K, const void* V, const float* W0, const float* eta,
                                          void* Z, float* W_final, void* stream) {
  ttt_status st = validate_chunked(desc, nchunks, Q, K, V, W0, eta, Z, W_final);
  if (st != TTT_OK) return st;
  if (nchunks == 1) return ttt_linear_fwd(desc, Q, K, V, W0, eta, Z, W_final, stream);
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  if (ttt_linear_chunked_workspace_bytes(desc, nchunks) > TTT_NOALLOC_SCRATCH_BYTES) return TTT_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return TTT_ERR_HIP;
  // (the chunked passes write every map and start state before reading it, so
  // the scratch needs no clearing between calls)
  return run_chunked(desc, nchunks, Q, K, V, W0, eta, Z, W_final, ws, stream);
}

namespace {

ttt_status run_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K, const void* V,
                       const float* W0, const float* eta, void* Z, float* W_final, void* workspace,
                       void* stream) {
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  a.nchunk = nchunks;
  a.mb1 = chunk0_minibatches(desc->T / 16, nchunks);
  a.maps = static_cast<float*>(workspace);
  a.Wstart = a.maps + chains * (nchunks - 2) * 2 * desc->d * desc->d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // chunk 0 and the maps of chunks 1 .. n-2 (one workgroup per unit; the row
  // block flag applies to the last launch only)
  ttt::LinearArgs a1 = a;
  a1.rb = 1;
  hipError_t e = ttt::launch_linear_mfma_head_maps(a1, s);
  if (e == hipSuccess && nchunks > 2) e = ttt::launch_linear_chunk_scan(a, s);
  if (e == hipSuccess) e = ttt::launch_linear_mfma(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // namespace

ttt_status ttt_linear_decode_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const void* Z, const float* W, const float* Wb,
                                      int64_t pos) {
  return validate_decode(desc, Q, K, V, eta, Z, W, Wb, pos);
}

ttt_status ttt_linear_decode(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, void* Z, float* W, float* Wb, int64_t pos, void* stream) {
  const ttt_status st = validate_decode(desc, Q, K, V, eta, Z, W, Wb, pos);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const hipError_t e =
      ttt::launch_linear_primal(make_decode_args(desc, Q, K, V, eta, Z, W, Wb, pos), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_linear_ln_decode_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                         const float* eta, const float* gamma, const float* beta, float eps,
                                         const void* Z, const float* W, const float* Wb, int64_t pos) {
  return validate_ln_decode(desc, Q, K, V, eta, gamma, beta, eps, Z, W, Wb, pos);
}

ttt_status ttt_linear_ln_decode(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                const float* eta, const float* gamma, const float* beta, float eps, void* Z,
                                float* W, float* Wb, int64_t pos, void* stream) {
  const ttt_status st = validate_ln_decode(desc, Q, K, V, eta, gamma, beta, eps, Z, W, Wb, pos);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  ttt::PrimalArgs a = make_decode_args(desc, Q, K, V, eta, Z, W, Wb, pos);
  a.gamma = gamma; a.beta = beta; a.eps = eps;
  const hipError_t e = ttt::launch_linear_primal(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                            const float* W1_0, const float* W2_0, const float* eta, const void* Z,
                            const float* W1_final, const float* W2_final) {
  return validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, nullptr);
}

const char* ttt_mlp_ln_kernel_name(const ttt_mlp_desc* d) {
  if (!d) return nullptr;
  if (d->flags & TTT_FLAG_PRIMAL)
    return ttt::mlp_primal_supported(d->d, d->dh) ? "ttt_mlp_ln_primal_d64h256" : nullptr;
  ttt::MlpArgs a = make_mlp_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr);
  return ttt::mlp_supported(a) ? "ttt_mlp_fwd_d64h256b16 (layer norm)" : nullptr;
}

const char* ttt_mlp_kernel_name(const ttt_mlp_desc* d) {
  if (!d) return nullptr;
  if (d->flags & TTT_FLAG_PRIMAL) return ttt::mlp_primal_supported(d->d, d->dh) ? "ttt_mlp_primal_d64h256" : nullptr;
  ttt::MlpArgs a = make_mlp_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr);
  return ttt::mlp_supported(a) ? ttt::mlp_name(a) : nullptr;
}

namespace {

ttt::MlpPrimalArgs make_mlp_primal_args(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V,
                                        const float* eta, void* Z) {
  ttt::MlpPrimalArgs a;
  a.B = d->B; a.H = d->H; a.T = d->T; a.d = d->d; a.dh = d->dh; a.b = d->b;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.eta = eta; a.esb = d->eta_stride_b; a.esh = d->eta_stride_h; a.est = d->eta_stride_t;
  a.Z = Z;
  a.W1_in = a.W2_in = a.W1b_in = a.W2b_in = nullptr;
  a.W1_out = a.W2_out = a.W1b_out = a.W2b_out = nullptr;
  a.w_in_bstride = 0;
  a.pos = 0;
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f;
  return a;
}

ttt_status validate_mlp_decode(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V,
                               const float* eta, const void* Z, const float* W1, const float* W2, const float* W1b,
                               const float* W2b, int64_t pos) {
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->dh < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if (d->flags != 0 || d->reserved != 0) return TTT_ERR_FLAGS;
  if (pos < 0) return TTT_ERR_POS;
  if (d->w_batch_stride != 0) return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->dh)) return TTT_ERR_SHAPE;
  if (!ttt::mlp_primal_supported(d->d, d->dh)) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) return TTT_OK;
  if (!W1 || !W2 || !W1b || !W2b) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !V || !Z || !eta)) return TTT_ERR_NULL;
  for (const float* p : {W1, W2, W1b, W2b})
    if (!aligned(p, 16)) return TTT_ERR_ALIGN;
  if (tok > 0 && (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Z, 16) || !aligned(eta, 4)))
    return TTT_ERR_ALIGN;
  const int64_t in_b = tok * dtype_size(d->in_dtype);
  const int64_t z_b = tok * dtype_size(d->out_dtype);
  const int64_t w_b = wel * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range ins[] = {{Q, in_b}, {K, in_b}, {V, in_b}, {eta, eta_b}};
  const Range outs[] = {{Z, z_b}, {W1, w_b}, {W2, w_b}, {W1b, w_b}, {W2b, w_b}};
  for (int i = 0; i < 5; ++i) {
    for (const Range& in : ins)
      if (overlaps(outs[i], in)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
  }
  return TTT_OK;
}

ttt_status validate_mlp_ln_decode(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V,
                                  const float* eta, const float* gamma, const float* beta, float eps, const void* Z,
                                  const float* W1, const float* W2, const float* W1b, const float* W2b,
                                  int64_t pos) {
  const ttt_status st = validate_mlp_decode(d, Q, K, V, eta, Z, W1, W2, W1b, W2b, pos);
  if (st != TTT_OK) return st;
  const int64_t chains = static_cast<int64_t>(d->B) * d->H;
  const int64_t w_b = chains * d->d * d->dh * 4;
  return check_ln(chains, d->H, d->d, gamma, beta, eps,
                  {Range{Z, chains * d->T * d->d * dtype_size(d->out_dtype)}, Range{W1, w_b}, Range{W2, w_b},
                   Range{W1b, w_b}, Range{W2b, w_b}});
}

ttt::MlpPrimalArgs make_mlp_decode_args(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                        const float* eta, void* Z, float* W1, float* W2, float* W1b, float* W2b,
                                        int64_t pos) {
  ttt::MlpPrimalArgs a = make_mlp_primal_args(desc, Q, K, V, eta, Z);
  a.W1_in = a.W1_out = W1;
  a.W2_in = a.W2_out = W2;
  a.W1b_in = a.W1b_out = W1b;
  a.W2b_in = a.W2b_out = W2b;
  a.w_in_bstride = static_cast<int64_t>(desc->H) * desc->d * desc->dh;
  a.pos = pos;
  return a;
}

}  // namespace

ttt_status ttt_mlp_decode_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                   const float* eta, const void* Z, const float* W1, const float* W2,
                                   const float* W1b, const float* W2b, int64_t pos) {
  return validate_mlp_decode(desc, Q, K, V, eta, Z, W1, W2, W1b, W2b, pos);
}

ttt_status ttt_mlp_decode(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* eta,
                          void* Z, float* W1, float* W2, float* W1b, float* W2b, int64_t pos, void* stream) {
  const ttt_status st = validate_mlp_decode(desc, Q, K, V, eta, Z, W1, W2, W1b, W2b, pos);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const hipError_t e = ttt::launch_mlp_primal(make_mlp_decode_args(desc, Q, K, V, eta, Z, W1, W2, W1b, W2b, pos),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_ln_decode_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const float* gamma, const float* beta, float eps,
                                      const void* Z, const float* W1, const float* W2, const float* W1b,
                                      const float* W2b, int64_t pos) {
  return validate_mlp_ln_decode(desc, Q, K, V, eta, gamma, beta, eps, Z, W1, W2, W1b, W2b, pos);
}

ttt_status ttt_mlp_ln_decode(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, const float* gamma, const float* beta, float eps, void* Z, float* W1,
                             float* W2, float* W1b, float* W2b, int64_t pos, void* stream) {
  const ttt_status st = validate_mlp_ln_decode(desc, Q, K, V, eta, gamma, beta, eps, Z, W1, W2, W1b, W2b, pos);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  ttt::MlpPrimalArgs a = make_mlp_decode_args(desc, Q, K, V, eta, Z, W1, W2, W1b, W2b, pos);
  a.gamma = gamma; a.beta = beta; a.eps = eps;
  const hipError_t e = ttt::launch_mlp_primal(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* W1_0,
                       const float* W2_0, const float* eta, void* Z, float* W1_final, float* W2_final,
                       void* stream) {
  bool ok;
  const ttt_status st = validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, &ok);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  if (desc->flags & TTT_FLAG_PRIMAL) {
    // token by token from W0 (the first token starts a mini-batch, so no
    // mini-batch-start state is read)
    ttt::MlpPrimalArgs p = make_mlp_primal_args(desc, Q, K, V, eta, Z);
    p.W1_in = p.W1b_in = W1_0;
    p.W2_in = p.W2b_in = W2_0;
    p.w_in_bstride = desc->w_batch_stride;
    p.W1_out = W1_final;
    p.W2_out = W2_final;
    const hipError_t e = ttt::launch_mlp_primal(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
  }
  const ttt::MlpArgs a = make_mlp_args(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final);
  const hipError_t e = ttt::launch_mlp(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_ln_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W1_0, const float* W2_0, const float* gamma, const float* beta, float eps,
                          const float* eta, void* Z, float* W1_final, float* W2_final, void* stream) {
  bool ok;
  ttt_status st = validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, &ok);
  if (st != TTT_OK) return st;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  const int64_t z_b = chains * desc->T * desc->d * dtype_size(desc->out_dtype);
  const int64_t w_b = chains * desc->d * desc->dh * 4;
  st = check_ln(chains, desc->H, desc->d, gamma, beta, eps,
                {Range{Z, z_b}, Range{W1_final, w_b}, Range{W2_final, w_b}});
  if (st != TTT_OK || chains == 0) return st;
  if (desc->flags & TTT_FLAG_PRIMAL) {
    ttt::MlpPrimalArgs p = make_mlp_primal_args(desc, Q, K, V, eta, Z);
    p.W1_in = p.W1b_in = W1_0;
    p.W2_in = p.W2b_in = W2_0;
    p.w_in_bstride = desc->w_batch_stride;
    p.W1_out = W1_final;
    p.W2_out = W2_final;
    p.gamma = gamma; p.beta = beta; p.eps = eps;
    const hipError_t e = ttt::launch_mlp_primal(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
  }
  ttt::MlpArgs a = make_mlp_args(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final);
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  const hipError_t e = ttt::launch_mlp(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int64_t ttt_mlp_bwd_workspace_bytes(const ttt_mlp_desc* d) {
  if (!d || d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->dh < 1 || d->b < 1) return -1;
  int64_t n = 1;
  const int64_t nb = (static_cast<int64_t>(d->T) + d->b - 1) / d->b;
  for (int64_t f : {static_cast<int64_t>(d->B), static_cast<int64_t>(d->H), nb, int64_t{2},
                    static_cast<int64_t>(d->d), static_cast<int64_t>(d->dh), int64_t{4}})
    if (!mul_ok(n, f)) return -1;
  return n;
}

namespace {

// Every host-side check of the TTT-MLP backward.
ttt_status validate_mlp_bwd(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V, const float* W1_0,
                            const float* W2_0, const float* eta, const float* dZ, const float* dW1f,
                            const float* dW2f, const void* ws, int64_t ws_bytes, const float* dQ, const float* dK,
                            const float* dV, const float* deta, const float* dW1, const float* dW2) {
  if (!d) return TTT_ERR_NULL;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->d < 1 || d->dh < 1 || d->b < 1) return TTT_ERR_SHAPE;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return TTT_ERR_DTYPE;
  if ((d->flags & ~static_cast<uint32_t>(TTT_FLAG_PRIMAL)) != 0 || d->reserved != 0) return TTT_ERR_FLAGS;
  const int64_t hs = static_cast<int64_t>(d->H) * d->d * d->dh;
  if (d->w_batch_stride != 0 && d->w_batch_stride != hs) return TTT_ERR_STRIDE;
  if (d->eta_stride_b < 0 || d->eta_stride_h < 0 || d->eta_stride_t < 0) return TTT_ERR_STRIDE;
  int64_t chains = 1, tok = 1, wel = 1;
  if (!mul_ok(chains, d->B) || !mul_ok(chains, d->H) || chains > INT_MAX) return TTT_ERR_SHAPE;
  tok = chains;
  if (!mul_ok(tok, d->T) || !mul_ok(tok, d->d)) return TTT_ERR_SHAPE;
  wel = chains;
  if (!mul_ok(wel, d->d) || !mul_ok(wel, d->dh)) return TTT_ERR_SHAPE;
  const int64_t need = ttt_mlp_bwd_workspace_bytes(d);
  if (need < 0) return TTT_ERR_SHAPE;
  // dZ and every gradient are fp32; the Q/K/V dtype is in_dtype
  if (d->out_dtype != TTT_F32 || !ttt::mlp_bwd_supported(d->d, d->dh, d->b)) return TTT_ERR_UNSUPPORTED;
  if (chains == 0) return TTT_OK;
  if (!W1_0 || !W2_0 || !dW1 || !dW2) return TTT_ERR_NULL;
  if (tok > 0 && (!Q || !K || !V || !eta || !dZ || !dQ || !dK || !dV || !deta)) return TTT_ERR_NULL;
  for (const float* p : {W1_0, W2_0, dW1, dW2}) if (!aligned(p, 16)) return TTT_ERR_ALIGN;
  for (const float* p : {dW1f, dW2f}) if (p && !aligned(p, 16)) return TTT_ERR_ALIGN;
  if (tok > 0) {
    for (const void* p : {Q, K, V}) if (!aligned(p, static_cast<int>(dtype_size(d->in_dtype)))) return TTT_ERR_ALIGN;
    for (const float* p : {dQ, dK}) if (!aligned(p, 16)) return TTT_ERR_ALIGN;
    for (const float* p : {dZ, dV, deta, eta}) if (!aligned(p, 4)) return TTT_ERR_ALIGN;
  }
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return TTT_ERR_WORKSPACE;
  const int64_t in_b = tok * dtype_size(d->in_dtype), f_b = tok * 4;
  const int64_t w0_b = (d->w_batch_stride == 0 ? hs : wel) * 4, w_b = wel * 4;
  const int64_t eta_b =
      tok > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range ins[] = {{Q, in_b}, {K, in_b}, {V, in_b}, {W1_0, w0_b}, {W2_0, w0_b}, {eta, eta_b},
                       {dZ, f_b}, {dW1f, dW1f ? w_b : 0}, {dW2f, dW2f ? w_b : 0}};
  const Range outs[] = {{dQ, f_b}, {dK, f_b}, {dV, f_b}, {deta, chains * d->T * 4}, {dW1, w_b}, {dW2, w_b},
                        {ws, need}};
  for (int i = 0; i < 7; ++i) {
    for (const Range& in : ins)
      if (overlaps(outs[i], in)) return TTT_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
  }
  return TTT_OK;
}

// The matrix-core (dual-form) backward takes the shape it supports with
// 16-byte aligned token and gradient tensors; everything else, and
// TTT_FLAG_PRIMAL, runs the primal kernel.
bool mlp_bwd_dual_shape(const ttt_mlp_desc* d) {
  return !(d->flags & TTT_FLAG_PRIMAL) && ttt::mlp_bwd_mfma_supported(d->d, d->dh, d->b, d->in_dtype, d->T);
}

}  // namespace

ttt_status ttt_mlp_bwd_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                const float* W1_0, const float* W2_0, const float* eta, const float* dZ,
                                const float* dW1_final, const float* dW2_final, const void* workspace,
                                int64_t workspace_bytes, const float* dQ, const float* dK, const float* dV,
                                const float* deta, const float* dW1_0, const float* dW2_0) {
  return validate_mlp_bwd(desc, Q, K, V, W1_0, W2_0, eta, dZ, dW1_final, dW2_final, workspace, workspace_bytes, dQ,
                          dK, dV, deta, dW1_0, dW2_0);
}

ttt_status ttt_mlp_bwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* W1_0,
                       const float* W2_0, const float* eta, const float* dZ, const float* dW1_final,
                       const float* dW2_final, void* workspace, int64_t workspace_bytes, float* dQ, float* dK,
                       float* dV, float* deta, float* dW1_0, float* dW2_0, void* stream) {
  const ttt_status st = validate_mlp_bwd(desc, Q, K, V, W1_0, W2_0, eta, dZ, dW1_final, dW2_final, workspace,
                                         workspace_bytes, dQ, dK, dV, deta, dW1_0, dW2_0);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  ttt::MlpBwdArgs a;
  a.B = desc->B; a.H = desc->H; a.T = desc->T; a.d = desc->d; a.dh = desc->dh; a.b = desc->b;
  a.in_dtype = desc->in_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.W1_in = W1_0; a.W2_in = W2_0; a.w_in_bstride = desc->w_batch_stride;
  a.eta = eta; a.esb = desc->eta_stride_b; a.esh = desc->eta_stride_h; a.est = desc->eta_stride_t;
  a.dZ = dZ; a.dW1f = dW1_final; a.dW2f = dW2_final;
  a.ws = static_cast<float*>(workspace);
  a.dQ = dQ; a.dK = dK; a.dV = dV; a.deta = deta; a.dW1 = dW1_0; a.dW2 = dW2_0;
  a.gamma = nullptr; a.beta = nullptr; a.eps = 0.f; a.dgamma = nullptr; a.dbeta = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  bool dual = mlp_bwd_dual_shape(desc);
  if (desc->T > 0)
    for (const void* p : {Q, K, V, static_cast<const void*>(dZ), static_cast<const void*>(dQ),
                          static_cast<const void*>(dK), static_cast<const void*>(dV)})
      dual = dual && aligned(p, 16);
  if (!dual) {
    const hipError_t e = ttt::launch_mlp_bwd(a, s);
    return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
  }
  if (desc->T > 0) {
    // pass 1: the forward kernel writes the state at every mini-batch start
    ttt::MlpArgs f = make_mlp_args(desc, Q, K, V, W1_0, W2_0, eta, nullptr, nullptr, nullptr);
    f.ckpt = a.ws;
    const hipError_t e1 = ttt::launch_mlp_ckpt(f, s);
    if (e1 != hipSuccess) return TTT_ERR_HIP;
  }
  const hipError_t e = ttt::launch_mlp_bwd_mfma(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

const char* ttt_mlp_bwd_kernel_name(const ttt_mlp_desc* d) {
  if (!d) return nullptr;
  if (!ttt::mlp_bwd_supported(d->d, d->dh, d->b) || d->out_dtype != TTT_F32) return nullptr;
  return mlp_bwd_dual_shape(d) ? "ttt_mlp_bwd_d64h256b16" : "ttt_mlp_bwd_d64h256";
}

}  // extern "C"

namespace {

// ttt_mlp_bwd's checks, then the layer-norm parameters and their gradients:
// gamma, beta [H, d] and dgamma, dbeta [B, H, d] fp32, 4-byte aligned, the
// latter two outputs overlapping no input and no other output.
ttt_status validate_mlp_ln_bwd(const ttt_mlp_desc* d, const void* Q, const void* K, const void* V, const float* W1_0,
                               const float* W2_0, const float* gamma, const float* beta, float eps, const float* eta,
                               const float* dZ, const float* dW1f, const float* dW2f, const void* ws,
                               int64_t ws_bytes, const float* dQ, const float* dK, const float* dV, const float* deta,
                               const float* dW1, const float* dW2, const float* dgamma, const float* dbeta) {
  const ttt_status st = validate_mlp_bwd(d, Q, K, V, W1_0, W2_0, eta, dZ, dW1f, dW2f, ws, ws_bytes, dQ, dK, dV, deta,
                                         dW1, dW2);
  if (st != TTT_OK) return st;
  const int64_t chains = static_cast<int64_t>(d->B) * d->H;
  const int64_t tok = chains * d->T * d->d * 4, w_b = chains * d->d * d->dh * 4, cd_b = chains * d->d * 4;
  const int64_t need = ttt_mlp_bwd_workspace_bytes(d);
  const std::initializer_list<Range> all_outs = {{dQ, tok}, {dK, tok}, {dV, tok}, {deta, chains * d->T * 4},
                                                 {dW1, w_b}, {dW2, w_b}, {ws, need}, {dgamma, cd_b}, {dbeta, cd_b}};
  const ttt_status sl = check_ln(chains, d->H, d->d, gamma, beta, eps, all_outs);
  if (sl != TTT_OK) return sl;
  if (chains == 0) return TTT_OK;
  if (!dgamma || !dbeta) return TTT_ERR_NULL;
  if (!aligned(dgamma, 4) || !aligned(dbeta, 4)) return TTT_ERR_ALIGN;
  const int64_t in_b = tok / 4 * dtype_size(d->in_dtype);
  const int64_t w0_b = (d->w_batch_stride == 0 ? static_cast<int64_t>(d->H) * d->d * d->dh * 4 : w_b);
  const int64_t eta_b =
      d->T > 0 ? eta_extent(d->B, d->H, d->T, d->eta_stride_b, d->eta_stride_h, d->eta_stride_t) * 4 : 0;
  const Range ins[] = {{Q, in_b}, {K, in_b}, {V, in_b}, {W1_0, w0_b}, {W2_0, w0_b}, {eta, eta_b}, {dZ, tok},
                       {dW1f, dW1f ? w_b : 0}, {dW2f, dW2f ? w_b : 0}};
  // dgamma and dbeta are the last two outputs: each against every input and
  // every output before it (ttt_mlp_bwd's checks covered the others)
  const Range* outs = all_outs.begin();
  const int n_out = static_cast<int>(all_outs.size());
  for (int i = n_out - 2; i < n_out; ++i) {
    for (const Range& in : ins)
      if (overlaps(outs[i], in)) return TTT_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
  }
  return TTT_OK;
}

}  // namespace

extern "C" {

ttt_status ttt_mlp_ln_bwd_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                   const float* W1_0, const float* W2_0, const float* gamma, const float* beta,
                                   float eps, const float* eta, const float* dZ, const float* dW1_final,
                                   const float* dW2_final, const void* workspace, int64_t workspace_bytes,
                                   const float* dQ, const float* dK, const float* dV, const float* deta,
                                   const float* dW1_0, const float* dW2_0, const float* dgamma, const float* dbeta) {
  return validate_mlp_ln_bwd(desc, Q, K, V, W1_0, W2_0, gamma, beta, eps, eta, dZ, dW1_final, dW2_final, workspace,
                             workspace_bytes, dQ, dK, dV, deta, dW1_0, dW2_0, dgamma, dbeta);
}

ttt_status ttt_mlp_ln_bwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* W1_0,
                          const float* W2_0, const float* gamma, const float* beta, float eps, const float* eta,
                          const float* dZ, const float* dW1_final, const float* dW2_final, void* workspace,
                          int64_t workspace_bytes, float* dQ, float* dK, float* dV, float* deta, float* dW1_0,
                          float* dW2_0, float* dgamma, float* dbeta, void* stream) {
  const ttt_status st = validate_mlp_ln_bwd(desc, Q, K, V, W1_0, W2_0, gamma, beta, eps, eta, dZ, dW1_final,
                                            dW2_final, workspace, workspace_bytes, dQ, dK, dV, deta, dW1_0, dW2_0,
                                            dgamma, dbeta);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  ttt::MlpBwdArgs a;
  a.B = desc->B; a.H = desc->H; a.T = desc->T; a.d = desc->d; a.dh = desc->dh; a.b = desc->b;
  a.in_dtype = desc->in_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.W1_in = W1_0; a.W2_in = W2_0; a.w_in_bstride = desc->w_batch_stride;
  a.eta = eta; a.esb = desc->eta_stride_b; a.esh = desc->eta_stride_h; a.est = desc->eta_stride_t;
  a.dZ = dZ; a.dW1f = dW1_final; a.dW2f = dW2_final;
  a.ws = static_cast<float*>(workspace);
  a.dQ = dQ; a.dK = dK; a.dV = dV; a.deta = deta; a.dW1 = dW1_0; a.dW2 = dW2_0;
  a.gamma = gamma; a.beta = beta; a.eps = eps; a.dgamma = dgamma; a.dbeta = dbeta;
  const hipError_t e = ttt::launch_mlp_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

const char* ttt_mlp_ln_bwd_kernel_name(const ttt_mlp_desc* d) {
  if (!d) return nullptr;
  if (!ttt::mlp_bwd_supported(d->d, d->dh, d->b) || d->out_dtype != TTT_F32) return nullptr;
  return "ttt_mlp_bwd_d64h256 (layer norm)";
}

}  // extern "C"
