// C ABI of libttt.so: argument validation and kernel dispatch.
// The entry points and their contracts are documented in include/ttt.h.
#include <limits.h>
#include <stdint.h>

#include "../../include/ttt.h"
#include "ttt_internal.h"

namespace {

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

enum Kernel { K_NONE, K_GENERIC, K_MFMA, K_PRIMAL };

constexpr uint32_t kRowFlags = TTT_FLAG_ROWS1 | TTT_FLAG_ROWS2 | TTT_FLAG_ROWS4;

Kernel pick_linear(const ttt::LinearArgs& a, uint32_t flags) {
  if (flags & TTT_FLAG_PRIMAL) return ttt::linear_primal_supported(a.d) ? K_PRIMAL : K_NONE;
  if (flags & TTT_FLAG_GENERIC) return ttt::linear_generic_supported(a.d, a.b) ? K_GENERIC : K_NONE;
  if (ttt::linear_mfma_supported(a)) return K_MFMA;
  if (flags & kRowFlags) return K_NONE;  // row blocks exist only in the matrix-core kernel
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
  a.nchunk = 1; a.Tc = d->T; a.Wstart = nullptr; a.maps = nullptr;
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
  if (d->flags != 0 || d->reserved != 0) return TTT_ERR_FLAGS;
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
  if (!ttt::mlp_supported(a)) return TTT_ERR_UNSUPPORTED;
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
  else if (k == K_PRIMAL)
    e = ttt::launch_linear_primal(make_primal_args_fwd(desc, Q, K, V, W0, eta, Z, W_final), s);
  else
    e = ttt::launch_linear_generic(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_linear_fwd_save(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                               const float* W0, const float* eta, void* Z, float* W_final, float* E_saved,
                               void* stream) {
  Kernel k;
  const ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (desc->flags & TTT_FLAG_PRIMAL) return TTT_ERR_FLAGS;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  const int64_t tok = chains * desc->T * desc->d;
  if (tok > 0) {
    if (!E_saved) return TTT_ERR_NULL;
    if (!aligned(E_saved, 16)) return TTT_ERR_ALIGN;
    const int64_t in_b = tok * dtype_size(desc->in_dtype), z_b = tok * dtype_size(desc->out_dtype);
    const int64_t hdd = static_cast<int64_t>(desc->H) * desc->d * desc->d;
    const int64_t w0_b = (desc->w0_batch_stride == 0 ? hdd : chains * desc->d * desc->d) * 4;
    const int64_t eta_b =
        eta_extent(desc->B, desc->H, desc->T, desc->eta_stride_b, desc->eta_stride_h, desc->eta_stride_t) * 4;
    const Range re{E_saved, tok * 4};
    for (Range r : {Range{Q, in_b}, Range{K, in_b}, Range{V, in_b}, Range{eta, eta_b}, Range{W0, w0_b},
                    Range{Z, z_b}, Range{W_final, chains * desc->d * desc->d * 4}})
      if (overlaps(re, r)) return TTT_ERR_ALIAS;
  }
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

ttt_status ttt_linear_ln_fwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* W0, const float* gamma, const float* beta, float eps, const float* eta,
                             void* Z, float* W_final, void* stream) {
  Kernel k;
  const ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (desc->flags != 0 || k != K_MFMA) return TTT_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps > 1e30f) return TTT_ERR_SHAPE;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  if (!gamma || !beta) return TTT_ERR_NULL;
  if (!aligned(gamma, 4) || !aligned(beta, 4)) return TTT_ERR_ALIGN;
  const int64_t hd_b = static_cast<int64_t>(desc->H) * desc->d * 4;
  const int64_t z_b = chains * desc->T * desc->d * dtype_size(desc->out_dtype);
  for (Range out : {Range{Z, z_b}, Range{W_final, chains * desc->d * desc->d * 4}})
    for (Range in : {Range{gamma, hd_b}, Range{beta, hd_b}})
      if (overlaps(out, in)) return TTT_ERR_ALIAS;
  ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.rb = 1;
  const hipError_t e = ttt::launch_linear_mfma(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

int64_t ttt_linear_chunked_workspace_bytes(const ttt_linear_desc* desc, int32_t nchunks) {
  if (!desc || nchunks < 1 || desc->B < 0 || desc->H < 0 || desc->d < 1) return -1;
  if (nchunks == 1) return 0;
  const int64_t per_chain = (static_cast<int64_t>(nchunks - 1) * 2 + nchunks) * desc->d * desc->d * 4;
  return static_cast<int64_t>(desc->B) * desc->H * per_chain;
}

ttt_status ttt_linear_fwd_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K,
                                  const void* V, const float* W0, const float* eta, void* Z, float* W_final,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  Kernel k;
  ttt_status st = validate_linear(desc, Q, K, V, W0, eta, Z, W_final, &k);
  if (st != TTT_OK) return st;
  if (nchunks < 1 || desc->T % (16 * nchunks) != 0) return TTT_ERR_SHAPE;
  if ((desc->flags & ~kRowFlags) != 0 || k != K_MFMA) return TTT_ERR_UNSUPPORTED;
  // workgroups of the map launch (2 maps per chunk but the last) and of the chunk forward
  if (static_cast<int64_t>(desc->B) * desc->H * 2 * nchunks * row_blocks(desc->flags) > INT_MAX)
    return TTT_ERR_SHAPE;
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
  ttt::LinearArgs a = make_linear_args(desc, Q, K, V, W0, eta, Z, W_final);
  a.nchunk = nchunks;
  a.Tc = desc->T / nchunks;
  a.maps = static_cast<float*>(workspace);
  a.Wstart = a.maps + chains * (nchunks - 1) * 2 * desc->d * desc->d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = ttt::launch_linear_mfma_maps(a, s);
  if (e == hipSuccess) e = ttt::launch_linear_chunk_scan(a, s);
  if (e == hipSuccess) e = ttt::launch_linear_mfma(a, s);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

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
  ttt::PrimalArgs a;
  a.B = desc->B; a.H = desc->H; a.T = desc->T; a.d = desc->d; a.b = desc->b;
  a.in_dtype = desc->in_dtype; a.out_dtype = desc->out_dtype;
  a.Q = Q; a.K = K; a.V = V;
  a.W_in = W; a.Wb_in = Wb; a.w_in_bstride = static_cast<int64_t>(desc->H) * desc->d * desc->d;
  a.eta = eta; a.esb = desc->eta_stride_b; a.esh = desc->eta_stride_h; a.est = desc->eta_stride_t;
  a.Z = Z; a.W_out = W; a.Wb_out = Wb; a.pos = pos;
  const hipError_t e = ttt::launch_linear_primal(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                            const float* W1_0, const float* W2_0, const float* eta, const void* Z,
                            const float* W1_final, const float* W2_final) {
  return validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, nullptr);
}

const char* ttt_mlp_kernel_name(const ttt_mlp_desc* d) {
  if (!d) return nullptr;
  ttt::MlpArgs a = make_mlp_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr);
  return ttt::mlp_supported(a) ? ttt::mlp_name(a) : nullptr;
}

ttt_status ttt_mlp_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* W1_0,
                       const float* W2_0, const float* eta, void* Z, float* W1_final, float* W2_final,
                       void* stream) {
  bool ok;
  const ttt_status st = validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, &ok);
  if (st != TTT_OK) return st;
  if (static_cast<int64_t>(desc->B) * desc->H == 0) return TTT_OK;
  const ttt::MlpArgs a = make_mlp_args(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final);
  const hipError_t e = ttt::launch_mlp(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

ttt_status ttt_mlp_ln_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W1_0, const float* W2_0, const float* gamma, const float* beta, float eps,
                          const float* eta, void* Z, float* W1_final, float* W2_final, void* stream) {
  bool ok;
  const ttt_status st = validate_mlp(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final, &ok);
  if (st != TTT_OK) return st;
  if (!(eps >= 0.f) || eps > 1e30f) return TTT_ERR_SHAPE;
  const int64_t chains = static_cast<int64_t>(desc->B) * desc->H;
  if (chains == 0) return TTT_OK;
  if (!gamma || !beta) return TTT_ERR_NULL;
  if (!aligned(gamma, 4) || !aligned(beta, 4)) return TTT_ERR_ALIGN;
  const int64_t hd_b = static_cast<int64_t>(desc->H) * desc->d * 4;
  const int64_t z_b = chains * desc->T * desc->d * dtype_size(desc->out_dtype);
  const int64_t w_b = chains * desc->d * desc->dh * 4;
  for (Range out : {Range{Z, z_b}, Range{W1_final, w_b}, Range{W2_final, w_b}})
    for (Range in : {Range{gamma, hd_b}, Range{beta, hd_b}})
      if (overlaps(out, in)) return TTT_ERR_ALIAS;
  ttt::MlpArgs a = make_mlp_args(desc, Q, K, V, W1_0, W2_0, eta, Z, W1_final, W2_final);
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  const hipError_t e = ttt::launch_mlp(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

}  // extern "C"
