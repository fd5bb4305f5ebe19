// TTT-MLP dual-form forward (d = 64, dh = 256, b = 16, bf16 Q/K/V).
#include "ttt_internal.h"

namespace ttt {

bool mlp_supported(const MlpArgs& a) {
  (void)a;
  return false;
}

const char* mlp_name(const MlpArgs& a) {
  (void)a;
  return "ttt_mlp_fwd_d64h256b16";
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorInvalidValue;
}

}  // namespace ttt
