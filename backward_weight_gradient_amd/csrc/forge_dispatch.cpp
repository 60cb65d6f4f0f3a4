// Runtime dispatch of a call to the kernels of its (optimizer, state
// formats) combination.  Sees only declarations: the kernels are
// instantiated in the family sources.
#include "forge_internal.h"

namespace forge {

hipError_t launch_fused(const KArgs& a, int in_fmt, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return combo_fused<O, M, V>(a, in_fmt, w_fmt, st);
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_fused_group(const GroupArgs& g, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return combo_group<O, M, V>(g, w_fmt, st);
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_fused_acc(const KArgs& a, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return combo_fused_acc<O, M, V>(a, w_fmt, st);
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_fused_fp8w(const KArgs& a, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return combo_fused_fp8w<O, M, V>(a, st);
  FORGE_FP8W_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_step(const KArgs& a, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return combo_step<O, M, V>(a, w_fmt, st);
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace forge
