// Internal interface between the host API (forge_api.cpp) and the gfx950
// kernels (forge_device.h, forge_k_*.hip, forge_dispatch.cpp).  Not part of
// the public ABI.
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

namespace forge {

enum Fmt : int { FMT_NONE = -1, FMT_F32 = 0, FMT_BF16 = 1, FMT_S8 = 2, FMT_U8 = 3, FMT_E4M3 = 4 };

// Formats stored as 8-bit codes with one fp32 scale per block of a row.
constexpr bool fmt_blocked(int f) { return f == FMT_S8 || f == FMT_U8 || f == FMT_E4M3; }
enum Opt : int {
  OPT_ADAMW = 0, OPT_LION = 1, OPT_SGDM = 2, OPT_NADAM = 3, OPT_RADAM = 4, OPT_RMSPROP = 5, OPT_ADAGRAD = 6,
  OPT_SGD = 7
};

// Which states an optimizer keeps: m (first moment / momentum) and v
// (second moment / squared-gradient sum).
constexpr bool opt_has_m(int o) {
  return o == OPT_ADAMW || o == OPT_LION || o == OPT_SGDM || o == OPT_NADAM || o == OPT_RADAM;
}
constexpr bool opt_has_v(int o) {
  return o == OPT_ADAMW || o == OPT_NADAM || o == OPT_RADAM || o == OPT_RMSPROP || o == OPT_ADAGRAD;
}

// Scalars of the element-wise step, computed once per call on the host in
// double precision and rounded once to fp32.
struct EpiConst {
  float lr;        // eta
  float b1, b2;    // beta1 (SGD-m: momentum), beta2
  float omb1;      // 1 - beta1
  float omb2;      // 1 - beta2
  float eps;
  float decay;     // 1 - eta * lambda   (decoupled decay: AdamW, Lion)
  float wd;        // lambda             (L2 decay: SGD-m)
  float bc1;       // 1 / (1 - beta1^t)
  float lrbc1;     // eta / (1 - beta1^t)   (AdamW)
  float bc2s;      // 1 / sqrt(1 - beta2^t)
  float na1;       // NAdam: mu_{t+1} / (1 - prod_{i<=t+1} mu_i)   (weight of m')
  float na2;       // NAdam: (1 - mu_t) / (1 - prod_{i<=t} mu_i)   (weight of G)
  float rc;        // RAdam, rectified: r_t sqrt(1 - beta2^t) / (1 - beta1^t)
  int32_t rect;    // RAdam: 1 once rho_t > 5 (adaptive step), else 0 (momentum step)
  uint32_t keyW, keyM, keyV;  // stochastic-rounding keys of the three tensors
  uint32_t sr;     // all ones: stochastic rounding of bf16 (and E4M3 weight) stores, 0: round to nearest even
};

// Everything a launch needs.  Pointers are device pointers; leading
// dimensions are in elements.
struct KArgs {
  const void* X;  int64_t ldx;    // [BT, K]
  const void* dY; int64_t lddy;   // [BT, N]
  void* W;  int64_t ldw;          // [N, K]
  float* wsc;                     // block scales of an E4M3 weight [N, K/block] (else null)
  void* m;  int64_t ldm; float* ms;   // state 1 (+ int8 scales [N, K/block])
  void* v;  int64_t ldv; float* vs;   // state 2 (+ int8 scales)
  void* dW; int64_t lddw;         // G buffer [N, K]: unfused workspace (ld = K) or fp32 accumulator
  int32_t dw_fmt;                 // FMT_F32 / FMT_BF16 for dW
  int32_t vec_dw;                 // dW rows allow 16-byte vector access
  int32_t dw_add;                 // k_gemm: dW += G instead of dW = G (fp32 accumulation)
  int32_t BT, N, K;
  int32_t tiles_n, tiles_k;       // ceil(N/128), ceil(K/128)
  int32_t block;                  // int8 block length (32, 64, 128)
  int32_t vec_in;                 // X / dY rows allow 16-byte vector loads
  int32_t vec_state;              // W / m / v rows allow 8-element vector access
  int32_t dma_ok;                 // bf16 X / dY qualify for the direct-to-LDS mainloop
  EpiConst c;
};

// Up to GROUP_MAX independent layers launched together (same formats and
// optimizer).  first_tile[i] is the first workgroup of layer i;
// first_tile[n] is the grid size.
constexpr int GROUP_MAX = 8;
struct GroupArgs {
  KArgs layer[GROUP_MAX];
  int32_t first_tile[GROUP_MAX + 1];
  int32_t n;
};

constexpr int WIDE_MIN_BT = 2048;  // token count from which the 256 x 256 kernel is used (measured: faster from 2048 on)

// Supported (optimizer, m format, v format) combinations, by family; each
// family's kernels are instantiated in its own source file.
#define FORGE_ADAMW_LIST(X)        \
  X(OPT_ADAMW, FMT_F32, FMT_F32)   \
  X(OPT_ADAMW, FMT_BF16, FMT_BF16) \
  X(OPT_ADAMW, FMT_S8, FMT_U8)     \
  X(OPT_ADAMW, FMT_E4M3, FMT_E4M3)
#define FORGE_LION_LIST(X)         \
  X(OPT_LION, FMT_F32, FMT_NONE)   \
  X(OPT_LION, FMT_BF16, FMT_NONE)  \
  X(OPT_LION, FMT_S8, FMT_NONE)    \
  X(OPT_LION, FMT_E4M3, FMT_NONE)
#define FORGE_SGDM_LIST(X)         \
  X(OPT_SGDM, FMT_F32, FMT_NONE)   \
  X(OPT_SGDM, FMT_BF16, FMT_NONE)  \
  X(OPT_SGDM, FMT_S8, FMT_NONE)    \
  X(OPT_SGDM, FMT_E4M3, FMT_NONE)
#define FORGE_ADAM_VARIANT_LIST(X)  \
  X(OPT_NADAM, FMT_F32, FMT_F32)    \
  X(OPT_NADAM, FMT_BF16, FMT_BF16)  \
  X(OPT_RADAM, FMT_F32, FMT_F32)    \
  X(OPT_RADAM, FMT_BF16, FMT_BF16)
#define FORGE_SECOND_MOMENT_LIST(X)    \
  X(OPT_RMSPROP, FMT_NONE, FMT_F32)    \
  X(OPT_RMSPROP, FMT_NONE, FMT_BF16)   \
  X(OPT_ADAGRAD, FMT_NONE, FMT_F32)    \
  X(OPT_ADAGRAD, FMT_NONE, FMT_BF16)   \
  X(OPT_SGD, FMT_NONE, FMT_NONE)
// Combinations that also take an E4M3 weight with block scales (bf16 inputs):
// AdamW, Lion and SGD-momentum with every state format they support.
#define FORGE_FP8W_LIST(X)         \
  X(OPT_ADAMW, FMT_F32, FMT_F32)   \
  X(OPT_ADAMW, FMT_BF16, FMT_BF16) \
  X(OPT_ADAMW, FMT_S8, FMT_U8)     \
  X(OPT_ADAMW, FMT_E4M3, FMT_E4M3) \
  X(OPT_LION, FMT_F32, FMT_NONE)   \
  X(OPT_LION, FMT_BF16, FMT_NONE)  \
  X(OPT_LION, FMT_E4M3, FMT_NONE)  \
  X(OPT_SGDM, FMT_F32, FMT_NONE)   \
  X(OPT_SGDM, FMT_BF16, FMT_NONE)  \
  X(OPT_SGDM, FMT_E4M3, FMT_NONE)
#define FORGE_STATE_LIST(X) \
  FORGE_ADAMW_LIST(X) FORGE_LION_LIST(X) FORGE_SGDM_LIST(X) FORGE_ADAM_VARIANT_LIST(X) FORGE_SECOND_MOMENT_LIST(X)

// The input-gradient GEMM dX = dY W (dY [BT, N], W [N, K], dX [BT, K]).
struct DgArgs {
  const void* dY; int64_t lddy;
  const void* W; int64_t ldw;
  void* dX; int64_t ldx;
  int32_t BT, N, K;
  int32_t tiles_m, tiles_k;       // ceil(BT/128), ceil(K/128) (MFMA kernel)
  int32_t in_fmt, w_fmt, dx_fmt;  // dtypes of dY, W, dX (W may be E4M3 with block scales wsc)
  const float* wsc;               // E4M3 W: fp32 scales [N, K / wblock]
  int32_t wblock;
  int32_t vec_out;                // dX rows allow 4-element vector stores
  int32_t splits;                 // > 1: the reduction split across workgroups (fast path only)
  float* ws;                      // splits x [BT, K] fp32 partials (splits > 1)
};
// forge_k_dgrad.hip: fast = bf16 dY and W with 16-byte aligned rows, N and K multiples of 8.
hipError_t launch_dgrad(const DgArgs& g, bool fast, hipStream_t stream);
// dX from an E4M3 weight (g.wsc, g.wblock), bf16 dY: the bf16 matrix-core kernel when fast (aligned rows,
// N % 8 == 0, K % 16 == 0, 32-bit buffer offsets), else the fp32 matrix-core kernel; other dY: the plain one.
hipError_t launch_dgrad_fp8w(const DgArgs& g, bool fast, hipStream_t stream);
// The split path with the partials in the library's own per-device scratch
// array (no caller workspace, no allocation); g.splits * BT * K * 4 must not
// exceed DGRAD_SCRATCH_BYTES.
constexpr int64_t DGRAD_SCRATCH_BYTES = 64ll << 20;
hipError_t launch_dgrad_scratch(DgArgs g, bool fast, hipStream_t stream);

// Plan of the split dX for dY [BT, N], W [N, K].
//  wide (k_dgrad_wide, 256 x 256 tiles, one workgroup per CU): for a long
//    reduction (at least 64 chunks of 32), BT >= 256 and fewer 128-token
//    tiles than two per CU (the 128-token kernel cannot fill the chip
//    twice; larger shapes keep it, unsplit), the split count
//    s <= 8 (each split at least 32 chunks) that minimises
//    ceil(tiles s / 256) ceil(chunks / s) -- rounds of workgroups times
//    chunks per split -- the smallest such s, taken when s > 1 and
//    tiles x s gives at least 3/4 of the CUs a workgroup (measured at
//    BT 512: q / o_proj, 16-chunk splits on 256 workgroups, are slower than
//    the 128-token kernel, because each split's fp32 partial tile is
//    written and read back);
//  else 128-token tiles (k_dgrad_bf16<128>): 1 (no split) when those, or the
//    unsplit kernel's 64-token tiles, already give every CU a workgroup
//    (measured at BT 512: q / o_proj unsplit on 64-token tiles 34 us, in 4
//    splits 39 us), else up to 4, so that tiles x splits fill the chip twice
//    (two workgroups per CU), each split covering at least 32 chunks
//    (measured: 8-chunk splits of k / v_proj at BT 512 run 50% slower than
//    the unsplit 64-token kernel).
struct DgPlan {
  bool wide;
  int splits;
};
inline DgPlan dgrad_plan(int64_t BT, int64_t N, int64_t K) {
  const int64_t nk = (N + 31) / 32;
  const int64_t t128 = ((BT + 127) / 128) * ((K + 127) / 128);
  const int64_t t256 = ((BT + 255) / 256) * ((K + 255) / 256);
  if (BT >= 256 && nk >= 64 && t128 < 512 && t256 > 0) {
    int best = 1;
    int64_t best_cost = -1;
    for (int s = 1; s <= 8 && nk / s >= 32; ++s) {
      const int64_t cost = ((t256 * s + 255) / 256) * ((nk + s - 1) / s);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = s;
      }
    }
    if (best > 1 && t256 * best >= 192) return {true, best};
  }
  const int64_t t64 = ((BT + 63) / 64) * ((K + 127) / 128);
  if (t128 == 0 || t128 >= 256 || t64 >= 256) return {false, 1};
  int64_t s = (512 + t128 - 1) / t128;
  if (s > 4) s = 4;
  while (s > 1 && nk / s < 32) --s;
  return {false, (int)s};
}
inline int dgrad_splits(int64_t BT, int64_t N, int64_t K) { return dgrad_plan(BT, N, K).splits; }

inline bool combo_supported(int in_fmt, int w_fmt, int opt, int m_fmt, int v_fmt) {
  if (in_fmt != FMT_F32 && in_fmt != FMT_BF16) return false;
  if (w_fmt == FMT_E4M3) {
    if (in_fmt != FMT_BF16) return false;
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return true;
    FORGE_FP8W_LIST(X)
#undef X
    return false;
  }
  if (w_fmt != FMT_F32 && w_fmt != FMT_BF16) return false;
#define X(O, M, V) \
  if (opt == O && m_fmt == M && v_fmt == V) return true;
  FORGE_STATE_LIST(X)
#undef X
  return false;
}

// Whether a layer can run in the grouped kernel (aligned bf16, short token axis).
inline bool group_eligible(const KArgs& a, int in_fmt) {
  return in_fmt == FMT_BF16 && a.dma_ok && a.vec_state && (a.K % 4) == 0 && a.BT < WIDE_MIN_BT;
}

// Launchers of one combination (defined in forge_device.h, instantiated by
// the family sources).  combo_step reads G from a.dW in format a.dw_fmt.
template <int O, int M, int V>
hipError_t combo_fused(const KArgs& a, int in_fmt, int w_fmt, hipStream_t st);
template <int O, int M, int V>
hipError_t combo_group(const GroupArgs& g, int w_fmt, hipStream_t st);
template <int O, int M, int V>
hipError_t combo_step(const KArgs& a, int w_fmt, hipStream_t st);
// Fused step with G = a.dW (fp32 accumulator) + this call's G (aligned bf16 inputs only).
template <int O, int M, int V>
hipError_t combo_fused_acc(const KArgs& a, int w_fmt, hipStream_t st);

// Runtime dispatch over the combinations (forge_dispatch.cpp).
// Fused weight-gradient + step: one workgroup per 128 x 128 tile of W.
hipError_t launch_fused(const KArgs& a, int in_fmt, int w_fmt, int opt, int m_fmt, int v_fmt,
                        hipStream_t stream);
template <int O, int M, int V>
hipError_t combo_fused_fp8w(const KArgs& a, hipStream_t st);
// Fused step with an E4M3 weight (a.wsc its block scales; bf16 inputs).
hipError_t launch_fused_fp8w(const KArgs& a, int opt, int m_fmt, int v_fmt, hipStream_t stream);
// Fused step of g.n group-eligible layers in one launch (bf16 inputs).
hipError_t launch_fused_group(const GroupArgs& g, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t stream);
// Fused step from an fp32 accumulator plus this call's gradient.
hipError_t launch_fused_acc(const KArgs& a, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t stream);
// Unfused baseline, phase 1, and gradient accumulation (forge_k_common.hip):
// G tiles -> a.dW (a.dw_fmt), or a.dW += G when a.dw_add.
hipError_t launch_gemm(const KArgs& a, int in_fmt, hipStream_t stream);
// Unfused baseline, phase 2: the same step, reading G from a.dW.
hipError_t launch_step(const KArgs& a, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t stream);
// forge_k_common.hip:
// Stochastic rounding of n floats with one key, element i using flat index i.
hipError_t launch_debug_sr(const float* in, uint16_t* out, uint32_t n, uint32_t key,
                           hipStream_t stream);
// E4M3 rounding (nearest even, saturating) of n floats.
hipError_t launch_debug_e4m3(const float* in, uint8_t* out, uint32_t n, hipStream_t stream);
hipError_t launch_debug_e4m3_sr(const float* in, uint8_t* out, uint32_t n, uint32_t key, hipStream_t stream);
constexpr int QUOTIENT_CHECK_BLOCKS = 2048;   // forge_debug_quotients: workgroups, 8 counters each
hipError_t launch_debug_quotients(unsigned long long* counts, hipStream_t stream);
// The 8-bit block quantiser of the epilogue (S8 / U8 / E4M3 codes and fp32
// scales) on a dense [rows, cols] fp32 array; positive: the second-moment rule.
hipError_t launch_debug_quant(const float* in, uint8_t* codes, float* scales, int rows, int cols, int fmt,
                              bool positive, int block, hipStream_t stream);
hipError_t launch_debug_copy(const void* src, void* dst, uint64_t bytes, hipStream_t stream);
hipError_t launch_debug_state_stream(uint16_t* W, float* m, float* v, int N, int K, hipStream_t stream);
hipError_t launch_debug_mfma(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace forge
