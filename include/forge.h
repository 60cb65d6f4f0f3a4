/*
 * forge.h -- C ABI of libforge: the weight gradient of a linear layer fused
 * with an element-wise optimizer step, for AMD MI355X (gfx950).
 *
 * What it computes (FORGE paper, arXiv 2606.22932 -- "the paper" below):
 *   for a linear layer Y = X W^T (section 2.1, Eq. 2) with
 *     X  [BT, K]  saved input activations (K = D_in),
 *     dY [BT, N]  upstream gradient dL/dY  (N = D_out),
 *     W  [N, K]   weight, nn.Linear layout,
 *   the weight gradient G = dY^T X, G[p,q] = sum_t dY[t,p] X[t,q]
 *   (section 2.1, Eq. 3; Appendix A, "Setup"), reduced over the token axis
 *   BT in fp32, one 128 x 128 tile of G at a time (section 2.2, Eq. 5), and
 *   an element-wise optimizer step (Appendix A, Definition 1) applied to each
 *   tile in registers as soon as it is complete (Algorithm 1, Phase 2).
 *   Only W and the optimizer state are written back (Algorithm 1, Phase 3);
 *   G itself never reaches device memory.
 *
 * Conventions shared by every entry point
 *   - All matrix data pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or retains them (forge_wgrad_unfused,
 *     forge_dgrad_split and forge_backward_step_split write into a
 *     caller-provided workspace).
 *   - Matrices are row-major; `ld` is the leading dimension in elements
 *     (ld >= cols); a matrix spans ((rows - 1) * ld + cols) elements, whose
 *     bytes must not exceed 2^48 (else FORGE_E_SHAPE).  Flat indices used by
 *     stochastic rounding are the logical row-major index p*K + q,
 *     independent of ld.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and return after the kernels are enqueued.  W, m, v and the
 *     block scales (int8 / E4M3 states) are updated in place.
 *   - Argument validation is synchronous and host-only.  On any error code
 *     other than FORGE_E_HIP nothing has been enqueued and nothing modified.
 *   - No exception crosses the ABI.  The library keeps no mutable global
 *     state apart from forge_dgrad_split_noalloc's per-device scratch array;
 *     calls on distinct streams may run concurrently on disjoint buffers.
 *   - Precondition the library cannot check (paper, Appendix A, Remark 1):
 *     the caller has already computed the input gradient dX = dY W from the
 *     pre-update W; a weight whose gradient comes from several consumers in
 *     one step (tied embeddings, expert-parallel experts) must not be stepped
 *     here.
 *   - Precondition of the fused schedule: no global gradient-norm clip, and
 *     forge_wgrad_step sees the whole gradient of the step; to accumulate
 *     micro-batches use forge_wgrad_accumulate and
 *     forge_wgrad_step_accumulated (paper, Appendix L).
 */
#ifndef FORGE_H
#define FORGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FORGE_OK = 0,
  FORGE_E_NULL = 1,        /* a required pointer (struct or data) is NULL           */
  FORGE_E_SHAPE = 2,       /* shapes disagree, ld < cols, or a size limit is exceeded */
  FORGE_E_DTYPE = 3,       /* a dtype is not allowed in that position               */
  FORGE_E_ALIGN = 4,       /* a data pointer is not aligned to its element size     */
  FORGE_E_STEP = 5,        /* step < 1                                              */
  FORGE_E_HYPER = 6,       /* a hyper-parameter is non-finite or out of range       */
  FORGE_E_ALIAS = 7,       /* an output buffer overlaps an input or another output  */
  FORGE_E_UNSUPPORTED = 8, /* a valid combination the library does not implement  */
  FORGE_E_HIP = 9,         /* the HIP runtime reported an error at launch           */
  FORGE_E_SCRATCH = 10     /* forge_dgrad_split_noalloc: the call needs more than
                              FORGE_DGRAD_SCRATCH_BYTES of scratch                   */
} forge_status;

typedef enum { FORGE_F32 = 0, FORGE_BF16 = 1, FORGE_S8 = 2, FORGE_U8 = 3, FORGE_E4M3 = 4 } forge_dtype;

/* Optimizers: the eight element-wise families the paper fuses in full
 * (Appendix N, "Fully fused").  Where the pages name a family without its
 * formula, the library follows the textbook rule as PyTorch implements it
 * (the pages verify every family against a PyTorch reference, Appendix N,
 * "Numerical verification"); "decoupled" decay is W <- (1 - lr wd) W before
 * the update, "coupled" (L2) decay adds wd W to the gradient. */
typedef enum {
  FORGE_ADAMW = 0,   /* Algorithm 1 Phase 2: bias correction, decoupled decay; m and v      */
  FORGE_LION = 1,    /* sign of the interpolated momentum (Chen et al. 2023); m only        */
  FORGE_SGDM = 2,    /* SGD with momentum: coupled decay, dampening 0, no Nesterov,
                        momentum = beta1; m (the momentum buffer) only                      */
  FORGE_NADAM = 3,   /* AdamW with the Nesterov-corrected first moment (Dozat 2016; momentum
                        schedule mu_t = beta1 (1 - 0.5 * 0.96^(0.004 t))), decoupled decay;
                        m and v                                                             */
  FORGE_RADAM = 4,   /* AdamW with the rectified variance term (Liu et al. 2019: the adaptive
                        step only once rho_t > 5), decoupled decay; m and v                 */
  FORGE_RMSPROP = 5, /* second moment only: v <- a v + (1 - a) g^2 with a = beta2, coupled
                        decay, no momentum, not centred; v only (m NULL)                    */
  FORGE_ADAGRAD = 6, /* cumulative squared gradient v <- v + g^2 (no decay of v, learning-
                        rate decay 0), coupled decay; v only (m NULL)                       */
  FORGE_SGD = 7      /* vanilla gradient descent with coupled decay; no state (m, v NULL)   */
} forge_optim;

/* Rounding of every bf16 store (paper, Appendix C). */
typedef enum {
  FORGE_ROUND_RNE = 0, /* round to nearest, ties to even                                 */
  FORGE_ROUND_SR = 1   /* stochastic rounding from a counter-based hash of
                          (seed, step, tensor, flat index)                               */
} forge_round;

typedef struct {
  void* data;     /* device pointer                                   */
  int32_t dtype;  /* forge_dtype                                      */
  int64_t rows;
  int64_t cols;
  int64_t ld;     /* leading dimension in elements, >= cols           */
} forge_mat;

/* One optimizer state tensor.  F32 / BF16: values in q.  S8 (first moment)
 * / U8 (second moment): codes in q plus one fp32 scale per `block`
 * consecutive elements of a row, `scale` being a dense row-major
 * [rows, cols / block] fp32 device array.  Stored value = code * scale.
 * S8 codes are symmetric in -127..127 (scale = absmax / 127); U8 codes
 * reserve 0 for an exact zero and use 1..255 for positive values
 * (scale = absmax / 255), which keeps the second moment away from zero
 * (paper, section 2.3 and Appendix B).
 * E4M3 (either moment; the paper's FP8 moment quantization, section 3.6):
 * OCP FP8 E4M3 codes (largest finite 448, no infinities) with the same
 * block scales: scale = absmax / 448, code = the E4M3 value nearest (ties
 * to even, saturating at 448) to x * (448 / absmax); a positive second
 * moment never takes code 0 (it takes the smallest subnormal, 2^-9).
 * Stored value = E4M3 value of the code * scale. */
typedef struct {
  forge_mat q;
  float* scale;   /* S8 / U8 / E4M3 only, else NULL               */
  int32_t block;  /* S8 / U8 / E4M3 only: 32, 64 or 128, else 0   */
} forge_state;

typedef struct {
  int32_t opt;    /* forge_optim */
  int32_t round;  /* forge_round */
  double lr;           /* eta                                                        */
  double beta1;        /* AdamW / NAdam / RAdam / Lion beta1; SGD-m momentum         */
  double beta2;        /* AdamW / NAdam / RAdam / Lion beta2; RMSprop smoothing a     */
  double eps;          /* AdamW, NAdam, RAdam, RMSprop, AdaGrad                       */
  double weight_decay; /* lambda: decoupled (AdamW, NAdam, RAdam, Lion), coupled L2
                          (SGD-m, RMSprop, AdaGrad, SGD)                             */
} forge_hyper;

/*
 * forge_wgrad_step -- the fused hot path.
 *
 * X  : [BT, K], dtype BF16 or F32.      dY : [BT, N], same dtype as X.
 * W  : [N, K], BF16 or F32, updated in place.
 * m  : [N, K] first state, F32 / BF16 / S8 / E4M3: AdamW, NAdam, RAdam, Lion,
 *      SGD-m (NULL for RMSprop, AdaGrad, SGD).
 * v  : [N, K] second state, F32 / BF16 / U8 / E4M3: AdamW, NAdam, RAdam,
 *      RMSprop, AdaGrad (NULL for Lion, SGD-m, SGD).
 * h  : optimizer and hyper-parameters.  step: the 1-based global step t,
 *      used by the AdamW bias correction 1/(1 - beta^t) and by the SR key.
 * seed: 64-bit stochastic-rounding seed.
 *
 * Supported combinations: X/dY in {BF16, F32} x W in {BF16, F32} x
 *   AdamW (m, v) in {(F32, F32), (BF16, BF16), (S8, U8), (E4M3, E4M3)},
 *   NAdam / RAdam (m, v) in {(F32, F32), (BF16, BF16)},
 *   Lion / SGD-m m in {F32, BF16, S8, E4M3},
 *   RMSprop / AdaGrad v in {F32, BF16}, or SGD (no state).
 *   A missing required state is E_NULL, a state the optimizer does not keep
 *   is E_UNSUPPORTED.
 * Int8 and E4M3 states need K % block == 0.  N * K must be < 2^32 (flat SR index).
 * BT may be 0 (G = 0: the step still applies decay / momentum).
 * N == 0 or K == 0 is a no-op.
 *
 * Errors: FORGE_E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_STEP, E_HYPER,
 * E_ALIAS, E_UNSUPPORTED (nothing enqueued) or E_HIP (launch failed).
 */
forge_status forge_wgrad_step(const forge_mat* X, const forge_mat* dY, forge_mat* W,
                              forge_state* m, forge_state* v, const forge_hyper* h,
                              int64_t step, uint64_t seed, void* stream);

/*
 * FP8 weight storage (paper, section 3.6 and Figure 7, "FP8 w": FP8 weight
 * quantization folded into the per-tile kernel; the pages give no format,
 * scale or rounding rule, so this is the library's reading).  The weight is
 * a forge_state of OCP E4M3 codes with one fp32 scale per `block`
 * (32 / 64 / 128) consecutive elements of a row, the moments' block scheme:
 * stored value = fp32(E4M3 value of the code * scale), scale =
 * fp32(absmax / 448), and the new weight of a block is encoded from
 * y = fp32(w * fp32(448 / absmax)):
 *   h->round == FORGE_ROUND_RNE: the E4M3 value nearest to y (ties to even,
 *     saturating at 448), as for E4M3 moments;
 *   h->round == FORGE_ROUND_SR: stochastic rounding with the weight's SR
 *     bits r (16 bits, the bf16 weight's key and flat index): for
 *     |y| >= 2^-6, r * 2^4 is added to the 20 low fraction bits of |y|'s
 *     fp32 pattern, which are then cleared; for |y| < 2^-6 (the subnormal
 *     range, spacing 2^-9) the value is ((floor(|y| 2^25) + r) >> 16) 2^-9;
 *     the magnitude saturates at 448 and the sign is kept.  |y| rounds away
 *     from zero with probability equal to its position between its two
 *     grid neighbours (quantised to 2^-16), so the store is unbiased.
 * Non-finite weights are outside the contract.  A block-scaled m / v must
 * use the weight's block size.
 *
 * forge_wgrad_step_fp8w -- forge_wgrad_step with such a weight: the fused
 * kernel decodes W, applies the step in fp32 and re-encodes W (codes and
 * scales, in place).  X and dY must be BF16.  Supported: AdamW with (m, v)
 * in {(F32, F32), (BF16, BF16), (S8, U8), (E4M3, E4M3)}; Lion and SGD-m
 * with m in {F32, BF16, E4M3}.  W->q.dtype must be FORGE_E4M3 (else E_DTYPE),
 * K % W->block == 0 (else E_SHAPE), W->scale non-NULL (else E_NULL) and
 * not overlapping any other buffer (else E_ALIAS).  Other arguments and
 * errors as forge_wgrad_step (E_UNSUPPORTED for fp32 inputs or another
 * optimizer / state combination).
 */
forge_status forge_wgrad_step_fp8w(const forge_mat* X, const forge_mat* dY, forge_state* W, forge_state* m,
                                   forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed,
                                   void* stream);

/* The validation of forge_wgrad_step_fp8w alone (no device call). */
forge_status forge_wgrad_check_fp8w(const forge_mat* X, const forge_mat* dY, const forge_state* W,
                                    const forge_state* m, const forge_state* v, const forge_hyper* h,
                                    int64_t step);

/*
 * forge_dgrad_fp8w -- forge_dgrad (dX = dY W, paper Appendix A, Remark 1)
 * from an E4M3 weight with block scales, decoded exactly to the values the
 * step stores (fp32 code value * scale), fp32 accumulation over N.
 * dY: [BT, N] BF16 or F32; dX: [BT, K] BF16 (round to nearest even) or F32,
 * not overlapping dY, W or its scales.  bf16 dY with 16-byte aligned rows
 * of dY and of the codes, N % 8 == 0 and K % 16 == 0 runs on the bf16
 * matrix cores: each decoded weight is split exactly into three bf16 terms
 * (8 significant bits each), so every product is exact and the sum is
 * accumulated in fp32.  Other bf16 dY runs on the fp32 matrix cores
 * (v_mfma_f32_32x32x2_f32 on the exactly decoded operands), fp32 dY on the
 * plain fp32 kernel.
 * Errors: those of forge_dgrad, and E_DTYPE / E_SHAPE / E_NULL / E_ALIGN
 * for the weight state as forge_wgrad_step_fp8w.
 */
forge_status forge_dgrad_fp8w(const forge_mat* dY, const forge_state* W, forge_mat* dX, void* stream);

/*
 * forge_wgrad_step_group -- forge_wgrad_step on n independent layers that
 * share one optimizer, step and hyper-parameters, with as few launches as
 * possible.  Layers whose gradients become available together in a backward
 * pass (q/k/v after attention, gate/up after the MLP activation) are the
 * intended use: their tiles are scheduled as one grid (the tile scheduling
 * of FORGE, Section 3 and Algorithm 1: one workgroup per 128 x 128 tile,
 * here over the union of the layers' tile spaces).
 *
 * layers[i] holds the arguments forge_wgrad_step takes for layer i, and its
 * own SR seed.  The result equals n separate forge_wgrad_step calls, bit for
 * bit.  Layers may share inputs (q/k/v read the same X) but nothing a layer
 * writes (W, m, v, scales) may overlap any buffer of another layer.  All
 * non-empty layers must have the same X / W / m / v dtypes and block size;
 * shapes and BT may differ.  Aligned bf16 layers with BT < 2048 run in one
 * launch; any other layer gets its own launch, on the same stream.
 *
 * Errors: FORGE_E_SHAPE (n < 1 or n > FORGE_GROUP_MAX), E_NULL, every error
 * of forge_wgrad_step for each layer, E_UNSUPPORTED (formats differ between
 * layers), E_ALIAS (between layers) -- all before anything is enqueued -- or
 * E_HIP.
 */
#define FORGE_GROUP_MAX 8

typedef struct {
  const forge_mat* X;
  const forge_mat* dY;
  forge_mat* W;
  forge_state* m;
  forge_state* v;  /* as forge_wgrad_step: NULL unless the optimizer keeps a second state */
  uint64_t seed;
} forge_layer;

forge_status forge_wgrad_step_group(const forge_layer* layers, int32_t n, const forge_hyper* h,
                                    int64_t step, void* stream);

/*
 * Exact gradient accumulation (paper, Appendix L): for an effective batch of
 * several micro-batches, each micro-step adds its weight gradient into an
 * fp32 accumulator in device memory, and the fused step fires once, at the
 * final micro-step, on the summed gradient.
 *
 * forge_wgrad_accumulate -- one micro-step: acc = dY^T X (first != 0) or
 * acc += dY^T X (first == 0), in fp32, with the tiled reduction of the
 * fused kernels (one fp32 addition of each tile's gradient into acc).
 * acc: [N, K] F32, caller-owned device buffer, any ld >= K, not overlapping X
 * or dY.  X, dY as for forge_wgrad_step (BT may be 0: acc = 0 or unchanged).
 * Errors: FORGE_E_NULL, E_SHAPE, E_DTYPE (acc not F32; X, dY as for
 * forge_wgrad_step), E_ALIGN, E_ALIAS (nothing enqueued) or E_HIP.
 */
forge_status forge_wgrad_accumulate(const forge_mat* X, const forge_mat* dY, forge_mat* acc, int32_t first,
                                    void* stream);

/*
 * forge_wgrad_step_accumulated -- the final micro-step: G = acc + dY^T X
 * (this micro-batch's gradient), then exactly the step of forge_wgrad_step
 * on G (same arguments, formats, rules and errors).  acc must not overlap
 * any other argument.  acc is consumed: its contents are unspecified after
 * the call (aligned bf16 inputs read it inside the fused kernel; other
 * layouts first add this micro-batch into it and then step from it, with
 * the same fp32 addition, so the result is the same either way).
 */
forge_status forge_wgrad_step_accumulated(const forge_mat* X, const forge_mat* dY, forge_mat* acc, forge_mat* W,
                                          forge_state* m, forge_state* v, const forge_hyper* h, int64_t step,
                                          uint64_t seed, void* stream);

/*
 * forge_dgrad -- the input gradient dX = dY W of the layer (the GEMM that
 * must read W before the fused step overwrites it: paper, Appendix A,
 * Remark 1), fp32 accumulation over N.
 * dY : [BT, N] BF16 or F32.   W : [N, K] BF16 or F32.
 * dX : [BT, K] BF16 (round to nearest even) or F32, written; must not
 *      overlap dY or W.
 * bf16 dY and W with 16-byte aligned rows and N, K multiples of 8 take the
 * MFMA kernel; any other combination a plain fp32 kernel.
 * Errors: FORGE_E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_ALIAS (nothing
 * enqueued) or E_HIP.
 */
forge_status forge_dgrad(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* stream);

/*
 * forge_dgrad_workspace_bytes -- bytes of device workspace forge_dgrad_split
 * uses for dY [BT, N] and W [N, K] on the MFMA path: splits x BT x K x 4 when
 * the reduction over N is split across workgroups (too few output tiles to
 * fill the chip and a long reduction: up to 8 splits of 256 x 256 tiles, or
 * up to 4 of 128-token tiles), else 0.  Non-positive or too-large sizes
 * give 0.  Host-only, no device call.
 */
int64_t forge_dgrad_workspace_bytes(int64_t BT, int64_t N, int64_t K);

/*
 * forge_dgrad_split -- forge_dgrad (same dX, paper, Appendix A, Remark 1)
 * with the reduction over N split across workgroups where
 * forge_dgrad_workspace_bytes is non-zero and the MFMA path applies: each
 * split writes an fp32 partial [BT, K] into `workspace`, and a second kernel
 * adds the partials in split order (a fixed order: the result is the same
 * from call to call, and within the fp32 summation bound of the exact
 * product like forge_dgrad's) and stores dX.  Elsewhere it is forge_dgrad
 * and the workspace is not touched.
 * workspace : caller-owned device memory of `workspace_bytes` bytes,
 *             16-byte aligned, not overlapping dY, W or dX; its contents
 *             are scratch (overwritten, not read before written).  May be
 *             NULL when no workspace is needed.
 * Errors: those of forge_dgrad; E_NULL (workspace needed but NULL), E_SHAPE
 * (workspace_bytes negative or smaller than needed), E_ALIGN, E_ALIAS
 * (nothing enqueued), or E_HIP.
 */
forge_status forge_dgrad_split(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* workspace,
                               int64_t workspace_bytes, void* stream);

/*
 * forge_dgrad_split_noalloc -- forge_dgrad_split for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, splits and reduction
 * order, so the same dX bit for bit, with the split partials in a
 * file-scope device array of FORGE_DGRAD_SCRATCH_BYTES (64 MiB) that the
 * library holds on each GPU it runs on until the process ends, instead of a
 * caller workspace.  The call allocates nothing.  Every call on a GPU shares
 * that GPU's array, so calls that may overlap on one GPU (several streams,
 * several host threads) race and must be serialised by the caller.
 * Shapes whose split needs more (forge_dgrad_workspace_bytes(BT, N, K) >
 * FORGE_DGRAD_SCRATCH_BYTES) are rejected with FORGE_E_SCRATCH before
 * anything is enqueued; every Llama-3.1-8B layer at BT <= 512 fits.
 * Arguments and other errors as forge_dgrad.
 */
#define FORGE_DGRAD_SCRATCH_BYTES (64ll << 20)
forge_status forge_dgrad_split_noalloc(const forge_mat* dY, const forge_mat* W, forge_mat* dX, void* stream);

/*
 * forge_backward_step -- a linear layer's whole weight-side backward in the
 * order Remark 1 requires: dX = dY W from the current W (forge_dgrad), then
 * forge_wgrad_step, enqueued in that order on `stream`.  Arguments as for
 * the two calls; dX must not overlap any other buffer.  Errors: those of
 * both calls, all checked before anything is enqueued, or E_HIP.
 */
forge_status forge_backward_step(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m,
                                 forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed,
                                 forge_mat* dX, void* stream);

/*
 * forge_backward_step_split -- forge_backward_step with dX computed as
 * forge_dgrad_split does (the same order: dX from the current W, then the
 * fused step).  workspace / workspace_bytes as for forge_dgrad_split
 * (forge_dgrad_workspace_bytes(BT, N, K) bytes); the workspace must not
 * overlap any other buffer either.  Errors: those of forge_backward_step and
 * of forge_dgrad_split, all checked before anything is enqueued, or E_HIP.
 */
forge_status forge_backward_step_split(const forge_mat* X, const forge_mat* dY, forge_mat* W, forge_state* m,
                                       forge_state* v, const forge_hyper* h, int64_t step, uint64_t seed,
                                       forge_mat* dX, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * forge_wgrad_check -- the validation of forge_wgrad_step alone: same
 * arguments, same return codes, no device call at all (usable on a host
 * without a GPU).
 */
forge_status forge_wgrad_check(const forge_mat* X, const forge_mat* dY, const forge_mat* W,
                               const forge_state* m, const forge_state* v, const forge_hyper* h,
                               int64_t step);

/*
 * forge_wgrad_unfused -- the two-phase baseline the fused path replaces
 * (paper, section 2.1: the gradient is stored in device memory, then the
 * optimizer reads it back).  Kernel 1 computes G with the same tiles and
 * accumulation order as forge_wgrad_step and writes it to `dW` ([N, K],
 * leading dimension K) as F32 or BF16 (round to nearest even); kernel 2
 * applies the same optimizer step reading G back.  With dW_dtype == F32 the
 * results are bit-identical to forge_wgrad_step (paper, Corollary 1(a)).
 * dW: caller-owned device workspace of N*K elements of dW_dtype, must not
 * overlap any other argument.  Other arguments and errors as
 * forge_wgrad_step.
 */
forge_status forge_wgrad_unfused(const forge_mat* X, const forge_mat* dY, forge_mat* W,
                                 forge_state* m, forge_state* v, const forge_hyper* h,
                                 int64_t step, uint64_t seed, void* dW, int32_t dW_dtype,
                                 void* stream);

/*
 * forge_debug_sr_bf16 -- test hook: rounds n fp32 values to bf16 with the
 * same device stochastic-rounding function and key derivation the step
 * kernels use for tensor `tensor_id` (0 = W, 1 = m, 2 = v), element i taking
 * flat index i.  in: n floats, out: n uint16 bf16 patterns, both device
 * pointers.  Errors: E_NULL, E_SHAPE (n < 0 or n >= 2^32), E_ALIAS,
 * E_STEP, E_HIP.
 */
forge_status forge_debug_sr_bf16(const float* in, uint16_t* out, int64_t n, uint64_t seed,
                                 int64_t step, uint32_t tensor_id, void* stream);

/*
 * forge_debug_e4m3 -- test hook: the device's E4M3 rounding (nearest, ties
 * to even, saturating at 448; the element code of the E4M3 state format) of
 * n floats, out[i] = code of in[i], through the same four-value packing the
 * fused step uses.  Device pointers.  Errors: E_NULL,
 * E_SHAPE (n < 0 or n >= 2^32), E_ALIGN, E_ALIAS, E_HIP.
 */
forge_status forge_debug_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

/*
 * forge_debug_e4m3_sr -- test hook: the FP8 weight store's stochastic
 * rounding onto the E4M3 grid (the reading of the paper's section 3.6 given
 * with forge_wgrad_step_fp8w below) of n floats, out[i] = code of in[i] with
 * the 16 SR bits of flat index i under the weight's key for (seed, step),
 * through the same four-value packing the fused step uses.  Values beyond
 * +-448 saturate.  Device pointers.  Errors: E_NULL, E_SHAPE (n < 0 or
 * n >= 2^32), E_STEP (step < 1), E_ALIGN, E_ALIAS, E_HIP.
 */
forge_status forge_debug_e4m3_sr(const float* in, uint8_t* out, int64_t n, uint64_t seed, int64_t step,
                                 void* stream);

/*
 * forge_debug_quotients -- test hook: an exhaustive check of the block
 * quantiser's scale and reciprocal (correctly rounded fp32 a / QMAX and
 * QMAX / a, paper section 2.3 and Appendix B) computed by short fma
 * sequences: for every fp32 a in [2^-64, 2^126) and QMAX in {127, 255, 448}
 * it compares them with IEEE division.  counts: device array of
 * FORGE_QUOTIENT_COUNTS uint64, 8-byte aligned; group g (entries 8g .. 8g+7,
 * g < FORGE_QUOTIENT_COUNTS / 8) receives the mismatch counts of a/127,
 * 127/a, a/255, 255/a, a/448, 448/a and, in entry 8g+6, the number of a
 * values it checked; entry 8g+7 is not written.  The sums over the groups
 * give the totals (the checked counts add up to 2^126 - 2^-64 in fp32 bit
 * patterns, 0x5F000000).  Errors: E_NULL, E_ALIGN, E_HIP.
 */
#define FORGE_QUOTIENT_COUNTS (2048 * 8)
forge_status forge_debug_quotients(uint64_t* counts, void* stream);

/*
 * forge_debug_quant -- test hook: the fused step's 8-bit block quantiser
 * (the store of an S8, U8 or E4M3 state: paper, section 2.3 and Appendix B
 * for int8, section 3.6 for FP8; the rules are those of forge_state above)
 * on its own, through the same device function and thread mapping as the
 * epilogue.  in: dense [rows, cols] fp32 device array; codes: dense
 * [rows, cols] bytes (int8 / uint8 / E4M3), 4-byte aligned; scales: dense
 * [rows, cols / block] fp32, written.
 * dtype FORGE_S8 takes the first-moment rule (second_moment = 0), FORGE_U8
 * the second-moment rule (second_moment = 1), FORGE_E4M3 either.
 * block: 32, 64 or 128 with cols % block == 0; rows * cols < 2^32.
 * A block whose absmax is below 2^-64 is quantised as if the exponent range
 * were unbounded (x * (QMAX / absmax) with no overflow).
 * Errors: E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_ALIAS, E_HIP.
 */
forge_status forge_debug_quant(const float* in, uint8_t* codes, float* scales, int64_t rows, int64_t cols,
                               int32_t dtype, int32_t second_moment, int32_t block, void* stream);

/*
 * forge_debug_copy -- measurement hook for the HBM roofline (the pages
 * measure their device's streaming bandwidth to quote fractions of it):
 * copies `bytes` from src to dst in 16-byte non-temporal loads and stores
 * (the fused epilogue's access width), one contiguous chunk per workgroup.  Device pointers,
 * 16-byte aligned, non-overlapping; bytes a multiple of 16.  Errors: E_NULL,
 * E_SHAPE (bytes < 0 or not a multiple of 16), E_ALIGN, E_ALIAS, E_HIP.
 */
forge_status forge_debug_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * forge_debug_state_stream -- measurement hook for the HBM roofline of the
 * fused step's own traffic: streams a bf16 W and fp32 m, v [N, K] (dense,
 * row-major) through the epilogue's access pattern -- 128 x 128 tiles in
 * row-major order, one 256-thread workgroup per tile, 16-byte non-temporal
 * accesses (8-byte for W), 8 row passes in flight -- reading and writing
 * every element once (20 bytes per element) with no gradient and a trivial
 * update (m and v incremented by 1, W's bit pattern by 1).  Device
 * pointers: W 8-byte aligned, m and v 16-byte aligned, pairwise disjoint.
 * N and K multiples of 128, N * K < 2^32.  Errors: E_SHAPE, E_NULL,
 * E_ALIGN, E_ALIAS, E_HIP.
 */
forge_status forge_debug_state_stream(uint16_t* W, float* m, float* v, int64_t N, int64_t K, void* stream);

/*
 * forge_debug_mfma_peak -- measurement hook for the matrix-core roofline:
 * `blocks` workgroups of 4 waves; every wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 (32,768 flops each) on register
 * operands of ones, i.e. blocks * 4 * iters * 131,072 flops.  out: device
 * array of 256 * blocks floats, each set to 64 * iters (exact).  Errors:
 * E_NULL, E_SHAPE (blocks or iters outside 1 .. 2^20), E_ALIGN, E_HIP.
 */
forge_status forge_debug_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream);

/* Human-readable name of a status code (static string). */
const char* forge_status_str(forge_status s);

/* Library version string (static). */
const char* forge_version(void);

/* HIP's description of the error behind the last FORGE_E_HIP returned on the
 * calling thread ("no error" if there was none).  The string is static and
 * stays valid until the process ends. */
const char* forge_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FORGE_H */
