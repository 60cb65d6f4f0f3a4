// gfx950 kernels: fused weight gradient + element-wise optimizer step.
//
// FORGE paper (arXiv 2606.22932), section 2.2 and Algorithm 1: for every
// 128 x 128 tile (i, j) of W the tile gradient
//     G_ij = sum_kappa dY[kappa, rows_i]^T X[kappa, cols_j]        (Eq. 5)
// is accumulated over token chunks kappa in fp32 (Phase 1), the optimizer is
// applied to the tile in place (Phase 2) and only W and its state are
// written back (Phase 3).
//
// Mainloop (bf16): both operands have the token axis -- the contraction
// axis -- as their slow axis in memory, so a chunk of TK tokens x 128
// features is copied row by row (16-byte loads along the features, fully
// coalesced) into LDS, and the MFMA operands, which need 8 consecutive
// tokens of one feature per lane, are read back with the gfx950 transposing
// LDS read (ds_read_b64_tr_b16).  Rows are XOR-swizzled in 64-byte units so
// that the four token rows one transposing read touches fall in distinct
// banks.  v_mfma_f32_32x32x16_bf16, 4 waves in a 2 x 2 arrangement of 64 x
// 64 sub-tiles, double-buffered LDS stages.  fp32 inputs use
// v_mfma_f32_32x32x2_f32 straight from a row-major LDS copy.
//
// Epilogue: the fp32 accumulators are staged through LDS so that each
// thread owns 8 consecutive elements of a row; W / m / v are then read and
// written with 16-byte accesses, and an int8 block (<= 128 elements of one
// row) is owned by <= 16 adjacent lanes, which reduce its absmax with lane
// shuffles.  The element-wise step is written once (step_chunk) and is used
// by the fused kernel and by the unfused baseline's step kernel alike, so
// the two are bit-identical when the baseline keeps G in fp32 (paper,
// Corollary 1(a)).
//
// All arithmetic is IEEE fp32 with explicit fmaf; the library is compiled
// with -ffp-contract=off so no other contraction happens.

#include "forge_internal.h"

namespace forge {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int TILE = 128;                        // T_R = T_C
constexpr int NT = 256;                          // threads per workgroup (4 waves)
constexpr int GP = TILE + 4;                     // fp32 row pitch of the staged G tile
constexpr int LDS_G = TILE * GP * 4;             // 67,584 bytes
constexpr int LDS_MAIN = 2 * 2 * 64 * TILE * 2;  // 2 stages x (dY, X) x 64 tok x 128 x bf16 = 65,536
constexpr int LDS_BYTES = LDS_G > LDS_MAIN ? LDS_G : LDS_MAIN;
constexpr uint32_t GOLDEN = 0x9E3779B9u;

// ------------------------------------------------------------------------
// Rounding helpers (paper, Appendix C)
// ------------------------------------------------------------------------
// MurmurHash3 32-bit finaliser (Appleby, public domain).
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Stochastic rounding: add 16 random bits below the bf16 cut and truncate;
// the carry into the kept half happens with probability (x - x_lo)/ULP.
__device__ __forceinline__ uint32_t bf16_sr_bits(float x, uint32_t key, uint32_t idx) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return bf16_rne_bits(x);  // Inf / NaN
  uint32_t r = fmix32(key ^ (idx * GOLDEN)) >> 16;
  return (u + r) >> 16;
}

__device__ __forceinline__ float bf16_val(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------------------------------
// Tile order: workgroup b runs on XCD b % 8; give each XCD a contiguous
// range of logical tiles, and walk that range in groups of GROUP tile rows so
// that neighbouring workgroups share the activation panels in that XCD's L2.
// ------------------------------------------------------------------------
__device__ __forceinline__ void tile_coords(int bid, int tiles_n, int tiles_k, int& ti, int& tj) {
  const int T = tiles_n * tiles_k;
  const int x = bid & 7, pos = bid >> 3;
  const int q = T >> 3, r = T & 7;
  const int logical = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + pos;
  constexpr int GROUP = 8;
  const int gsize = GROUP * tiles_k;
  const int g = logical / gsize;
  const int first = g * GROUP;
  const int rows = min(tiles_n - first, GROUP);
  const int in = logical - g * gsize;
  ti = first + in % rows;
  tj = in / rows;
}

// ------------------------------------------------------------------------
// Mainloop, bf16 inputs
// ------------------------------------------------------------------------
struct MainBF16 {
  static constexpr int TK = 64;                       // tokens per chunk
  static constexpr int OPB = TK * TILE * 2;           // bytes per operand per stage
  static constexpr int STAGE = 2 * OPB;
  u32x4 ra[4], rb[4];                                 // next chunk, in flight

  // One 16-byte row segment: 8 features of token `tok`, zero outside.
  __device__ __forceinline__ static u32x4 load8(const uint16_t* base, int64_t ld, int tok, int BT,
                                                int f, int F, bool vec) {
    if (tok < BT && vec && f + 8 <= F)
      return *reinterpret_cast<const u32x4*>(base + (int64_t)tok * ld + f);
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      e[i] = (tok < BT && f + i < F) ? (uint32_t)base[(int64_t)tok * ld + f + i] : 0u;
    return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
  }

  __device__ __forceinline__ void load(const KArgs& a, int kc, int row0, int col0) {
    const int tid = threadIdx.x;
    const int f = (tid & 15) * 8;
    const bool vec = a.vec_in != 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = kc * TK + (tid >> 4) + 16 * r;
      ra[r] = load8(static_cast<const uint16_t*>(a.dY), a.lddy, tok, a.BT, row0 + f, a.N, vec);
      rb[r] = load8(static_cast<const uint16_t*>(a.X), a.ldx, tok, a.BT, col0 + f, a.K, vec);
    }
  }

  // byte offset of (token row t, feature f) in an operand region
  __device__ __forceinline__ static int off(int t, int f) { return t * (TILE * 2) + ((f * 2) ^ ((t & 3) << 6)); }

  __device__ __forceinline__ void store(char* stage) const {
    const int tid = threadIdx.x;
    const int f = (tid & 15) * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = (tid >> 4) + 16 * r;
      *reinterpret_cast<u32x4*>(stage + off(t, f)) = ra[r];
      *reinterpret_cast<u32x4*>(stage + OPB + off(t, f)) = rb[r];
    }
  }

  // 8 consecutive tokens of feature f0 + lane%32 (lane l gets tokens
  // t0 + 8*(l/32) + 0..7): two transposing reads of 4 tokens each.
  __device__ __forceinline__ static bf16x8 frag(char* region, int t0, int f0, int lane) {
    const int t = t0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int f = f0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(region + off(t, f)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(region + off(t + 4, f)));
    const s16x4 both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, both);
  }

  __device__ __forceinline__ static void compute(f32x16 (&acc)[2][2], char* stage, int wr, int wc,
                                                 int lane) {
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = frag(stage, ks * 16, wr * 64 + b * 32, lane);
        fb[b] = frag(stage + OPB, ks * 16, wc * 64 + b * 32, lane);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------------------
// Mainloop, fp32 inputs
// ------------------------------------------------------------------------
struct MainF32 {
  static constexpr int TK = 32;
  static constexpr int OPB = TK * TILE * 4;
  static constexpr int STAGE = 2 * OPB;
  f32x4 ra[4], rb[4];

  __device__ __forceinline__ static f32x4 load4(const float* base, int64_t ld, int tok, int BT, int f,
                                                int F, bool vec) {
    if (tok < BT && vec && f + 4 <= F) return *reinterpret_cast<const f32x4*>(base + (int64_t)tok * ld + f);
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (tok < BT && f + i < F) ? base[(int64_t)tok * ld + f + i] : 0.f;
    return r;
  }

  __device__ __forceinline__ void load(const KArgs& a, int kc, int row0, int col0) {
    const int tid = threadIdx.x;
    const int f = (tid & 31) * 4;
    const bool vec = a.vec_in != 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = kc * TK + (tid >> 5) + 8 * r;
      ra[r] = load4(static_cast<const float*>(a.dY), a.lddy, tok, a.BT, row0 + f, a.N, vec);
      rb[r] = load4(static_cast<const float*>(a.X), a.ldx, tok, a.BT, col0 + f, a.K, vec);
    }
  }

  __device__ __forceinline__ void store(char* stage) const {
    const int tid = threadIdx.x;
    const int f = (tid & 31) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = (tid >> 5) + 8 * r;
      *reinterpret_cast<f32x4*>(stage + (t * TILE + f) * 4) = ra[r];
      *reinterpret_cast<f32x4*>(stage + OPB + (t * TILE + f) * 4) = rb[r];
    }
  }

  __device__ __forceinline__ static void compute(f32x16 (&acc)[2][2], char* stage, int wr, int wc,
                                                 int lane) {
    const float* A = reinterpret_cast<const float*>(stage);
    const float* B = reinterpret_cast<const float*>(stage + OPB);
#pragma unroll 4
    for (int ks = 0; ks < TK / 2; ++ks) {
      const int t = ks * 2 + (lane >> 5);
      float fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = A[t * TILE + wr * 64 + b * 32 + (lane & 31)];
        fb[b] = B[t * TILE + wc * 64 + b * 32 + (lane & 31)];
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
    }
  }
};

template <int IN> struct MainSel;
template <> struct MainSel<FMT_BF16> { using T = MainBF16; };
template <> struct MainSel<FMT_F32> { using T = MainF32; };

// Phase 1 of Algorithm 1 for tile (row0, col0), then the fp32 tile in LDS:
// sG[r * GP + c] = G[row0 + r][col0 + c].
template <int IN>
__device__ __forceinline__ void tile_gradient(const KArgs& a, char* lds, int row0, int col0) {
  using M = typename MainSel<IN>::T;
  static_assert(2 * M::STAGE <= LDS_BYTES, "LDS budget");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;

  const int nk = (a.BT + M::TK - 1) / M::TK;
  M ml;
  if (nk > 0) {
    ml.load(a, 0, row0, col0);
    ml.store(lds);
    __syncthreads();
  }
  for (int kc = 0; kc < nk; ++kc) {
    char* cur = lds + (kc & 1) * M::STAGE;
    if (kc + 1 < nk) ml.load(a, kc + 1, row0, col0);
    M::compute(acc, cur, wr, wc, lane);
    if (kc + 1 < nk) ml.store(lds + ((kc + 1) & 1) * M::STAGE);
    __syncthreads();
  }
  // Stage G (the mainloop buffers are dead after the last barrier).
  float* sG = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wr * 64 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int c = wc * 64 + bj * 32 + (lane & 31);
        sG[r * GP + c] = acc[bi][bj][e];
      }
  __syncthreads();
}

// ------------------------------------------------------------------------
// Element-wise step on 8 consecutive elements of one row (Algorithm 1
// Phase 2 and 3; Appendix N families)
// ------------------------------------------------------------------------
template <int FMT> struct Io;

template <> struct Io<FMT_F32> {
  __device__ __forceinline__ static void load(const void* base, int64_t off, int nv, bool vec, float (&x)[8]) {
    const float* p = static_cast<const float*>(base) + off;
    if (vec && nv == 8) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[i + 4] = b[i]; }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = i < nv ? p[i] : 0.f;
    }
  }
  __device__ __forceinline__ static void store(void* base, int64_t off, int nv, bool vec, const float (&x)[8],
                                               int, uint32_t, uint32_t) {
    float* p = static_cast<float*>(base) + off;
    if (vec && nv == 8) {
      *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < nv) p[i] = x[i];
    }
  }
};

template <> struct Io<FMT_BF16> {
  __device__ __forceinline__ static void load(const void* base, int64_t off, int nv, bool vec, float (&x)[8]) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if (vec && nv == 8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(a[i] << 16);
        x[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = i < nv ? bf16_val(p[i]) : 0.f;
    }
  }
  // sr != 0: stochastic rounding keyed on (key, idx0 + i); else RNE.
  __device__ __forceinline__ static void store(void* base, int64_t off, int nv, bool vec, const float (&x)[8],
                                               int sr, uint32_t key, uint32_t idx0) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = sr ? bf16_sr_bits(x[i], key, idx0 + i) : bf16_rne_bits(x[i]);
    uint16_t* p = static_cast<uint16_t*>(base) + off;
    if (vec && nv == 8) {
      *reinterpret_cast<u32x4*>(p) =
          u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < nv) p[i] = (uint16_t)b[i];
    }
  }
};

// int8 codes: load = dequantise (code * scale in fp32).
template <> struct Io<FMT_S8> {
  __device__ __forceinline__ static void load_codes(const void* base, int64_t off, int nv, bool vec,
                                                    float scale, float (&x)[8]) {
    const int8_t* p = static_cast<const int8_t*>(base) + off;
    if (vec && nv == 8) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)(int8_t)((a[i >> 2] >> (8 * (i & 3))) & 0xFF) * scale;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = i < nv ? (float)p[i] * scale : 0.f;
    }
  }
};
template <> struct Io<FMT_U8> {
  __device__ __forceinline__ static void load_codes(const void* base, int64_t off, int nv, bool vec,
                                                    float scale, float (&x)[8]) {
    const uint8_t* p = static_cast<const uint8_t*>(base) + off;
    if (vec && nv == 8) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)((a[i >> 2] >> (8 * (i & 3))) & 0xFF) * scale;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = i < nv ? (float)p[i] * scale : 0.f;
    }
  }
};

// Block-absmax quantisation of 8 values per lane; a block is `lpb` adjacent
// lanes (lpb = block / 8, a power of two <= 16).  Every lane of the wave
// must call this (lane shuffles).  SIGNED: codes -127..127, scale a/127.
// Unsigned: code 0 only for an exact zero, else 1..255, scale a/255.
template <bool SIGNED>
__device__ __forceinline__ void quantize8(const float (&x)[8], int lpb, bool valid, void* codes_base,
                                          int64_t off, bool vec, float* scale_ptr, bool write_scale) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, SIGNED ? fabsf(x[i]) : x[i]);
  if (!valid) a = 0.f;
  for (int o = 1; o < lpb; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  const float qmax = SIGNED ? 127.f : 255.f;
  const float s = a > 0.f ? a / qmax : 0.f;
  const float inv = a > 0.f ? qmax / a : 0.f;
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r = rintf(x[i] * inv);
    if (SIGNED) {
      r = fminf(fmaxf(r, -127.f), 127.f);
      q[i] = (uint32_t)(int32_t)r & 0xFFu;
    } else {
      r = fminf(fmaxf(r, 1.f), 255.f);
      q[i] = x[i] == 0.f ? 0u : (uint32_t)r;
    }
  }
  if (!valid) return;
  if (write_scale) *scale_ptr = s;
  uint8_t* p = static_cast<uint8_t*>(codes_base) + off;
  if (vec) {
    *reinterpret_cast<u32x2*>(p) = u32x2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                         q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)q[i];
  }
}

// Loaded state of one 8-element chunk.
struct Chunk {
  float w[8], m[8], v[8];
};

template <int OPT, int WF, int MF, int VF>
struct Step {
  static constexpr bool HAS_V = (OPT == OPT_ADAMW);

  __device__ __forceinline__ static void load(const KArgs& a, int p, int q, int nv, Chunk& c) {
    const bool vec = a.vec_state != 0;
    if (p >= a.N || nv <= 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = c.m[i] = c.v[i] = 0.f;
      return;
    }
    if constexpr (!HAS_V) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c.v[i] = 0.f;
    }
    Io<WF>::load(a.W, (int64_t)p * a.ldw + q, nv, vec, c.w);
    if constexpr (MF == FMT_S8) {
      const float s = a.ms[(int64_t)p * (a.K / a.block) + q / a.block];
      Io<FMT_S8>::load_codes(a.m, (int64_t)p * a.ldm + q, nv, vec, s, c.m);
    } else {
      Io<MF>::load(a.m, (int64_t)p * a.ldm + q, nv, vec, c.m);
    }
    if constexpr (HAS_V) {
      if constexpr (VF == FMT_U8) {
        const float s = a.vs[(int64_t)p * (a.K / a.block) + q / a.block];
        Io<FMT_U8>::load_codes(a.v, (int64_t)p * a.ldv + q, nv, vec, s, c.v);
      } else {
        Io<VF>::load(a.v, (int64_t)p * a.ldv + q, nv, vec, c.v);
      }
    }
  }

  // The optimizer on one element, fp32 (Algorithm 1 Phase 2 for AdamW).
  __device__ __forceinline__ static void phi(const EpiConst& k, float g, float& w, float& m, float& v) {
    if constexpr (OPT == OPT_ADAMW) {
      m = fmaf(k.b1, m, k.omb1 * g);                  // m' = b1 m + (1-b1) G
      v = fmaf(k.b2, v, k.omb2 * (g * g));            // v' = b2 v + (1-b2) G^2
      const float den = fmaf(sqrtf(v), k.bc2s, k.eps);  // sqrt(v'/(1-b2^t)) + eps
      const float upd = (m * k.bc1) / den;            // m_hat / den
      w = fmaf(k.decay, w, -k.lr * upd);              // (1 - lr wd) W - lr upd
    } else if constexpr (OPT == OPT_LION) {
      const float c = fmaf(k.b1, m, k.omb1 * g);      // interpolation
      const float s = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
      w = fmaf(k.decay, w, -k.lr * s);
      m = fmaf(k.b2, m, k.omb2 * g);
    } else {                                          // SGD with momentum
      const float gg = fmaf(k.wd, w, g);              // coupled L2
      m = fmaf(k.b1, m, gg);                          // b' = mu b + g
      w = fmaf(-k.lr, m, w);                          // W - lr b'
    }
  }

  // Apply phi to the chunk and store.  Must be called by every lane of the
  // wave when a state is int8 (lane shuffles).
  __device__ __forceinline__ static void apply_store(const KArgs& a, int p, int q, int nv, const float (&g)[8],
                                                     Chunk& c) {
    const bool valid = p < a.N && nv > 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) phi(a.c, g[i], c.w[i], c.m[i], c.v[i]);
    const bool vec = a.vec_state != 0;
    const uint32_t idx0 = (uint32_t)p * (uint32_t)a.K + (uint32_t)q;
    if (valid) Io<WF>::store(a.W, (int64_t)p * a.ldw + q, nv, vec, c.w, a.c.sr, a.c.keyW, idx0);
    if constexpr (MF == FMT_S8) {
      const int lpb = a.block >> 3;
      const bool first = ((threadIdx.x & (lpb - 1)) == 0);
      quantize8<true>(c.m, lpb, valid, a.m, (int64_t)p * a.ldm + q, vec,
                      a.ms + (int64_t)p * (a.K / a.block) + q / a.block, first);
    } else {
      if (valid) Io<MF>::store(a.m, (int64_t)p * a.ldm + q, nv, vec, c.m, a.c.sr, a.c.keyM, idx0);
    }
    if constexpr (HAS_V) {
      if constexpr (VF == FMT_U8) {
        const int lpb = a.block >> 3;
        const bool first = ((threadIdx.x & (lpb - 1)) == 0);
        quantize8<false>(c.v, lpb, valid, a.v, (int64_t)p * a.ldv + q, vec,
                         a.vs + (int64_t)p * (a.K / a.block) + q / a.block, first);
      } else {
        if (valid) Io<VF>::store(a.v, (int64_t)p * a.ldv + q, nv, vec, c.v, a.c.sr, a.c.keyV, idx0);
      }
    }
  }
};

// Epilogue over one 128 x 128 tile: thread t owns, in pass s, the 8
// elements of row (s*16 + t/16) starting at column 8*(t%16).  G comes from
// the LDS staging buffer (fused) or from dW (unfused step kernel).
template <class S, bool FROM_LDS>
__device__ __forceinline__ void tile_epilogue(const KArgs& a, const float* sG, int row0, int col0) {
  const int tid = threadIdx.x;
  const int cl = (tid & 15) * 8;
  const int q = col0 + cl;
  const int nv = min(8, a.K - q);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    Chunk c[4];
    float g[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int rl = (half * 4 + s) * 16 + (tid >> 4);
      S::load(a, row0 + rl, q, nv, c[s]);
      if constexpr (FROM_LDS) {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[s][i] = sG[rl * GP + cl + i];
      } else {
        const int p = row0 + rl;
        const bool ok = p < a.N && nv > 0;
        const int64_t off = (int64_t)p * a.K + q;
        const bool vec = (a.K & 7) == 0;
        if (!ok) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[s][i] = 0.f;
        } else if (a.dw_fmt == FMT_F32) {
          Io<FMT_F32>::load(a.dW, off, nv, vec, g[s]);
        } else {
          Io<FMT_BF16>::load(a.dW, off, nv, vec, g[s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int rl = (half * 4 + s) * 16 + (tid >> 4);
      S::apply_store(a, row0 + rl, q, nv, g[s], c[s]);
    }
  }
}

// ------------------------------------------------------------------------
// Kernels
// ------------------------------------------------------------------------
template <int IN, int OPT, int WF, int MF, int VF>
__global__ void __launch_bounds__(NT, 2) k_fused(const KArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  const int row0 = ti * TILE, col0 = tj * TILE;
  tile_gradient<IN>(a, lds, row0, col0);
  tile_epilogue<Step<OPT, WF, MF, VF>, true>(a, reinterpret_cast<const float*>(lds), row0, col0);
}

template <int IN>
__global__ void __launch_bounds__(NT, 2) k_gemm(const KArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  const int row0 = ti * TILE, col0 = tj * TILE;
  tile_gradient<IN>(a, lds, row0, col0);
  const float* sG = reinterpret_cast<const float*>(lds);
  const int tid = threadIdx.x;
  const int cl = (tid & 15) * 8;
  const int q = col0 + cl;
  const int nv = min(8, a.K - q);
  const bool vec = (a.K & 7) == 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int rl = s * 16 + (tid >> 4);
    const int p = row0 + rl;
    if (p >= a.N || nv <= 0) continue;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = sG[rl * GP + cl + i];
    const int64_t off = (int64_t)p * a.K + q;
    if (a.dw_fmt == FMT_F32) Io<FMT_F32>::store(a.dW, off, nv, vec, g, 0, 0, 0);
    else Io<FMT_BF16>::store(a.dW, off, nv, vec, g, 0, 0, 0);
  }
}

template <int OPT, int WF, int MF, int VF>
__global__ void __launch_bounds__(NT, 2) k_step(const KArgs a) {
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  tile_epilogue<Step<OPT, WF, MF, VF>, false>(a, nullptr, ti * TILE, tj * TILE);
}

__global__ void k_debug_sr(const float* __restrict__ in, uint16_t* __restrict__ out, uint32_t n, uint32_t key) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint16_t)bf16_sr_bits(in[i], key, i);
}

// ------------------------------------------------------------------------
// Dispatch
// ------------------------------------------------------------------------
// Supported (opt, m, v) state layouts.
#define FORGE_STATE_LIST(X)                       \
  X(OPT_ADAMW, FMT_F32, FMT_F32)                  \
  X(OPT_ADAMW, FMT_BF16, FMT_BF16)                \
  X(OPT_ADAMW, FMT_S8, FMT_U8)                    \
  X(OPT_LION, FMT_F32, FMT_NONE)                  \
  X(OPT_LION, FMT_BF16, FMT_NONE)                 \
  X(OPT_LION, FMT_S8, FMT_NONE)                   \
  X(OPT_SGDM, FMT_F32, FMT_NONE)                  \
  X(OPT_SGDM, FMT_BF16, FMT_NONE)                 \
  X(OPT_SGDM, FMT_S8, FMT_NONE)

bool combo_supported(int in_fmt, int w_fmt, int opt, int m_fmt, int v_fmt) {
  if (in_fmt != FMT_F32 && in_fmt != FMT_BF16) return false;
  if (w_fmt != FMT_F32 && w_fmt != FMT_BF16) return false;
#define X(O, M, V) if (opt == O && m_fmt == M && v_fmt == V) return true;
  FORGE_STATE_LIST(X)
#undef X
  return false;
}

static inline dim3 tile_grid(const KArgs& a) { return dim3((unsigned)(a.tiles_n * a.tiles_k)); }

template <int IN, int WF>
static hipError_t fused_w(const KArgs& a, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V)                                                                 \
  if (opt == O && m_fmt == M && v_fmt == V) {                                      \
    hipLaunchKernelGGL((k_fused<IN, O, WF, M, V>), tile_grid(a), dim3(NT), 0, st, a); \
    return hipGetLastError();                                                      \
  }
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_fused(const KArgs& a, int in_fmt, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
  if (in_fmt == FMT_BF16) {
    if (w_fmt == FMT_BF16) return fused_w<FMT_BF16, FMT_BF16>(a, opt, m_fmt, v_fmt, st);
    if (w_fmt == FMT_F32) return fused_w<FMT_BF16, FMT_F32>(a, opt, m_fmt, v_fmt, st);
  } else if (in_fmt == FMT_F32) {
    if (w_fmt == FMT_BF16) return fused_w<FMT_F32, FMT_BF16>(a, opt, m_fmt, v_fmt, st);
    if (w_fmt == FMT_F32) return fused_w<FMT_F32, FMT_F32>(a, opt, m_fmt, v_fmt, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const KArgs& a, int in_fmt, hipStream_t st) {
  if (in_fmt == FMT_BF16) hipLaunchKernelGGL((k_gemm<FMT_BF16>), tile_grid(a), dim3(NT), 0, st, a);
  else if (in_fmt == FMT_F32) hipLaunchKernelGGL((k_gemm<FMT_F32>), tile_grid(a), dim3(NT), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int WF>
static hipError_t step_w(const KArgs& a, int opt, int m_fmt, int v_fmt, hipStream_t st) {
#define X(O, M, V)                                                              \
  if (opt == O && m_fmt == M && v_fmt == V) {                                   \
    hipLaunchKernelGGL((k_step<O, WF, M, V>), tile_grid(a), dim3(NT), 0, st, a); \
    return hipGetLastError();                                                   \
  }
  FORGE_STATE_LIST(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_step(const KArgs& a, int w_fmt, int opt, int m_fmt, int v_fmt, hipStream_t st) {
  if (w_fmt == FMT_BF16) return step_w<FMT_BF16>(a, opt, m_fmt, v_fmt, st);
  if (w_fmt == FMT_F32) return step_w<FMT_F32>(a, opt, m_fmt, v_fmt, st);
  return hipErrorInvalidValue;
}

hipError_t launch_debug_sr(const float* in, uint16_t* out, uint32_t n, uint32_t key, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255u) / 256u);
  hipLaunchKernelGGL(k_debug_sr, dim3(blocks), dim3(256), 0, st, in, out, n, key);
  return hipGetLastError();
}

}  // namespace forge
