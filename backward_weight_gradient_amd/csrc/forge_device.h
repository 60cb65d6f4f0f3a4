#pragma once

// gfx950 device code: fused weight gradient + element-wise optimizer step.
//
// Every kernel here is a template; the family sources (forge_k_*.hip)
// instantiate the launchers at the end of this file for their optimizer /
// state combinations, so the families compile in parallel.
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
// banks.  v_mfma_f32_32x32x16_bf16: 128 x 128 tiles with 4 waves in a 2 x 2
// arrangement of 64 x 64 (a 3- or 4-stage LDS-DMA ring for aligned shapes,
// for three or two workgroups per CU; double-buffered register staging
// otherwise); for long token axes 256 x 256
// tiles with 8 waves of 128 x 64.  fp32 inputs use v_mfma_f32_32x32x2_f32
// straight from a row-major LDS copy.
//
// Epilogue: the fp32 accumulators are staged through LDS (the whole tile, or
// in two 64-row halves where three workgroups share a CU) so that each
// thread owns two 4-element segments of a row; the 16 lanes of a row read
// and write W / m / v in contiguous 64-element runs, and an 8-bit state
// block (<= 128 elements of one row) is owned by <= 16 adjacent lanes,
// which reduce its absmax with DPP row operations.  The element-wise step
// is written once (Step::apply_store) and is used by the fused kernels and
// by the unfused baseline's step kernel alike, so the two are bit-identical
// when the baseline keeps G in fp32 (paper, Corollary 1(a)).
//
// All arithmetic is IEEE fp32 with explicit fmaf (the library is compiled
// with -ffp-contract=off so no other contraction happens); the AdamW square
// root and reciprocal are the hardware instructions, the block-scale
// divisions are correctly rounded.

#include <type_traits>

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
constexpr int LDS_HALF = 3 * 2 * 32 * TILE * 2;  // 3-stage DMA ring = 49,152 bytes, >= 64 rows of G (33,792)
constexpr uint32_t GOLDEN = 0x9E3779B9u;

// ------------------------------------------------------------------------
// Rounding helpers (paper, Appendix C)
// ------------------------------------------------------------------------
// SR bits, 16 per element, from a counter-based hash.  The elements with
// flat indices (p K + q) 2j and 2j + 1 share the word
// h_j = fmix32(key ^ (j * 0x9E3779B9 mod 2^32)), fmix32 being MurmurHash3's
// 32-bit finaliser (Appleby, public domain: xor-shifts by 16, 13, 16 around
// multiplies by 0x85EBCA6B and 0xC2B2AE35); the even element takes its top
// half, the odd one its bottom half.  sr_pair(key, j * GOLDEN) is h_j.
__device__ __forceinline__ uint32_t sr_pair(uint32_t key, uint32_t jmul) {
  uint32_t h = key ^ jmul;
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// The SR bits of flat index idx in the top half of a word (the operand
// layout of the v_cvt_sr_* converters).
__device__ __forceinline__ uint32_t sr_elem_word(uint32_t key, uint32_t idx) {
  const uint32_t h = sr_pair(key, (idx >> 1) * GOLDEN);
  return (idx & 1u) ? h << 16 : h;
}

// fp32 -> bf16 on the gfx950 converters.  v_cvt_pk_bf16_f32 rounds two
// values to nearest even (a NaN becomes the quiet NaN with the same top
// bits).  v_cvt_sr_bf16_f32 adds the top 16 bits of its second operand to
// the 16 bits below the cut and truncates, which is the add-and-truncate
// stochastic rounding: the carry into the kept half happens with
// probability (x - x_lo)/ULP; infinities keep their pattern and NaN is made
// quiet, as in round to nearest.  Both instructions agree bit for bit with
// these definitions on every special pattern (zeros, subnormals, the
// largest finite values, infinities, quiet and signalling NaNs) against
// boundary random words and on 2 million random patterns.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) { return bf16x2_rne(x, 0.f) & 0xFFFFu; }

// a -> low half, b -> high half, with random words ra, rb.
__device__ __forceinline__ uint32_t bf16x2_sr(float a, float b, uint32_t ra, uint32_t rb) {
  bf16x2_t s = {};
  s = __builtin_amdgcn_cvt_sr_bf16_f32(s, a, ra, false);
  s = __builtin_amdgcn_cvt_sr_bf16_f32(s, b, rb, true);
  return __builtin_bit_cast(uint32_t, s);
}
__device__ __forceinline__ uint32_t bf16_sr_bits(float x, uint32_t key, uint32_t idx) {
  return bf16x2_sr(x, 0.f, sr_elem_word(key, idx), 0u) & 0xFFFFu;
}

// Two stored bf16 patterns (a low, b high) with random words ra, rb:
// stochastic rounding where srmask is all ones, round to nearest even where
// it is zero.  Both are formed and the mask selects, so the wave-uniform
// mode costs no branch.
__device__ __forceinline__ uint32_t bf16x2_select(float a, float b, uint32_t ra, uint32_t rb, uint32_t srmask) {
  const uint32_t s = bf16x2_sr(a, b, ra, rb);
  const uint32_t n = bf16x2_rne(a, b);
  return (s & srmask) | (n & ~srmask);
}

// The pair of elements 2j (a, low half) and 2j + 1 (b, high half) with one
// hash: jmul = j * GOLDEN.
__device__ __forceinline__ uint32_t bf16x2_store(float a, float b, uint32_t srmask, uint32_t key, uint32_t jmul) {
  const uint32_t h = sr_pair(key, jmul);
  return bf16x2_select(a, b, h, h << 16, srmask);
}

// How a bf16 store picks its rounding: RM_SEL from the wave-uniform mask at
// run time (both roundings formed, one kept), RM_SR / RM_RNE fixed at
// compile time (the fused kernels branch once per tile on the mask and run
// an epilogue specialised to it; the stored bits are the same).
constexpr int RM_SEL = 0, RM_SR = 1, RM_RNE = 2;

__device__ __forceinline__ float bf16_val(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------------------------------
// Tile order: row-major over the tile grid.  The tiles in flight across the
// whole chip then cover whole rows of W / m / v, which is what the HBM
// streams best (measured on MI355X with the state stream of a 14336 x 4096
// layer: giving every XCD its own contiguous block of tiles streams 8%
// slower, column-major order 22% slower).  Workgroups are dispatched
// round-robin to the 8 XCDs, so each XCD still sees every 8th tile of a few
// consecutive tile rows: its L2 holds the dY panels of those rows and, for
// a 4096-wide layer, an eighth of the X panels.
// ------------------------------------------------------------------------
__device__ __forceinline__ void tile_coords(int bid, int tiles_n, int tiles_k, int& ti, int& tj) {
  (void)tiles_n;
  ti = bid / tiles_k;
  tj = bid - ti * tiles_k;
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
// Mainloop, bf16 inputs, asynchronous: buffer loads straight into LDS
// (buffer_load_dwordx4 ... lds), S stages in flight, no register staging.
// A load instruction writes its 64 lanes' 16 bytes lane-linearly at a
// wave-uniform LDS address, so each lane fetches the global chunk that the
// swizzled layout expects at its slot.  Out-of-range offsets read as zero,
// which pads the token tail and a feature tail that is a multiple of 8.
// Requires 16-byte aligned rows (ld % 8 == 0), N % 8 == K % 8 == 0 and
// operands smaller than 4 GiB; other shapes use MainBF16.
// ------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): out-of-range offsets return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int STAGES>
struct MainBF16DmaT {
  static constexpr int TK = 32;                        // tokens per chunk
  static constexpr int S = STAGES;                     // LDS stages (S - 1 chunks in flight)
  static constexpr int OPB = TK * TILE * 2;            // 8 KiB per operand per stage
  static constexpr int STAGE = 2 * OPB;
  static constexpr int LOADS = 4;                      // buffer loads per thread per chunk

  __amdgpu_buffer_rsrc_t rA, rB;
  uint32_t oobA, oobB;         // an offset past the end: reads zero
  uint32_t baseA[2], baseB[2]; // byte offset of this lane's feature chunk in token row 0
  int trow[2];                 // token row within the chunk
  bool fokA[2], fokB[2];       // feature chunk inside the matrix
  int gwave;                   // wave index within the mainloop group

  // gtid: thread index within the 256 threads that run the mainloop
  __device__ __forceinline__ void init(const KArgs& a, int row0, int col0, int gtid) {
    const int lane = gtid & 63, wave = gtid >> 6;
    gwave = wave;
    oobA = (uint32_t)((uint64_t)a.BT * a.lddy * 2);
    oobB = (uint32_t)((uint64_t)a.BT * a.ldx * 2);
    rA = make_rsrc(a.dY, oobA);
    rB = make_rsrc(a.X, oobB);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = 4 * (2 * wave + r) + (lane >> 4);
      const int c = (lane & 15) ^ ((t & 3) << 2);        // logical 8-feature chunk at this slot
      trow[r] = t;
      fokA[r] = row0 + c * 8 < a.N;
      fokB[r] = col0 + c * 8 < a.K;
      baseA[r] = (uint32_t)(row0 + c * 8) * 2;
      baseB[r] = (uint32_t)(col0 + c * 8) * 2;
    }
  }

  __device__ __forceinline__ void issue(const KArgs& a, int kc, char* stage) const {
    const int wave = gwave;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int tok = kc * TK + trow[r];
      const bool tok_ok = tok < a.BT;
      const uint32_t oa = (tok_ok && fokA[r]) ? (uint32_t)tok * (uint32_t)(a.lddy * 2) + baseA[r] : oobA;
      const uint32_t ob = (tok_ok && fokB[r]) ? (uint32_t)tok * (uint32_t)(a.ldx * 2) + baseB[r] : oobB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(stage + (2 * wave + r) * 1024), 16, oa, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(stage + OPB + (2 * wave + r) * 1024), 16, ob, 0,
                                               0, 0);
    }
  }

  // Wait until this wave's loads of the chunk issued `ahead` chunks ago
  // have landed (later chunks may still be in flight).
  __device__ __forceinline__ static void wait_chunk(int ahead) {
    if (ahead >= 2) wait_vmcnt<2 * LOADS>();
    else if (ahead == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  }
};

using MainBF16Dma = MainBF16DmaT<4>;    // 64 KiB ring: two workgroups per CU
using MainBF16Dma3 = MainBF16DmaT<3>;   // 48 KiB ring: three workgroups per CU
static_assert(MainBF16Dma3::S * MainBF16Dma3::STAGE <= LDS_HALF && 64 * GP * 4 <= LDS_HALF &&
                  3 * LDS_HALF <= 160 * 1024,
              "three workgroups per CU: the ring and a 64-row half of G each fit, three fit in 160 KiB");
static_assert(2 * LDS_BYTES <= 160 * 1024, "two workgroups per CU");

// Transposing LDS read issued as inline assembly: the compiler cannot tell
// which stage an in-flight LDS DMA writes, and would otherwise wait for all
// of them (vmcnt(0)) before every LDS read.  Completion is awaited
// explicitly with lds_wait below.
__device__ __forceinline__ u32x2 tr_read(uint32_t lds_addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(lds_addr));
  return v;
}

// The same read at a VGPR address plus an immediate byte offset (the
// instruction's 16-bit offset field), so that reads at fixed distances share
// one address register.
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_at(uint32_t lds_addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "i"(OFF));
  return v;
}

__device__ __forceinline__ bf16x8 frag_join(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Wait for LDS reads until at most N are outstanding; the fragments are
// threaded through the statement so that their uses stay after it.
template <int N>
__device__ __forceinline__ void lds_wait(u32x2 (&f)[8]) {
  static_assert(N == 0 || N == 8, "lgkmcnt");
  if constexpr (N == 0)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                 "+v"(f[6]), "+v"(f[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                 "+v"(f[6]), "+v"(f[7]));
}

// Workgroup barrier without a memory fence: LDS-DMA completion is awaited
// per wave with wait_vmcnt before it (a fenced barrier would wait for every
// load in flight).  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Synchronisation of the waves that share an LDS ring: the workgroup barrier.
struct WorkgroupSync {
  __device__ __forceinline__ void arrive_wait() { bar(); }
};

// Phase 1 with the asynchronous mainloop, run by the 256 threads gtid =
// 0..255 of a group of 4 waves that share the LDS ring at `ring`.  Calls
// sync.arrive_wait() exactly max(nk, 0) times (once per token chunk), where
// nk = ceil(BT / 32).  The vmcnt waits count this wave's loads in issue
// order, so no other global load of these waves may be in flight.
template <class M, class Sync>
__device__ __forceinline__ void dma_accumulate(const KArgs& a, char* ring, int row0, int col0, int gtid,
                                               f32x16 (&acc)[2][2], Sync& sync) {
  static_assert(M::TK == 32, "two 16-token k-steps per chunk");
  const int lane = gtid & 63, wave = gtid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)ring;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  const int nk = (a.BT + M::TK - 1) / M::TK;
  // MFMA operand fragment of a 16-token k-step and a 32-feature block by two
  // transposing reads: lane l reads token rows t and t + 4 at features f ..
  // f + 3, t = 8 (l / 32) + (l % 16) / 4, f = 16 ((l / 16) % 2) + 4 (l % 4)
  // (8 consecutive tokens of one feature per lane after the transpose).
  // Byte offsets of this lane's reads within a stage, per block b:
  uint32_t fofsA[2], fofsB[2];
  {
    const int t = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int f = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      fofsA[b] = (uint32_t)MainBF16::off(t, wr * 64 + b * 32 + f);
      fofsB[b] = (uint32_t)(M::OPB + MainBF16::off(t, wc * 64 + b * 32 + f));
    }
  }
  M ml;
  ml.init(a, row0, col0, gtid);
#pragma unroll
  for (int k = 0; k < M::S - 1; ++k)
    if (k < nk) ml.issue(a, k, ring + k * M::STAGE);
  for (int kc = 0; kc < nk; ++kc) {
    // loads issued after chunk kc: chunks kc+1 .. min(kc+S-2, nk-1)
    M::wait_chunk(min(M::S - 2, nk - 1 - kc));
    sync.arrive_wait();   // chunk kc visible to all 4 waves; all of them done with chunk kc-1
    if (kc + M::S - 1 < nk) ml.issue(a, kc + M::S - 1, ring + ((kc + M::S - 1) % M::S) * M::STAGE);
    const uint32_t cur = lds0 + (uint32_t)((kc % M::S) * M::STAGE);
    // operand fragments of the chunk's two k-steps: [A0 lo, A0 hi, A1 lo, A1 hi, B0 lo, B0 hi, B1 lo, B1 hi]
    // (the hi half is 4 token rows = 1024 bytes on, the second k-step 16
    // rows = 4096 bytes on, the swizzle unchanged)
    u32x2 f0[8], f1[8];
    uint32_t pa[2], pb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      pa[b] = cur + fofsA[b];
      pb[b] = cur + fofsB[b];
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f0[2 * b] = tr_read_at<0>(pa[b]);
      f0[2 * b + 1] = tr_read_at<1024>(pa[b]);
      f0[4 + 2 * b] = tr_read_at<0>(pb[b]);
      f0[4 + 2 * b + 1] = tr_read_at<1024>(pb[b]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f1[2 * b] = tr_read_at<4096>(pa[b]);
      f1[2 * b + 1] = tr_read_at<5120>(pa[b]);
      f1[4 + 2 * b] = tr_read_at<4096>(pb[b]);
      f1[4 + 2 * b + 1] = tr_read_at<5120>(pb[b]);
    }
    lds_wait<8>(f0);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_join(f0[2 * bi], f0[2 * bi + 1]),
                                                              frag_join(f0[4 + 2 * bj], f0[4 + 2 * bj + 1]),
                                                              acc[bi][bj], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // the wait below stays after these MFMAs
    lds_wait<0>(f1);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_join(f1[2 * bi], f1[2 * bi + 1]),
                                                              frag_join(f1[4 + 2 * bj], f1[4 + 2 * bj + 1]),
                                                              acc[bi][bj], 0, 0, 0);
  }
  wait_vmcnt<0>();
}

// Accumulator layout of v_mfma_f32_32x32x*: lane l, register 4j+i of block
// (bi, bj) holds row 8j + 4(l/32) + i, column l%32 of that 32 x 32 block.
__device__ __forceinline__ void store_acc(float* sG, const f32x16 (&acc)[2][2], int gtid) {
  const int lane = gtid & 63, wave = gtid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
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
}

// Rows 64h .. 64h + 63 of the tile, held by the waves with wr = h, into rows
// 0..63 of sG (called by those two waves only).
__device__ __forceinline__ void store_acc_half(float* sG, const f32x16 (&acc)[2][2], int gtid) {
  const int lane = gtid & 63, wc = (gtid >> 6) & 1;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int c = wc * 64 + bj * 32 + (lane & 31);
        sG[r * GP + c] = acc[bi][bj][e];
      }
}

// Phase 1 for a 256-thread workgroup; same output as tile_gradient.
__device__ __forceinline__ void tile_gradient_dma(const KArgs& a, char* lds, int row0, int col0) {
  static_assert(MainBF16Dma::S * MainBF16Dma::STAGE <= LDS_BYTES, "LDS budget");
  f32x16 acc[2][2];
  WorkgroupSync sync;
  dma_accumulate<MainBF16Dma>(a, lds, row0, col0, threadIdx.x, acc, sync);
  bar();   // every wave is done reading the stages before G overwrites them
  store_acc(reinterpret_cast<float*>(lds), acc, threadIdx.x);
  __syncthreads();
}

// ------------------------------------------------------------------------
// Wide mainloop for long token axes: a 256 x 256 macro tile per workgroup.
// Per token the workgroup fetches 1 KiB of dY and X for 128 Ki MFMA flops,
// half the bytes per flop of the 128 x 128 tile, which matters once BT is
// long enough that the activation panels no longer stay in L2.  Same
// asynchronous LDS-DMA ring (4 stages of 32 tokens, 512-byte rows
// XOR-swizzled in 64-byte units) and transposing reads as MainBF16Dma; NW
// waves share the ring, each issuing its share of a chunk's 32 1-KiB loads.
// ------------------------------------------------------------------------
template <int NW>                                       // waves sharing the ring
struct MainWideT {
  static constexpr int TK = 32;
  static constexpr int S = 4;
  static constexpr int W = 256;                         // macro tile edge
  static constexpr int ROWB = W * 2;                    // bytes per token row
  static constexpr int OPB = TK * ROWB;                 // 16 KiB per operand per stage
  static constexpr int STAGE = 2 * OPB;                 // 32 KiB
  static constexpr int ROUNDS = OPB / (NW * 64 * 16);   // load rounds per operand per chunk (8 waves: 2)
  static constexpr int LOADS = 2 * ROUNDS;              // buffer loads per thread per chunk

  __amdgpu_buffer_rsrc_t rA, rB;
  uint32_t oobA, oobB;
  uint32_t baseA[ROUNDS], baseB[ROUNDS];
  int trow[ROUNDS];
  bool fokA[ROUNDS], fokB[ROUNDS];
  int wave;

  __device__ __forceinline__ static int off(int t, int f) { return t * ROWB + ((f * 2) ^ ((t & 3) << 6)); }

  __device__ __forceinline__ void init(const KArgs& a, int row0, int col0) {
    const int lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    oobA = (uint32_t)((uint64_t)a.BT * a.lddy * 2);
    oobB = (uint32_t)((uint64_t)a.BT * a.ldx * 2);
    rA = make_rsrc(a.dY, oobA);
    rB = make_rsrc(a.X, oobB);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      // instruction (wave, r) fills bytes [(NW r + wave) KiB, +1 KiB) of the operand region: 2 token rows
      const int t = 2 * (NW * r + wave) + (lane >> 5);
      const int c = (lane & 31) ^ ((t & 3) << 2);        // logical 8-feature chunk at this slot
      trow[r] = t;
      fokA[r] = row0 + c * 8 < a.N;
      fokB[r] = col0 + c * 8 < a.K;
      baseA[r] = (uint32_t)(row0 + c * 8) * 2;
      baseB[r] = (uint32_t)(col0 + c * 8) * 2;
    }
  }

  // Load J of this wave's share of chunk kc (round J / 2, operand J % 2).
  // Tokens past BT (including whole chunks past the end) read as zeros.
  template <int J>
  __device__ __forceinline__ void issue_one(const KArgs& a, int kc, char* stage) const {
    constexpr int r = J >> 1;
    const int tok = kc * TK + trow[r];
    const bool tok_ok = tok < a.BT;
    if constexpr ((J & 1) == 0) {
      const uint32_t oa = (tok_ok && fokA[r]) ? (uint32_t)tok * (uint32_t)(a.lddy * 2) + baseA[r] : oobA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(stage + (NW * r + wave) * 1024), 16, oa, 0, 0, 0);
    } else {
      const uint32_t ob = (tok_ok && fokB[r]) ? (uint32_t)tok * (uint32_t)(a.ldx * 2) + baseB[r] : oobB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(stage + OPB + (NW * r + wave) * 1024), 16, ob, 0, 0,
                                               0);
    }
  }

  __device__ __forceinline__ void issue(const KArgs& a, int kc, char* stage) const {
    issue_seq(a, kc, stage, std::make_integer_sequence<int, LOADS>{});
  }
  template <int... J>
  __device__ __forceinline__ void issue_seq(const KArgs& a, int kc, char* stage, std::integer_sequence<int, J...>) const {
    (issue_one<J>(a, kc, stage), ...);
  }
};

// ------------------------------------------------------------------------
// The wide mainloop's waves: 8 in a 2 x 4 arrangement of 128 x 64 parts (8
// accumulator blocks, 128 registers per wave), so two waves share each SIMD
// and one's LDS-read, load-issue and barrier stalls overlap the other's
// MFMAs (measured 9% faster at BT = 8192 than 4 waves holding 128 x 128
// each, one per SIMD).  Per 16-token k-step a wave runs 8 MFMAs and reads
// 12 fragments of the next k-step (4 dY blocks, 2 X blocks, two halves
// each), the reads and its 4 loads per chunk interleaved with the MFMAs and
// pinned by a scheduling barrier, so LDS latency and the address unit's
// queue drain behind the matrix pipe instead of stalling the wave's in-order
// issue.  The k-steps run in token order, so every element of G sees the
// MFMA sequence of the other mainloops.
// ------------------------------------------------------------------------
using MainWide = MainWideT<8>;

// Fragment registers of a k-step: 0..7 dY blocks (r / 2, half r % 2),
// 8..11 X blocks ((r - 8) / 2, half r % 2); adr[0..3] dY blocks, adr[4..5]
// X blocks at token 0 of the stage.  MFMA slot I reads fragment I and, when
// I is even, fragment 8 + I / 2; when DMA and I is even it issues load I / 2.
template <bool READ, bool DMA, int T0, int I>
__device__ __forceinline__ void wide_one(f32x16 (&acc)[4][2], const u32x2 (&cur)[12], u32x2 (&nxt)[12],
                                       const uint32_t (&adr)[6], const MainWide& ml, const KArgs& a, int kdma,
                                       char* dstage) {
  constexpr int bi = I >> 1, bj = I & 1;
  acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_join(cur[2 * bi], cur[2 * bi + 1]),
                                                        frag_join(cur[8 + 2 * bj], cur[8 + 2 * bj + 1]),
                                                        acc[bi][bj], 0, 0, 0);
  if constexpr (READ) {
    nxt[I] = tr_read_at<(T0 + 4 * (I & 1)) * MainWide::ROWB>(adr[I >> 1]);
    if constexpr ((I & 1) == 0) {
      constexpr int R = 8 + I / 2;
      nxt[R] = tr_read_at<(T0 + 4 * (R & 1)) * MainWide::ROWB>(adr[4 + ((R - 8) >> 1)]);
    }
  }
  if constexpr (DMA && (I & 1) == 0) ml.template issue_one<I / 2>(a, kdma, dstage);
  __builtin_amdgcn_sched_barrier(0);
}

template <bool READ, bool DMA, int T0, int... I>
__device__ __forceinline__ void wide_kstep_seq(f32x16 (&acc)[4][2], const u32x2 (&cur)[12], u32x2 (&nxt)[12],
                                             const uint32_t (&adr)[6], const MainWide& ml, const KArgs& a, int kdma,
                                             char* dstage, std::integer_sequence<int, I...>) {
  (wide_one<READ, DMA, T0, I>(acc, cur, nxt, adr, ml, a, kdma, dstage), ...);
}

template <bool READ, bool DMA, int T0>
__device__ __forceinline__ void wide_kstep(f32x16 (&acc)[4][2], const u32x2 (&cur)[12], u32x2 (&nxt)[12],
                                         const uint32_t (&adr)[6], const MainWide& ml, const KArgs& a, int kdma,
                                         char* dstage) {
  static_assert(MainWide::LOADS == 4, "one load per even MFMA slot");
  wide_kstep_seq<READ, DMA, T0>(acc, cur, nxt, adr, ml, a, kdma, dstage, std::make_integer_sequence<int, 8>{});
}

__device__ __forceinline__ void lds_wait12(u32x2 (&f)[12]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]), "+v"(f[7]),
                 "+v"(f[8]), "+v"(f[9]), "+v"(f[10]), "+v"(f[11]));
}

// Accumulate the wave's 128 x 64 part of the macro tile at (row0, col0).
// Software pipeline: the fragments of each k-step are read while the
// previous k-step's MFMAs run.  The one barrier per chunk sits between the
// chunk's two k-steps: by then every wave has finished reading the chunk, so
// its stage is refilled with the chunk S ahead, and the next chunk has
// landed, so its first k-step can be read during the second k-step here.
// Loads past the last chunk zero-fill a stage never read again, so every
// vmcnt wait is a constant.
__device__ __forceinline__ void wide_accumulate(const KArgs& a, char* ring, int row0, int col0,
                                                 f32x16 (&acc)[4][2]) {
  using M = MainWide;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 2, wc = wave & 3;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)ring;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  const int nk = (a.BT + M::TK - 1) / M::TK;
  if (nk == 0) return;
  M ml;
  ml.init(a, row0, col0);
  uint32_t off[6];
  {
    const int tl = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int fl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < 4; ++b) off[b] = (uint32_t)M::off(tl, wr * 128 + b * 32 + fl);
#pragma unroll
    for (int b = 0; b < 2; ++b) off[4 + b] = (uint32_t)(M::OPB + M::off(tl, wc * 64 + b * 32 + fl));
  }
  static_assert(M::S == 4, "the waits below assume 4 stages");
#pragma unroll
  for (int k = 0; k < M::S; ++k) ml.issue(a, k, ring + k * M::STAGE);
  wait_vmcnt<3 * M::LOADS>();   // chunk 0
  bar();
  u32x2 f0[12], f1[12];
  uint32_t adr[6];
#pragma unroll
  for (int r = 0; r < 6; ++r) adr[r] = lds0 + off[r];
#pragma unroll
  for (int r = 0; r < 12; ++r)
    f0[r] = tr_read(adr[r < 8 ? (r >> 1) : 4 + ((r - 8) >> 1)] + (uint32_t)(4 * (r & 1) * M::ROWB));
  lds_wait12(f0);
  for (int kc = 0; kc < nk; ++kc) {
    wide_kstep<true, false, 16>(acc, f0, f1, adr, ml, a, 0, ring);   // k-step 0 of chunk kc; read k-step 1
    lds_wait12(f1);
    wait_vmcnt<2 * M::LOADS>();   // chunk kc + 1
    bar();                        // all waves done with stage kc % S; chunk kc + 1 visible
    const uint32_t st = lds0 + (uint32_t)(((kc + 1) % M::S) * M::STAGE);
#pragma unroll
    for (int r = 0; r < 6; ++r) adr[r] = st + off[r];
    // k-step 1 of chunk kc; read k-step 0 of chunk kc + 1; refill stage kc % S with chunk kc + S
    wide_kstep<true, true, 0>(acc, f1, f0, adr, ml, a, kc + M::S, ring + (kc % M::S) * M::STAGE);
    lds_wait12(f0);
  }
  wait_vmcnt<0>();
}

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
// Element-wise step (Algorithm 1 Phase 2 and 3; Appendix N families)
//
// Epilogue thread mapping: in pass s (0..7) thread t owns row
// s*16 + t/16 of the tile and two 4-element segments of it, at columns
// 4*(t%16) and 64 + 4*(t%16).  The 16 lanes of a row therefore access one
// contiguous 64-element run per instruction (whole 128-byte lines for
// every format but int8), and a row's 128 columns stay within 16 lanes for
// the int8 block reduction.
// ------------------------------------------------------------------------
// Raw (undecoded) storage of 4 consecutive elements, so that the loads of
// later passes can be in flight while earlier ones are computed.
// OCP FP8 E4M3 ("fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// largest finite 448, no infinities, S.1111.111 is NaN), converted with
// gfx950's FP8 instructions, which take and produce this format.  Encoding
// rounds to nearest, ties to even (the mode register's default); inputs are
// first clamped to +-448, so values beyond the largest finite saturate
// instead of becoming NaN.  The sign of a zero result follows the input.
// Both directions are exact functions of their inputs.
__device__ __forceinline__ uint32_t e4m3_pack4(float y0, float y1, float y2, float y3) {
  const auto sat = [](float y) { return fminf(fmaxf(y, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(y0), sat(y1), 0, false);   // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(y2), sat(y3), w, true);        // bytes 2, 3
  return (uint32_t)w;
}

// Stochastic rounding onto the E4M3 grid (the FP8 weight store): |y| goes
// to one of its two neighbouring grid values, away from zero with
// probability equal to its fractional position between them (quantised to
// 2^-16), saturating at 448 and keeping the sign.  In the normal range
// (|y| >= 2^-6, 3 fraction bits) this adds r16 * 2^4 to the 20 fp32 fraction
// bits E4M3 drops and clears them; in the subnormal range (spacing 2^-9) the
// value is ((floor(|y| 2^25) + r16) >> 16) 2^-9.  gfx950's v_cvt_sr_fp8_f32
// computes exactly this when its input is clamped to +-448 and its random
// word carries r16 in the top half with the low half clear (it adds the top
// 20 bits of the word); forge_debug_e4m3_sr exposes the function for a
// bit-for-bit comparison with the definition.  r[i]: words whose top 16 bits
// are the SR bits of element i.
__device__ __forceinline__ uint32_t e4m3_sr_pack4(const float (&y)[4], const uint32_t (&r)[4]) {
  const auto sat = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
  int w = 0;
  w = __builtin_amdgcn_cvt_sr_fp8_f32(sat(y[0]), (int)(r[0] & 0xFFFF0000u), w, 0);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(sat(y[1]), (int)(r[1] & 0xFFFF0000u), w, 1);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(sat(y[2]), (int)(r[2] & 0xFFFF0000u), w, 2);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(sat(y[3]), (int)(r[3] & 0xFFFF0000u), w, 3);
  return (uint32_t)w;
}

// Block scale a / QMAX and reciprocal QMAX / a, a > 0, as correctly rounded
// fp32 quotients.  For 2^-64 <= a < 2^126 short fma sequences give them
// (Markstein's residual correction): a / Q = q0 + fma(-Q, q0, a) / Q with
// q0 = a * fp32(1/Q); Q / a from the hardware reciprocal refined by one
// Newton step y, then q0 = Q * y and q0 + fma(-a, q0, Q) * y.  Both equal
// IEEE division for every fp32 a in that range and each QMAX used (127,
// 255, 448; checked exhaustively by forge_debug_quotients).  Outside it the
// caller divides with IEEE division.
__device__ __forceinline__ float quot_by_q(float a, float q, float rq) {
  const float q0 = a * rq;
  return fmaf(fmaf(-q, q0, a), rq, q0);
}
__device__ __forceinline__ float q_by_quot(float q, float a) {
  float y = __builtin_amdgcn_rcpf(a);
  y = fmaf(fmaf(-a, y, 1.f), y, y);
  const float q0 = q * y;
  return fmaf(fmaf(-a, q0, q), y, q0);
}
__device__ __forceinline__ bool quot_fast_range(float a) { return a >= 0x1p-64f && a < 0x1p126f; }

__device__ __forceinline__ void e4m3_unpack4(uint32_t w, float* x) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);        // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);         // bytes 2, 3
  x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
}

// Unsigned max across the lanes of one 16-lane DPP row.  CTRL selects the
// partner: 0xB1 quad_perm [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1]
// (lane ^ 2), 0x141 row_half_mirror (lane i <-> 7 - i: the other quad of
// its 8 lanes), 0x140 row_mirror (lane i <-> 15 - i: the other half of the
// row).  Every partner lies in the same row, so all lanes must be active.
// Applied to the bit patterns of non-negative floats, unsigned max is the
// float max, exact and independent of the reduction order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t x) {
  return max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t lanes8_max(uint32_t x) {   // over aligned groups of 8 lanes
  return dpp_umax<0x141>(dpp_umax<0x4E>(dpp_umax<0xB1>(x)));
}
__device__ __forceinline__ uint32_t lanes16_max(uint32_t x) {  // over each 16-lane row
  return dpp_umax<0x140>(lanes8_max(x));
}

template <int FMT> struct Raw4;
template <> struct Raw4<FMT_F32> { f32x4 v; };
template <> struct Raw4<FMT_BF16> { u32x2 v; };
template <> struct Raw4<FMT_S8> { uint32_t v; float s; };
template <> struct Raw4<FMT_U8> { uint32_t v; float s; };
template <> struct Raw4<FMT_E4M3> { uint32_t v; float s; };
template <> struct Raw4<FMT_NONE> {};

// State tensors are streamed once per step: their accesses are marked
// non-temporal so that they do not evict the activation panels the
// neighbouring tiles re-read from L2.
template <typename T> __device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}
template <typename T> __device__ __forceinline__ void st_nt(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

// Element offsets of one thread's segment in the current pass.
//  FAST: rows allow aligned 4-element vector accesses and K % 4 == 0, so a
//        segment is either entirely inside the matrix or entirely outside;
//        only `ok` is consulted.
//  otherwise: `nv` (0..4) elements are inside; accesses are element-wise
//        unless `vec` and nv == 4.
struct Seg {
  bool ok;      // row < N and at least one column inside
  int nv;       // valid elements (<= 4)
  int q;        // first column
};

// seg: the segment's first element.
template <int FMT, bool FAST>
__device__ __forceinline__ void ld4(Raw4<FMT>& r, const void* seg, const Seg& g, bool vec) {
  if constexpr (FMT == FMT_F32) {
    const float* p = static_cast<const float*>(seg);
    if (FAST || (vec && g.nv == 4)) {
      r.v = ld_nt<f32x4>(p);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[i] = i < g.nv ? p[i] : 0.f;
    }
  } else if constexpr (FMT == FMT_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(seg);
    if (FAST || (vec && g.nv == 4)) {
      r.v = ld_nt<u32x2>(p);
    } else {
      uint32_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = i < g.nv ? (uint32_t)p[i] : 0u;
      r.v = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    }
  } else if constexpr (fmt_blocked(FMT)) {
    const uint8_t* p = static_cast<const uint8_t*>(seg);
    if (FAST || (vec && g.nv == 4)) {
      r.v = ld_nt<uint32_t>(p);
    } else {
      uint32_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = i < g.nv ? (uint32_t)p[i] : 0u;
      r.v = e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24);
    }
  }
}

template <int FMT>
__device__ __forceinline__ void zero4(Raw4<FMT>& r) {
  if constexpr (FMT == FMT_F32) r.v = f32x4{0.f, 0.f, 0.f, 0.f};
  else if constexpr (FMT == FMT_BF16) r.v = u32x2{0u, 0u};
  else if constexpr (fmt_blocked(FMT)) { r.v = 0u; r.s = 0.f; }
}

// Decode to fp32; int8 codes are dequantised as code * scale (one fp32 multiply).
template <int FMT>
__device__ __forceinline__ void dec4(const Raw4<FMT>& r, float* x) {
  if constexpr (FMT == FMT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = r.v[i];
  } else if constexpr (FMT == FMT_BF16) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      x[2 * i] = __uint_as_float(r.v[i] << 16);
      x[2 * i + 1] = __uint_as_float(r.v[i] & 0xFFFF0000u);
    }
  } else if constexpr (FMT == FMT_S8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)(int8_t)((r.v >> (8 * i)) & 0xFFu) * r.s;
  } else if constexpr (FMT == FMT_U8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)((r.v >> (8 * i)) & 0xFFu) * r.s;
  } else if constexpr (FMT == FMT_E4M3) {
    e4m3_unpack4(r.v, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= r.s;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 0.f;
  }
}

// The codes of a block-scaled state as fp32 values, without the scale:
// callers whose only use of the decoded state x is a product c * x fold the
// scale into c (one multiply per segment instead of one per element).
template <int FMT>
__device__ __forceinline__ void dec4_codes(const Raw4<FMT>& r, float* x) {
  static_assert(fmt_blocked(FMT), "block-scaled formats only");
  if constexpr (FMT == FMT_S8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)(int8_t)((r.v >> (8 * i)) & 0xFFu);
  } else if constexpr (FMT == FMT_U8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)((r.v >> (8 * i)) & 0xFFu);
  } else {
    e4m3_unpack4(r.v, x);
  }
}

// Store 4 fp32 values as FMT at seg, the segment's first element (int8
// formats go through quantize_chunk instead).
// bf16: stochastic rounding when sr is all ones (idx = flat index of the
// first element), round to nearest even when it is zero.  FAST segments
// start at an even flat index (K % 4 == 0), so they are two hash pairs.
template <int FMT, bool FAST, int RM = RM_SEL>
__device__ __forceinline__ void st4(void* seg, const Seg& g, bool vec, const float* x, uint32_t sr, uint32_t key,
                                    uint32_t idx) {
  if constexpr (FMT == FMT_F32) {
    float* p = static_cast<float*>(seg);
    if (FAST || (vec && g.nv == 4)) {
      st_nt<f32x4>(p, f32x4{x[0], x[1], x[2], x[3]});
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < g.nv) p[i] = x[i];
    }
  } else if constexpr (FMT == FMT_BF16) {
    uint32_t lo, hi;
    if constexpr (RM == RM_RNE) {
      lo = bf16x2_rne(x[0], x[1]);
      hi = bf16x2_rne(x[2], x[3]);
    } else if constexpr (RM == RM_SR && FAST) {
      const uint32_t jmul = (idx >> 1) * GOLDEN;
      const uint32_t h0 = sr_pair(key, jmul), h1 = sr_pair(key, jmul + GOLDEN);
      lo = bf16x2_sr(x[0], x[1], h0, h0 << 16);
      hi = bf16x2_sr(x[2], x[3], h1, h1 << 16);
    } else if constexpr (RM == RM_SR) {
      lo = bf16x2_sr(x[0], x[1], sr_elem_word(key, idx), sr_elem_word(key, idx + 1u));
      hi = bf16x2_sr(x[2], x[3], sr_elem_word(key, idx + 2u), sr_elem_word(key, idx + 3u));
    } else if constexpr (FAST) {
      const uint32_t jmul = (idx >> 1) * GOLDEN;
      lo = bf16x2_store(x[0], x[1], sr, key, jmul);
      hi = bf16x2_store(x[2], x[3], sr, key, jmul + GOLDEN);
    } else {
      lo = bf16x2_select(x[0], x[1], sr_elem_word(key, idx), sr_elem_word(key, idx + 1u), sr);
      hi = bf16x2_select(x[2], x[3], sr_elem_word(key, idx + 2u), sr_elem_word(key, idx + 3u), sr);
    }
    uint16_t* p = static_cast<uint16_t*>(seg);
    if (FAST || (vec && g.nv == 4)) {
      st_nt<u32x2>(p, u32x2{lo, hi});
    } else {
      const uint32_t b[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < g.nv) p[i] = (uint16_t)b[i];
    }
  }
}

// Block-absmax quantisation of a chunk (two 4-element segments 64 columns
// apart) to 8-bit codes with one fp32 scale per block.  codes[g]: segment
// g's first code; scales[g]: the scale of the block segment g lies in.  block == 128: one
// block spans both segments of the 16 lanes of a row; block 64 / 32: each
// segment lies in its own block, shared by 16 / 8 adjacent lanes.  Every
// lane of the wave must call this (DPP reductions).  8-bit states need
// K % block == 0, so a segment is either entirely inside or outside.
//  FMT_S8   (first moment): codes -127..127, scale a/127.
//  FMT_U8   (second moment): code 0 only for an exact zero, else 1..255,
//           scale a/255.
//  FMT_E4M3 (either): scale a/448, code = the E4M3 value nearest to
//           x * (448/a); with POSITIVE (the second moment) a positive value
//           never becomes code 0 but the smallest subnormal 2^-9, which is
//           what rounding max(y, 2^-9) gives for every positive y.
// a is the block absmax; the scale and the reciprocal are correctly rounded
// fp32 quotients (quot_by_q / q_by_quot, IEEE division outside their
// range).  A block whose absmax is below 2^-64 (a long-decayed moment)
// would overflow QMAX / a; there the values and the reciprocal are taken
// 2^64 times larger and smaller (exact scalings), which gives the product
// x * (QMAX / a) as if the exponent range were unbounded -- the same bits as
// the plain product wherever that one is finite.
// With |x| <= a the scaled value y = x * (QMAX / a) stays below
// QMAX (1 + 2^-23), so rint(y) never leaves -127..127 (S8) or 0..255 (U8):
// S8 needs no clamp, and U8 codes come from v_cvt_pk_u8_f32, which rounds
// to nearest even, clamps to 0..255 and inserts the byte.
// SRW (the E4M3 weight store): when sr is nonzero the codes are drawn by
// e4m3_sr_pack4 with the SR bits of flat indices idx[g] + i (key `key`),
// else they are the nearest ones.
template <int FMT, bool POSITIVE, bool SRW = false>
__device__ __forceinline__ void quantize_chunk(const float (&x_in)[8], int block, const Seg (&sg)[2],
                                               uint8_t* const (&codes)[2], bool vec, float* const (&scales)[2],
                                               uint32_t sr = 0, uint32_t key = 0,
                                               const uint32_t* idx = nullptr) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x_in[i];
  constexpr float QMAX = FMT == FMT_S8 ? 127.f : FMT == FMT_U8 ? 255.f : 448.f;
  constexpr float RQ = 1.f / QMAX;
  // absmax as the unsigned max of |x| bit patterns (for non-negative floats
  // the same order); the second moment is never negative, so with POSITIVE
  // the patterns are compared as they are
  uint32_t ab[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, POSITIVE ? __float_as_uint(x[4 * g + i]) : __float_as_uint(x[4 * g + i]) & 0x7FFFFFFFu);
    ab[g] = sg[g].ok ? m : 0u;
  }
  if (block == 128) {
    ab[0] = ab[1] = lanes16_max(max(ab[0], ab[1]));
  } else if (block == 64) {
    ab[0] = lanes16_max(ab[0]);
    ab[1] = lanes16_max(ab[1]);
  } else {
    ab[0] = lanes8_max(ab[0]);
    ab[1] = lanes8_max(ab[1]);
  }
  const float a[2] = {__uint_as_float(ab[0]), __uint_as_float(ab[1])};
  float sc[2], inv[2];
  sc[0] = quot_by_q(a[0], QMAX, RQ);                    // 0 for a = 0
  inv[0] = a[0] > 0.f ? q_by_quot(QMAX, a[0]) : 0.f;
  if (block == 128) {
    sc[1] = sc[0];
    inv[1] = inv[0];
  } else {
    sc[1] = quot_by_q(a[1], QMAX, RQ);
    inv[1] = a[1] > 0.f ? q_by_quot(QMAX, a[1]) : 0.f;
  }
  const bool rare0 = a[0] != 0.f && !quot_fast_range(a[0]), rare1 = a[1] != 0.f && !quot_fast_range(a[1]);
  if (rare0 || rare1) {   // rare; skipped by the whole wave when no lane needs it
    const bool rare[2] = {rare0, rare1};
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (!rare[g]) continue;
      sc[g] = a[g] > 0.f ? a[g] / QMAX : 0.f;
      if (a[g] > 0.f && a[g] < 0x1p-64f) {
        inv[g] = QMAX / (a[g] * 0x1p64f);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * g + i] *= 0x1p64f;
      } else {
        inv[g] = a[g] > 0.f ? QMAX / a[g] : 0.f;
      }
    }
  }
  const int lpb = block == 32 ? 8 : 16;
  const bool writer = (threadIdx.x & (lpb - 1)) == 0;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint32_t word = 0;
    if constexpr (FMT == FMT_E4M3) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xv = x[4 * g + i];
        y[i] = xv * inv[g];
        if (POSITIVE) y[i] = xv > 0.f ? fmaxf(y[i], 0x1p-9f) : y[i];
      }
      if constexpr (SRW) {
        if (sr) {   // wave-uniform
          // idx[g] is even (K % block == 0): the segment is two hash pairs
          const uint32_t jmul = (idx[g] >> 1) * GOLDEN;
          const uint32_t h0 = sr_pair(key, jmul), h1 = sr_pair(key, jmul + GOLDEN);
          const uint32_t r[4] = {h0, h0 << 16, h1, h1 << 16};
          word = e4m3_sr_pack4(y, r);
        } else {
          word = e4m3_pack4(y[0], y[1], y[2], y[3]);
        }
      } else {
        word = e4m3_pack4(y[0], y[1], y[2], y[3]);
      }
    } else if constexpr (FMT == FMT_S8) {
      // rint(y) from one fp32 addition: with |y| < 2^22 the sum y + 1.5 * 2^23
      // is y rounded to an integer k, to nearest with ties to even (a unit
      // in the last place of the sum is 1, and the sum's last mantissa bit is
      // k's), and the sum's low byte is k in two's complement.  Two byte
      // permutes and an or pack the four codes.
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(x[4 * g + i] * inv[g] + 0x1.8p23f);
      word = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
    } else {   // U8: code 0 only for an exact zero, a positive value at least 1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xv = x[4 * g + i];
        const float y = xv != 0.f ? fmaxf(xv * inv[g], 1.f) : 0.f;
        word = __builtin_amdgcn_cvt_pk_u8_f32(y, i, word);
      }
    }
    if (!sg[g].ok) continue;
    if (writer && (block != 128 || g == 0)) *scales[g] = sc[g];
    uint8_t* p = codes[g];
    if (vec) {
      st_nt<uint32_t>(p, word);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = (uint8_t)((word >> (8 * i)) & 0xFFu);
    }
  }
}

// Addressing of the elements a thread steps in one tile.  Every stream has
// a tile base (its row row0, column col0) and a step per pass (RPP rows),
// both uniform over the workgroup and so held in scalar registers, and the
// thread one byte offset from the tile base (its row tid / 16, column
// 4 (tid % 16)); the second segment sits 64 columns further, a constant
// (scales: s1 bytes further).  A state access is then a scalar base plus the
// pass step (added on the scalar unit) plus the thread's offset, which the
// FAST kernels keep in 32 bits (the host routes rows of 2^26 bytes or more to
// the other kernels): one 64-bit add of a scalar and a zero-extended vector
// register per access, no per-pass vector multiplies.  The flat SR index
// (p K + q) likewise advances by a uniform step per pass.
template <bool FAST>
struct TileRows {
  using Off = std::conditional_t<FAST, uint32_t, uint64_t>;
  char* w;                 // W, m, v, and the G source (dW / accumulator) at (row0, col0)
  char* m;
  char* v;
  const char* g;
  char* ms;                // block scales at (row0, col0 / block)
  char* vs;
  char* ws;                // the weight's block scales (E4M3 weight)
  int64_t dw, dm, dv, dg;  // bytes from one pass's rows to the next
  int64_t ds;              // scale bytes from one pass's rows to the next
  int64_t s1;              // scale bytes from segment 0's block to segment 1's
  Off ow, om, ov, og, os;  // this thread's byte offsets from the tile bases
  uint32_t idx;            // p0 K (mod 2^32): the flat index of the thread's row in pass 0
  uint32_t didx;           // RPP K
  uint32_t qg[2];          // q of the thread's two segments
};

// base + pass + off + extra, with base + pass uniform and off the thread's
// offset: the shape the loads and stores take as scalar base plus vector
// offset (plus the immediate offset field for a constant extra).
template <class O>
__device__ __forceinline__ char* at(char* base, int64_t pass, O off, int64_t extra) {
  return (base + pass) + (uint64_t)off + extra;
}
template <class O>
__device__ __forceinline__ const char* at(const char* base, int64_t pass, O off, int64_t extra) {
  return (base + pass) + (uint64_t)off + extra;
}

// BLK: the 8-bit block size when fixed at compile time (0: a.block at run time).
template <int OPT, int WF, int MF, int VF, bool FAST, int BLK = 0>
struct Step {
  static_assert(BLK == 0 || BLK == 32 || BLK == 64 || BLK == 128, "block of 32, 64 or 128");
  static constexpr int FIXED_BLOCK = BLK;
  static constexpr bool HAS_M = opt_has_m(OPT);
  static constexpr bool HAS_V = opt_has_v(OPT);
  static constexpr int WFMT = WF;
  static constexpr int MFMT = HAS_M ? MF : FMT_NONE;
  static constexpr int VFMT = HAS_V ? VF : FMT_NONE;
  // bf16 weight and bf16 moments: the stores whose rounding is worth fixing
  // per tile (elsewhere the second epilogue copy costs registers: spills)
  static constexpr bool BF16_STORE = WFMT == FMT_BF16 && (MFMT == FMT_BF16 || VFMT == FMT_BF16);

  // Everything one chunk reads, still undecoded.
  struct Pending {
    Raw4<WF> w[2];
    Raw4<MFMT> m[2];
    Raw4<VFMT> v[2];
  };

  static constexpr int esz(int fmt) { return fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 2 : 1; }

  __device__ __forceinline__ static void load(const KArgs& a, const TileRows<FAST>& tr, int s, const Seg (&sg)[2],
                                              Pending& r) {
    const bool vec = a.vec_state != 0;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (!sg[g].ok) {
        zero4(r.w[g]); zero4(r.m[g]); zero4(r.v[g]);
        continue;
      }
      ld4<WF, FAST>(r.w[g], at(tr.w, s * tr.dw, tr.ow, 64 * g * esz(WF)), sg[g], vec);
      if constexpr (fmt_blocked(WF))
        r.w[g].s = *reinterpret_cast<const float*>(at(tr.ws, s * tr.ds, tr.os, g * tr.s1));
      if constexpr (HAS_M) {
        ld4<MF, FAST>(r.m[g], at(tr.m, s * tr.dm, tr.om, 64 * g * esz(MF)), sg[g], vec);
        if constexpr (fmt_blocked(MF))
          r.m[g].s = *reinterpret_cast<const float*>(at(tr.ms, s * tr.ds, tr.os, g * tr.s1));
      }
      if constexpr (HAS_V) {
        ld4<VF, FAST>(r.v[g], at(tr.v, s * tr.dv, tr.ov, 64 * g * esz(VF)), sg[g], vec);
        if constexpr (fmt_blocked(VF))
          r.v[g].s = *reinterpret_cast<const float*>(at(tr.vs, s * tr.ds, tr.os, g * tr.s1));
      }
    }
  }

  // The optimizer on one element, fp32 (Algorithm 1 Phase 2 for AdamW; the
  // other families of the paper's Appendix N list replace this body only).
  // sqrt and the reciprocal are the hardware instructions (<= 1 ulp).
  __device__ __forceinline__ static void phi(const EpiConst& k, float g, float& w, float& m, float& v) {
    if constexpr (OPT == OPT_ADAMW) {
      m = fmaf(k.b1, m, k.omb1 * g);                                     // m' = b1 m + (1-b1) G
      v = fmaf(k.b2, v, k.omb2 * (g * g));                               // v' = b2 v + (1-b2) G^2
      const float den = fmaf(__builtin_amdgcn_sqrtf(v), k.bc2s, k.eps);  // sqrt(v'/(1-b2^t)) + eps
      const float upd = (m * k.lrbc1) * __builtin_amdgcn_rcpf(den);      // lr m_hat / den
      w = fmaf(k.decay, w, -upd);                                        // (1 - lr wd) W - lr m_hat / den
    } else if constexpr (OPT == OPT_NADAM) {
      m = fmaf(k.b1, m, k.omb1 * g);
      v = fmaf(k.b2, v, k.omb2 * (g * g));
      const float den = fmaf(__builtin_amdgcn_sqrtf(v), k.bc2s, k.eps);  // sqrt(v'/(1-b2^t)) + eps
      const float num = fmaf(k.na1, m, k.na2 * g);                       // Nesterov-corrected m_hat
      w = fmaf(k.decay, w, -k.lr * (num * __builtin_amdgcn_rcpf(den)));
    } else if constexpr (OPT == OPT_RADAM) {
      m = fmaf(k.b1, m, k.omb1 * g);
      v = fmaf(k.b2, v, k.omb2 * (g * g));
      const float den = __builtin_amdgcn_sqrtf(v) + k.eps;               // sqrt(v') + eps
      const float upd = k.rect ? (m * k.rc) * __builtin_amdgcn_rcpf(den) : m * k.bc1;
      w = fmaf(k.decay, w, -k.lr * upd);
    } else if constexpr (OPT == OPT_LION) {
      const float c = fmaf(k.b1, m, k.omb1 * g);                         // interpolation
      const float s = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
      w = fmaf(k.decay, w, -k.lr * s);
      m = fmaf(k.b2, m, k.omb2 * g);
    } else if constexpr (OPT == OPT_RMSPROP) {
      const float gg = fmaf(k.wd, w, g);                                 // coupled L2
      v = fmaf(k.b2, v, k.omb2 * (gg * gg));                             // a v + (1-a) g^2
      const float den = __builtin_amdgcn_sqrtf(v) + k.eps;
      w = fmaf(-k.lr, gg * __builtin_amdgcn_rcpf(den), w);
    } else if constexpr (OPT == OPT_ADAGRAD) {
      const float gg = fmaf(k.wd, w, g);                                 // coupled L2
      v = fmaf(gg, gg, v);                                               // v + g^2
      const float den = __builtin_amdgcn_sqrtf(v) + k.eps;
      w = fmaf(-k.lr, gg * __builtin_amdgcn_rcpf(den), w);
    } else if constexpr (OPT == OPT_SGD) {
      w = fmaf(-k.lr, fmaf(k.wd, w, g), w);                              // W - lr (G + wd W)
    } else {                                                             // SGD with momentum
      const float gg = fmaf(k.wd, w, g);                                 // coupled L2
      m = fmaf(k.b1, m, gg);                                             // b' = mu b + g
      w = fmaf(-k.lr, m, w);                                             // W - lr b'
    }
  }

  // Decode, apply phi and store one chunk of row p.  Must be called by every
  // lane of the wave when a state is int8 (lane shuffles).
  template <int RM = RM_SEL>
  __device__ __forceinline__ static void apply_store(const KArgs& a, const TileRows<FAST>& tr, int ps, const Seg (&sg)[2],
                                                     const float (&g)[8], const Pending& r) {
    float w[8], m[8], v[8];
    // A block-scaled m or v enters phi only through b1 m, b2 m (Lion) or
    // b2 v, so its scale s is folded into those factors: phi sees the codes
    // and (b s) instead of b and the dequantised code * s.
    constexpr bool FOLD_M = fmt_blocked(MFMT) && (OPT == OPT_ADAMW || OPT == OPT_LION || OPT == OPT_SGDM);
    constexpr bool FOLD_V = fmt_blocked(VFMT) && OPT == OPT_ADAMW;
    EpiConst kc[2] = {a.c, a.c};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      dec4<WF>(r.w[s], w + 4 * s);
      if constexpr (FOLD_M) {
        dec4_codes<MFMT>(r.m[s], m + 4 * s);
        kc[s].b1 = a.c.b1 * r.m[s].s;
        if constexpr (OPT == OPT_LION) kc[s].b2 = a.c.b2 * r.m[s].s;
      } else {
        dec4<MFMT>(r.m[s], m + 4 * s);
      }
      if constexpr (FOLD_V) {
        dec4_codes<VFMT>(r.v[s], v + 4 * s);
        kc[s].b2 = a.c.b2 * r.v[s].s;
      } else {
        dec4<VFMT>(r.v[s], v + 4 * s);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) phi(FOLD_M || FOLD_V ? kc[i >> 2] : a.c, g[i], w[i], m[i], v[i]);
    const bool vec = a.vec_state != 0;
    const uint32_t rowbase = tr.idx + (uint32_t)ps * tr.didx;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (!sg[s].ok) continue;
      const uint32_t idx = rowbase + tr.qg[s];
      if constexpr (!fmt_blocked(WF))
        st4<WF, FAST, RM>(at(tr.w, ps * tr.dw, tr.ow, 64 * s * esz(WF)), sg[s], vec, w + 4 * s, a.c.sr, a.c.keyW,
                      idx);
      if constexpr (HAS_M && !fmt_blocked(MF))
        st4<MF, FAST, RM>(at(tr.m, ps * tr.dm, tr.om, 64 * s * esz(MF)), sg[s], vec, m + 4 * s, a.c.sr, a.c.keyM,
                      idx);
      if constexpr (HAS_V && !fmt_blocked(VF))
        st4<VF, FAST, RM>(at(tr.v, ps * tr.dv, tr.ov, 64 * s * esz(VF)), sg[s], vec, v + 4 * s, a.c.sr, a.c.keyV,
                      idx);
    }
    // a block-scaled stream: segment pointers of the codes (1 byte each) and of the scales
    if constexpr (fmt_blocked(WF)) {
      const uint32_t im[2] = {rowbase + tr.qg[0], rowbase + tr.qg[1]};
      uint8_t* const cp[2] = {reinterpret_cast<uint8_t*>(at(tr.w, ps * tr.dw, tr.ow, 0)),
                              reinterpret_cast<uint8_t*>(at(tr.w, ps * tr.dw, tr.ow, 64))};
      float* const sp[2] = {reinterpret_cast<float*>(at(tr.ws, ps * tr.ds, tr.os, 0)),
                            reinterpret_cast<float*>(at(tr.ws, ps * tr.ds, tr.os, tr.s1))};
      quantize_chunk<WF, false, true>(w, BLK ? BLK : a.block, sg, cp, vec, sp, a.c.sr, a.c.keyW, im);
    }
    if constexpr (HAS_M && fmt_blocked(MF)) {
      uint8_t* const cp[2] = {reinterpret_cast<uint8_t*>(at(tr.m, ps * tr.dm, tr.om, 0)),
                              reinterpret_cast<uint8_t*>(at(tr.m, ps * tr.dm, tr.om, 64))};
      float* const sp[2] = {reinterpret_cast<float*>(at(tr.ms, ps * tr.ds, tr.os, 0)),
                            reinterpret_cast<float*>(at(tr.ms, ps * tr.ds, tr.os, tr.s1))};
      quantize_chunk<MF, false>(m, BLK ? BLK : a.block, sg, cp, vec, sp);
    }
    if constexpr (HAS_V && fmt_blocked(VF)) {
      uint8_t* const cp[2] = {reinterpret_cast<uint8_t*>(at(tr.v, ps * tr.dv, tr.ov, 0)),
                              reinterpret_cast<uint8_t*>(at(tr.v, ps * tr.dv, tr.ov, 64))};
      float* const sp[2] = {reinterpret_cast<float*>(at(tr.vs, ps * tr.ds, tr.os, 0)),
                            reinterpret_cast<float*>(at(tr.vs, ps * tr.ds, tr.os, tr.s1))};
      quantize_chunk<VF, true>(v, BLK ? BLK : a.block, sg, cp, vec, sp);
    }
  }
};

// Epilogue over one 128 x 128 tile.  Thread mapping: in pass s thread t
// (0..NTE-1 of the epilogue group) owns row s*(NTE/16) + t/16 of the tile
// and two 4-element segments of it, at columns 4*(t%16) and 64 + 4*(t%16);
// the 16 lanes of a row access one contiguous 64-element run per
// instruction (whole 128-byte lines for every format but int8), and a
// row's 128 columns stay within 16 lanes for the int8 block reduction.
// issue() requests the state of one pass into a slot; consume() decodes a
// slot, applies the step and stores.  G comes from the LDS staging buffer
// (GF == FMT_NONE) or from the dW workspace in format GF (unfused baseline).
// With ACC, G is the staged tile plus the fp32 accumulator a.dW (one fp32
// addition per element, the same one k_gemm's accumulation performs).
// FULL: the tile lies wholly inside the matrix (the host passes it only when
// N and K are multiples of the tile), so every segment is in bounds at
// compile time and the per-segment checks, and the branches around the
// loads, stores and block reductions they guard, fold away.
template <class S, int GF, bool FAST, int DEPTH, int NTE = NT, bool ACC = false, bool FULL = false>
struct Epilogue {
  static_assert(!ACC || GF == FMT_NONE, "the accumulator adds to the staged tile");
  static constexpr int PASSES = TILE * TILE / (8 * NTE);  // 8 with 256 threads, 4 with 512
  static constexpr int RPP = NTE / 16;                    // rows per pass
  static constexpr int GR = ACC ? FMT_F32 : GF;           // format of the G words loaded per pass
  typename S::Pending pend[DEPTH];
  Raw4<GR> graw[DEPTH][2];
  TileRows<FAST> tr;
  int tid;

  static constexpr int esz(int fmt) { return fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 2 : 1; }

  // Tile bases, per-pass steps and this thread's offsets for the tile at
  // (row0, col0).
  __device__ __forceinline__ void rows(const KArgs& a, int row0, int col0) {
    using Off = typename TileRows<FAST>::Off;
    const int64_t rl = tid >> 4, cl = 4 * (tid & 15);
    const int64_t p0 = row0 + rl;
    const auto base = [&](void* ptr, int64_t ld, int es) {
      return static_cast<char*>(ptr) + ((int64_t)row0 * ld + col0) * es;
    };
    tr.w = base(a.W, a.ldw, esz(S::WFMT));
    tr.dw = (int64_t)RPP * a.ldw * esz(S::WFMT);
    tr.ow = (Off)((rl * a.ldw + cl) * esz(S::WFMT));
    if constexpr (S::HAS_M) {
      tr.m = base(a.m, a.ldm, esz(S::MFMT));
      tr.dm = (int64_t)RPP * a.ldm * esz(S::MFMT);
      tr.om = (Off)((rl * a.ldm + cl) * esz(S::MFMT));
    }
    if constexpr (S::HAS_V) {
      tr.v = base(a.v, a.ldv, esz(S::VFMT));
      tr.dv = (int64_t)RPP * a.ldv * esz(S::VFMT);
      tr.ov = (Off)((rl * a.ldv + cl) * esz(S::VFMT));
    }
    if constexpr (GR != FMT_NONE) {
      tr.g = base(a.dW, a.lddw, esz(GR));
      tr.dg = (int64_t)RPP * a.lddw * esz(GR);
      tr.og = (Off)((rl * a.lddw + cl) * esz(GR));
    }
    if constexpr (fmt_blocked(S::MFMT) || fmt_blocked(S::VFMT) || fmt_blocked(S::WFMT)) {
      // block is 32, 64 or 128: block indices are shifts; col0 is a multiple of 128
      const int bsh = __builtin_ctz((unsigned)(S::FIXED_BLOCK ? S::FIXED_BLOCK : a.block));
      const int64_t spr = a.K >> bsh;                                  // scales per row
      const auto sbase = [&](float* ptr) {
        return reinterpret_cast<char*>(ptr + (int64_t)row0 * spr + (col0 >> bsh));
      };
      if constexpr (fmt_blocked(S::MFMT)) tr.ms = sbase(a.ms);
      if constexpr (fmt_blocked(S::VFMT)) tr.vs = sbase(a.vs);
      if constexpr (fmt_blocked(S::WFMT)) tr.ws = sbase(a.wsc);
      tr.ds = (int64_t)RPP * spr * 4;
      tr.os = (Off)((rl * spr + (cl >> bsh)) * 4);
      tr.s1 = (int64_t)(64 >> bsh) * 4;
    }
    tr.idx = (uint32_t)p0 * (uint32_t)a.K;
    tr.didx = (uint32_t)RPP * (uint32_t)a.K;
#pragma unroll
    for (int g = 0; g < 2; ++g) tr.qg[g] = (uint32_t)(col0 + 64 * g + (int)cl);
  }

  __device__ __forceinline__ void segs(const KArgs& a, int p, int col0, Seg (&sg)[2]) const {
    const int cl = 4 * (tid & 15);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      sg[g].q = col0 + 64 * g + cl;
      if constexpr (FULL) {
        sg[g].nv = 4;
        sg[g].ok = true;
      } else {
        sg[g].nv = max(0, min(4, a.K - sg[g].q));
        sg[g].ok = sg[g].nv > 0 && p < a.N;
      }
    }
  }

  __device__ __forceinline__ void issue(const KArgs& a, int row0, int col0, int s, int slot) {
    const int p = row0 + s * RPP + (tid >> 4);
    Seg sg[2];
    segs(a, p, col0, sg);
    S::load(a, tr, s, sg, pend[slot]);
    if constexpr (GR != FMT_NONE) {
      const bool gvec = a.vec_dw != 0;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (sg[g].ok) ld4<GR, FAST>(graw[slot][g], at(tr.g, s * tr.dg, tr.og, 64 * g * esz(GR)), sg[g], gvec);
        else zero4(graw[slot][g]);
      }
    }
  }

  // G of pass s (from sG or from the slot's dW words)
  // r_off: the tile row that sG's row 0 holds
  __device__ __forceinline__ void grad(const float* sG, int s, int slot, float (&g)[8], int r_off = 0) const {
    if constexpr (GF == FMT_NONE) {
      const int rl = s * RPP + (tid >> 4) - r_off, cl = 4 * (tid & 15);
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(sG + rl * GP + cl);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(sG + rl * GP + 64 + cl);
#pragma unroll
      for (int i = 0; i < 4; ++i) { g[i] = g0[i]; g[4 + i] = g1[i]; }
      if constexpr (ACC) {
        float acc[8];
        dec4<FMT_F32>(graw[slot][0], acc);
        dec4<FMT_F32>(graw[slot][1], acc + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = acc[i] + g[i];
      }
    } else {
      dec4<GF>(graw[slot][0], g);
      dec4<GF>(graw[slot][1], g + 4);
    }
  }

  template <int RM>
  __device__ __forceinline__ void consume(const KArgs& a, int row0, int col0, int s, const float (&g)[8],
                                          const typename S::Pending& cur) const {
    const int p = row0 + s * RPP + (tid >> 4);
    Seg sg[2];
    segs(a, p, col0, sg);
    S::template apply_store<RM>(a, tr, s, sg, g, cur);
  }

  // One tile with a rolling window of DEPTH passes in flight: prefetch()
  // requests the first DEPTH passes (state only, no G needed), and
  // run_prefetched() the rest of the tile.
  template <int NPRE = DEPTH>
  __device__ __forceinline__ void prefetch(const KArgs& a, int row0, int col0) {
    rows(a, row0, col0);
#pragma unroll
    for (int s = 0; s < NPRE && s < PASSES; ++s) issue(a, row0, col0, s, s);
  }

  // The passes NPRE .. DEPTH - 1 that prefetch<NPRE>() left out.
  template <int NPRE>
  __device__ __forceinline__ void prefetch_rest(const KArgs& a, int row0, int col0) {
#pragma unroll
    for (int s = NPRE; s < DEPTH && s < PASSES; ++s) issue(a, row0, col0, s, s);
  }

  template <int RM = RM_SEL>
  __device__ __forceinline__ void run_tile(const KArgs& a, const float* sG, int row0, int col0) {
    prefetch(a, row0, col0);
    run_prefetched<RM>(a, sG, row0, col0);
  }

  // The rest of the tile with G staged through LDS in two 64-row halves (sG
  // holds 64 rows): the waves that own a half (wr = h) write it, and all four
  // consume it in passes 4h .. 4h + 3.  Called right after the mainloop with
  // a barrier between: the stages are free.
  template <int RM = RM_SEL>
  __device__ __forceinline__ void run_halves(const KArgs& a, float* sG, const f32x16 (&acc)[2][2], int row0,
                                             int col0) {
    static_assert(NTE == NT && PASSES == 8, "four passes per 64-row half");
    const int wr = tid >> 7;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wr == h) store_acc_half(sG, acc, tid);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bar();   // the half is in LDS
#pragma unroll
      for (int s = 4 * h; s < 4 * h + 4; ++s) {
        const int slot = s % DEPTH;
        float g[8];
        grad(sG, s, slot, g, 64 * h);
        const typename S::Pending cur = pend[slot];
        if (s + DEPTH < PASSES) issue(a, row0, col0, s + DEPTH, slot);
        consume<RM>(a, row0, col0, s, g, cur);
      }
      if (h == 0) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bar();   // every wave has read the first half
      }
    }
  }

  template <int RM = RM_SEL>
  __device__ __forceinline__ void run_prefetched(const KArgs& a, const float* sG, int row0, int col0) {
#pragma unroll
    for (int s = 0; s < PASSES; ++s) {
      const int slot = s % DEPTH;
      float g[8];
      grad(sG, s, slot, g);
      const typename S::Pending cur = pend[slot];
      if (s + DEPTH < PASSES) issue(a, row0, col0, s + DEPTH, slot);
      consume<RM>(a, row0, col0, s, g, cur);
    }
  }

  // The same with the rounding mode fixed per tile from the wave-uniform
  // mask, where the step stores bf16.
  __device__ __forceinline__ void run_halves_rm(const KArgs& a, float* sG, const f32x16 (&acc)[2][2], int row0,
                                                int col0) {
    if constexpr (S::BF16_STORE) {
      if (a.c.sr) run_halves<RM_SR>(a, sG, acc, row0, col0);
      else run_halves<RM_RNE>(a, sG, acc, row0, col0);
    } else {
      run_halves(a, sG, acc, row0, col0);
    }
  }
  __device__ __forceinline__ void run_prefetched_rm(const KArgs& a, const float* sG, int row0, int col0) {
    if constexpr (S::BF16_STORE) {
      if (a.c.sr) run_prefetched<RM_SR>(a, sG, row0, col0);
      else run_prefetched<RM_RNE>(a, sG, row0, col0);
    } else {
      run_prefetched(a, sG, row0, col0);
    }
  }
  __device__ __forceinline__ void run_tile_rm(const KArgs& a, const float* sG, int row0, int col0) {
    prefetch(a, row0, col0);
    run_prefetched_rm(a, sG, row0, col0);
  }
};

// ------------------------------------------------------------------------
// Kernels
// ------------------------------------------------------------------------
// IN: input format.  FAST (bf16 inputs only): the asynchronous
// direct-to-LDS mainloop and the vector-only epilogue; the host selects it
// when X, dY and the state rows are aligned and N, K are multiples of 8.
//
// Occupancy.  FAST kernels whose pending state is small (at most 6 registers
// per 4-element segment: bf16 W with bf16 / 8-bit moments or one fp32 moment,
// fp32 W with one compact moment, SGD) run three workgroups per CU: a 3-stage
// ring, G staged in two 64-row halves, 2 passes of state in flight, <= 168
// VGPRs (without spills, except 2 registers in Lion with an E4M3 weight and
// E4M3 m).  With a larger state (two fp32 moments) the grouped
// kernel does the same with 2 passes in flight, none of them requested before
// the mainloop (so that they hold no registers during it; measured faster on
// the Llama decoder layer), while the single-layer kernel keeps two
// workgroups per CU, a 4-stage ring and 4 passes in flight (measured faster
// per layer, most on the short q / k / v / o launches).  Exact accumulation
// keeps two.
constexpr int raw_words(int fmt) {
  return fmt == FMT_F32 ? 4 : fmt == FMT_BF16 ? 2 : fmt == FMT_NONE ? 0 : 2;
}
template <int OPT, int WF, int MF, int VF, bool FAST>
constexpr int pending_words() {
  using S = Step<OPT, WF, MF, VF, FAST>;
  return raw_words(S::WFMT) + raw_words(S::MFMT) + raw_words(S::VFMT);
}
template <int OPT, int WF, int MF, int VF, bool FAST>
constexpr bool small_state() {
  // an E4M3 weight beside two moments re-encodes three blocks per chunk:
  // that epilogue spills within the register budget of three per CU
  return pending_words<OPT, WF, MF, VF, FAST>() <= 6 && !(fmt_blocked(WF) && opt_has_m(OPT) && opt_has_v(OPT));
}
template <int OPT, int WF, int MF, int VF, bool FAST, bool ACC, bool GROUP>
constexpr bool three_per_cu() {
  return FAST && !ACC && (GROUP || small_state<OPT, WF, MF, VF, FAST>());
}
template <int OPT, int WF, int MF, int VF, bool FAST>
constexpr bool scaled_state() {
  using S = Step<OPT, WF, MF, VF, FAST>;
  return fmt_blocked(S::MFMT) || fmt_blocked(S::VFMT) || fmt_blocked(S::WFMT);
}
// Passes of state in flight, and how many of them are requested before the
// mainloop.  In the grouped kernel (a few more registers for the layer
// lookup) states with block scales request none early: AdamW with int8 or
// E4M3 moments otherwise spills, and measured 9-10% slower on the Llama
// decoder layer (Lion with int8 m 2%), while bf16 moments and one fp32
// moment are 2-3% faster with both requested early.
constexpr int SMALL_DEPTH = 2, SMALL_PRE = 2, GROUP_LARGE_DEPTH = 2, GROUP_LARGE_PRE = 0;
template <int OPT, int WF, int MF, int VF, bool FAST, bool ACC, bool GROUP>
constexpr int epi_depth() {
  return !three_per_cu<OPT, WF, MF, VF, FAST, ACC, GROUP>() ? 4
         : small_state<OPT, WF, MF, VF, FAST>()              ? SMALL_DEPTH
         : pending_words<OPT, WF, MF, VF, FAST>() <= 10      ? GROUP_LARGE_DEPTH
                                                              : 1;   // fp32 W and two fp32 moments
}
template <int OPT, int WF, int MF, int VF, bool FAST, bool ACC, bool GROUP>
constexpr int epi_pre() {
  return !three_per_cu<OPT, WF, MF, VF, FAST, ACC, GROUP>() ? 4
         : !small_state<OPT, WF, MF, VF, FAST>()             ? GROUP_LARGE_PRE
         : GROUP && scaled_state<OPT, WF, MF, VF, FAST>()    ? 0
                                                              : SMALL_PRE;
}

template <int IN, bool FAST, int OPT, int WF, int MF, int VF, bool ACC = false, int BLK = 0, bool FULL = false>
__global__ void __launch_bounds__(NT, (three_per_cu<OPT, WF, MF, VF, FAST, ACC, false>() ? 3 : 2))
    k_fused(const KArgs a) {
  constexpr bool OCC3 = three_per_cu<OPT, WF, MF, VF, FAST, ACC, false>();
  __shared__ __attribute__((aligned(16))) char lds[OCC3 ? LDS_HALF : LDS_BYTES];
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  const int row0 = ti * TILE, col0 = tj * TILE;
  // FAST: the state of the first passes is requested before the mainloop,
  // so the HBM stream of this tile starts while its gradient is computed.
  // These loads are older than every mainloop load, so the mainloop's
  // in-order vmcnt waits still count exactly its own chunks.  (The
  // register-staged mainloop has no registers to spare for it.)
  Epilogue<Step<OPT, WF, MF, VF, FAST, BLK>, FMT_NONE, FAST, epi_depth<OPT, WF, MF, VF, FAST, ACC, false>(), NT, ACC, FULL>
      epi;
  epi.tid = threadIdx.x;
  if constexpr (OCC3) {
    constexpr int PRE = epi_pre<OPT, WF, MF, VF, FAST, ACC, false>();
    epi.template prefetch<PRE>(a, row0, col0);
    f32x16 acc[2][2];
    WorkgroupSync sync;
    dma_accumulate<MainBF16Dma3>(a, lds, row0, col0, threadIdx.x, acc, sync);
    bar();   // every wave is done reading the stages before G overwrites them
    epi.template prefetch_rest<PRE>(a, row0, col0);
    epi.run_halves_rm(a, reinterpret_cast<float*>(lds), acc, row0, col0);
  } else if constexpr (FAST) {
    epi.prefetch(a, row0, col0);
    tile_gradient_dma(a, lds, row0, col0);
    epi.run_prefetched_rm(a, reinterpret_cast<const float*>(lds), row0, col0);
  } else {
    tile_gradient<IN>(a, lds, row0, col0);
    epi.prefetch(a, row0, col0);
    epi.run_prefetched(a, reinterpret_cast<const float*>(lds), row0, col0);
  }
}

// Several independent layers in one launch: the workgroups cover the
// concatenation of the layers' tile spaces (layer order, row-major tiles
// within a layer).  Each workgroup finds its layer from the prefix tile
// counts (uniform scalar work) and then runs the k_fused code path of three
// workgroups per CU on it (for every state size, see above), so every
// element is computed as a separate call would compute it.  BLK: the block
// size of the 8-bit states when every layer has that one (0: each layer's).
template <int OPT, int WF, int MF, int VF, int BLK = 0, bool FULL = false>
__global__ void __launch_bounds__(NT, 3) k_fused_group(const GroupArgs g) {
  static_assert(three_per_cu<OPT, WF, MF, VF, true, false, true>(), "the grouped kernel runs three per CU");
  __shared__ __attribute__((aligned(16))) char lds[LDS_HALF];
  const int bid = (int)blockIdx.x;
  int li = 0;
#pragma unroll
  for (int i = 1; i < GROUP_MAX; ++i) li += (i < g.n && bid >= g.first_tile[i]) ? 1 : 0;
  const KArgs& a = g.layer[li];
  int ti, tj;
  tile_coords(bid - g.first_tile[li], a.tiles_n, a.tiles_k, ti, tj);
  const int row0 = ti * TILE, col0 = tj * TILE;
  Epilogue<Step<OPT, WF, MF, VF, true, BLK>, FMT_NONE, true, epi_depth<OPT, WF, MF, VF, true, false, true>(), NT, false,
           FULL> epi;
  constexpr int PRE = epi_pre<OPT, WF, MF, VF, true, false, true>();
  epi.tid = threadIdx.x;
  epi.template prefetch<PRE>(a, row0, col0);        // as in k_fused
  f32x16 acc[2][2];
  WorkgroupSync sync;
  dma_accumulate<MainBF16Dma3>(a, lds, row0, col0, threadIdx.x, acc, sync);
  bar();   // every wave is done reading the stages before G overwrites them
  epi.template prefetch_rest<PRE>(a, row0, col0);
  epi.run_halves_rm(a, reinterpret_cast<float*>(lds), acc, row0, col0);
}

constexpr int LDS_WIDE = MainWide::S * MainWide::STAGE;   // 128 KiB
static_assert(LDS_WIDE >= LDS_G, "the staged G tile aliases the ring");

// Wide variant for aligned bf16 layers with a long token axis: one 256 x 256
// macro tile per workgroup of 8 waves (one workgroup per CU: the ring takes
// 128 KiB of LDS).  After the mainloop the four 128 x 128 sub-tiles are
// staged through LDS one at a time, each by its two owner waves (wr = sub / 2,
// wc / 2 = sub % 2), and all 512 threads run the epilogue on it with 2 of its
// 4 passes in flight.
template <int OPT, int WF, int MF, int VF, bool FULL = false>
__global__ void __launch_bounds__(2 * NT, 1) k_fused_wide(const KArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_WIDE];
  const int tw = (a.K + MainWide::W - 1) / MainWide::W;
  const int mi = (int)blockIdx.x / tw;
  const int row0 = mi * MainWide::W, col0 = ((int)blockIdx.x - mi * tw) * MainWide::W;
  f32x16 acc[4][2];
  wide_accumulate(a, lds, row0, col0, acc);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave >> 2, wc = wave & 3;
  float* sG = reinterpret_cast<float*>(lds);
  Epilogue<Step<OPT, WF, MF, VF, true>, FMT_NONE, true, 2, 2 * NT, false, FULL> epi;   // 2 of the 4 passes in flight
  epi.tid = threadIdx.x;
  for (int sub = 0; sub < 4; ++sub) {
    const int srow0 = row0 + (sub >> 1) * TILE, scol0 = col0 + (sub & 1) * TILE;
    bar();                                   // the ring / the previous sub-tile is no longer read
    if (wr == (sub >> 1) && (wc >> 1) == (sub & 1)) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int c = (wc & 1) * 64 + bj * 32 + (lane & 31);
            sG[r * GP + c] = acc[bi][bj][e];
          }
    }
    __syncthreads();
    if (srow0 < a.N && scol0 < a.K) epi.run_tile_rm(a, sG, srow0, scol0);
  }
}

template <int IN, bool DMA>
__global__ void __launch_bounds__(NT, 2) k_gemm(const KArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  const int row0 = ti * TILE, col0 = tj * TILE;
  const int cl = 4 * (threadIdx.x & 15);
  const bool vec = a.vec_dw != 0;
  // Gradient accumulation (dw_add, fp32 dW): the old values of all 8 passes
  // are requested at once, before any store -- issued per pass, each load
  // would wait behind the previous pass's stores to the same buffer.  On the
  // DMA path they are requested before the mainloop (older than every chunk
  // load, so its in-order vmcnt waits stay exact), as the fused kernels do
  // with the optimizer state.
  Raw4<FMT_F32> old[8][2];
  const auto request_old = [&]() {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int p = row0 + s * 16 + (threadIdx.x >> 4);
      const char* rowp = static_cast<const char*>(a.dW) + (int64_t)p * a.lddw * 4;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        Seg sg;
        sg.q = col0 + 64 * g + cl;
        sg.nv = max(0, min(4, a.K - sg.q));
        sg.ok = sg.nv > 0 && p < a.N;
        if (sg.ok) ld4<FMT_F32, false>(old[s][g], rowp + (int64_t)sg.q * 4, sg, vec);
        else zero4(old[s][g]);
      }
    }
  };
  const bool add = a.dw_add != 0 && a.dw_fmt == FMT_F32;
  if constexpr (DMA) {
    if (add) request_old();
    tile_gradient_dma(a, lds, row0, col0);
  } else {
    tile_gradient<IN>(a, lds, row0, col0);
    if (add) request_old();
  }
  const float* sG = reinterpret_cast<const float*>(lds);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int rl = s * 16 + (threadIdx.x >> 4);
    const int p = row0 + rl;
    if (p >= a.N) continue;
    char* rowp = static_cast<char*>(a.dW) + (int64_t)p * a.lddw * (a.dw_fmt == FMT_F32 ? 4 : 2);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      Seg sg;
      sg.q = col0 + 64 * g + cl;
      sg.nv = max(0, min(4, a.K - sg.q));
      sg.ok = sg.nv > 0;
      if (!sg.ok) continue;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sG[rl * GP + 64 * g + cl + i];
      if (add) {                            // gradient accumulation: old + G, one fp32 addition
        float o[4];
        dec4<FMT_F32>(old[s][g], o);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = o[i] + x[i];
      }
      if (a.dw_fmt == FMT_F32) st4<FMT_F32, false>(rowp + (int64_t)sg.q * 4, sg, vec, x, 0, 0, 0);
      else st4<FMT_BF16, false>(rowp + (int64_t)sg.q * 2, sg, vec, x, 0, 0, 0);
    }
  }
}

template <int GF, bool FAST, int OPT, int WF, int MF, int VF>
__global__ void __launch_bounds__(NT, 2) k_step(const KArgs a) {
  int ti, tj;
  tile_coords(blockIdx.x, a.tiles_n, a.tiles_k, ti, tj);
  Epilogue<Step<OPT, WF, MF, VF, FAST>, GF, FAST, 4> epi;
  epi.tid = threadIdx.x;
  epi.run_tile(a, nullptr, ti * TILE, tj * TILE);
}

// ------------------------------------------------------------------------
// Launchers of one (optimizer, m format, v format) combination.
// ------------------------------------------------------------------------
static inline dim3 tile_grid(const KArgs& a) { return dim3((unsigned)(a.tiles_n * a.tiles_k)); }

// Whole tiles: every 128 x 128 tile of the layer lies inside it.
static inline bool whole_tiles(const KArgs& a) { return a.N % TILE == 0 && a.K % TILE == 0; }

// The compile-time FULL epilogue (no per-segment bounds checks) is taken where
// it was measured faster: 8-bit and fp32 states (the grouped Llama decoder
// layer 5% faster with fp32 moments, 8% with int8 or E4M3 moments; gate_proj
// int8 / E4M3 6-8%, Lion / SGD-m / SGD 4-6%).  With bf16 moments the
// unguarded code spills at three workgroups per CU and runs 10-14% slower, so
// those keep the checked epilogue.
constexpr bool full_pays(int m_fmt, int v_fmt) { return m_fmt != FMT_BF16 && v_fmt != FMT_BF16; }

template <int O, int M, int V>
hipError_t combo_fused(const KArgs& a, int in_fmt, int w_fmt, hipStream_t st) {
  const bool fast = a.dma_ok && a.vec_state && (a.K % 4) == 0;
  const dim3 b(NT);
  if (w_fmt != FMT_BF16 && w_fmt != FMT_F32) return hipErrorInvalidValue;
  const bool wbf = w_fmt == FMT_BF16;
  if (in_fmt == FMT_BF16 && fast && a.BT >= WIDE_MIN_BT) {
    const dim3 g((unsigned)(((a.N + 255) / 256) * ((a.K + 255) / 256)));
    // whole 128 x 128 sub-tiles: the epilogue without per-segment bounds checks
    // (not with bf16 moments, nor an fp32 weight beside 8-bit moments: those spill)
    if constexpr (full_pays(M, V)) {
      if (whole_tiles(a)) {
        if (wbf) {
          hipLaunchKernelGGL((k_fused_wide<O, FMT_BF16, M, V, true>), g, dim3(2 * NT), 0, st, a);
          return hipGetLastError();
        }
        if constexpr (!fmt_blocked(M) && !fmt_blocked(V)) {
          hipLaunchKernelGGL((k_fused_wide<O, FMT_F32, M, V, true>), g, dim3(2 * NT), 0, st, a);
          return hipGetLastError();
        }
      }
    }
    if (wbf) hipLaunchKernelGGL((k_fused_wide<O, FMT_BF16, M, V>), g, dim3(2 * NT), 0, st, a);
    else hipLaunchKernelGGL((k_fused_wide<O, FMT_F32, M, V>), g, dim3(2 * NT), 0, st, a);
  } else if (in_fmt == FMT_BF16 && fast) {
#define FORGE_FUSED_FAST(BLK, FULL)                                                                                     \
  if (wbf) hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_BF16, M, V, false, BLK, FULL>), tile_grid(a), b, 0, st, a); \
  else hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_F32, M, V, false, BLK, FULL>), tile_grid(a), b, 0, st, a);    \
  return hipGetLastError();
    // (an fp32 weight beside 8-bit moments spills with FULL: checked epilogue)
    const bool full = whole_tiles(a) && (wbf || !(fmt_blocked(M) || fmt_blocked(V)));
    // block-scaled moments in 128-element blocks: the block fixed at compile time (as in combo_group)
    if constexpr (fmt_blocked(M) || fmt_blocked(V)) {
      if (a.block == 128) {
        if (full) { FORGE_FUSED_FAST(128, true) }
        FORGE_FUSED_FAST(128, false)
      }
    } else if constexpr (full_pays(M, V) && !(M == FMT_F32 && V == FMT_F32)) {
      // (two fp32 moments at two workgroups per CU: measured 1% slower with FULL)
      if (full) { FORGE_FUSED_FAST(0, true) }
    }
    FORGE_FUSED_FAST(0, false)
#undef FORGE_FUSED_FAST
  } else if (in_fmt == FMT_BF16) {
    if (wbf) hipLaunchKernelGGL((k_fused<FMT_BF16, false, O, FMT_BF16, M, V>), tile_grid(a), b, 0, st, a);
    else hipLaunchKernelGGL((k_fused<FMT_BF16, false, O, FMT_F32, M, V>), tile_grid(a), b, 0, st, a);
  } else if (in_fmt == FMT_F32) {
    if (wbf) hipLaunchKernelGGL((k_fused<FMT_F32, false, O, FMT_BF16, M, V>), tile_grid(a), b, 0, st, a);
    else hipLaunchKernelGGL((k_fused<FMT_F32, false, O, FMT_F32, M, V>), tile_grid(a), b, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 8-bit states with 128-element blocks in every layer (the workloads' block)
// take a kernel with the block fixed at compile time: the quantiser's
// block-size branches and shifts fold away (measured 1-2% on the Llama
// decoder layer with int8 or E4M3 moments).
template <int O, int M, int V>
hipError_t combo_group(const GroupArgs& g, int w_fmt, hipStream_t st) {
  if (g.n < 1 || g.n > GROUP_MAX) return hipErrorInvalidValue;
  if (w_fmt != FMT_BF16 && w_fmt != FMT_F32) return hipErrorInvalidValue;
  const dim3 grid((unsigned)g.first_tile[g.n]);
  bool b128 = false, full = true;
  if constexpr (fmt_blocked(M) || fmt_blocked(V)) {
    b128 = true;
    for (int i = 0; i < g.n; ++i) b128 = b128 && g.layer[i].block == 128;
  }
  for (int i = 0; i < g.n; ++i) full = full && whole_tiles(g.layer[i]);
  if constexpr (fmt_blocked(M) || fmt_blocked(V)) full = full && w_fmt == FMT_BF16;   // as in combo_fused
#define FORGE_GROUP(BLK, FULL)                                                                                          \
  if (w_fmt == FMT_BF16) hipLaunchKernelGGL((k_fused_group<O, FMT_BF16, M, V, BLK, FULL>), grid, dim3(NT), 0, st, g);   \
  else hipLaunchKernelGGL((k_fused_group<O, FMT_F32, M, V, BLK, FULL>), grid, dim3(NT), 0, st, g);                      \
  return hipGetLastError();
  if constexpr (fmt_blocked(M) || fmt_blocked(V)) {
    if (b128) {
      if (full) { FORGE_GROUP(128, true) }
      FORGE_GROUP(128, false)
    }
  } else if constexpr (full_pays(M, V)) {
    if (full) { FORGE_GROUP(0, true) }
  }
  FORGE_GROUP(0, false)
#undef FORGE_GROUP
}

template <int O, int M, int V>
hipError_t combo_step(const KArgs& a, int w_fmt, hipStream_t st) {
  const bool fast = a.vec_state && a.vec_dw && (a.K % 4) == 0;
  if (w_fmt != FMT_BF16 && w_fmt != FMT_F32) return hipErrorInvalidValue;
  const bool wbf = w_fmt == FMT_BF16;
#define FORGE_STEP_LAUNCH(GF, FA)                                                                         \
  if (wbf) hipLaunchKernelGGL((k_step<GF, FA, O, FMT_BF16, M, V>), tile_grid(a), dim3(NT), 0, st, a);     \
  else hipLaunchKernelGGL((k_step<GF, FA, O, FMT_F32, M, V>), tile_grid(a), dim3(NT), 0, st, a);
  if (a.dw_fmt == FMT_F32) {
    if (fast) { FORGE_STEP_LAUNCH(FMT_F32, true) } else { FORGE_STEP_LAUNCH(FMT_F32, false) }
  } else if (a.dw_fmt == FMT_BF16) {
    if (fast) { FORGE_STEP_LAUNCH(FMT_BF16, true) } else { FORGE_STEP_LAUNCH(FMT_BF16, false) }
  } else {
    return hipErrorInvalidValue;
  }
#undef FORGE_STEP_LAUNCH
  return hipGetLastError();
}

template <int O, int M, int V>
hipError_t combo_fused_acc(const KArgs& a, int w_fmt, hipStream_t st) {
  if constexpr (full_pays(M, V) && !fmt_blocked(M) && !fmt_blocked(V)) {
    if (w_fmt == FMT_BF16 && whole_tiles(a)) {   // whole tiles: the unchecked epilogue
      hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_BF16, M, V, true, 0, true>), tile_grid(a), dim3(NT), 0, st, a);
      return hipGetLastError();
    }
  }
  if (w_fmt == FMT_BF16) hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_BF16, M, V, true>), tile_grid(a), dim3(NT), 0, st, a);
  else if (w_fmt == FMT_F32) hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_F32, M, V, true>), tile_grid(a), dim3(NT), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// An E4M3 weight with block scales (bf16 inputs): the same kernels as a bf16
// or fp32 weight, instantiated only for the combinations of the FP8-weight
// list.
template <int O, int M, int V>
hipError_t combo_fused_fp8w(const KArgs& a, hipStream_t st) {
  const bool fast = a.dma_ok && a.vec_state && (a.K % 4) == 0;
  if (fast && a.BT >= WIDE_MIN_BT) {
    const dim3 g((unsigned)(((a.N + 255) / 256) * ((a.K + 255) / 256)));
    hipLaunchKernelGGL((k_fused_wide<O, FMT_E4M3, M, V>), g, dim3(2 * NT), 0, st, a);
  } else if (fast && whole_tiles(a) && a.block == 128) {
    // whole tiles in 128-element blocks: the unchecked epilogue, the block fixed at compile time
    hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_E4M3, M, V, false, 128, true>), tile_grid(a), dim3(NT), 0, st, a);
  } else if (fast) {
    hipLaunchKernelGGL((k_fused<FMT_BF16, true, O, FMT_E4M3, M, V>), tile_grid(a), dim3(NT), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_fused<FMT_BF16, false, O, FMT_E4M3, M, V>), tile_grid(a), dim3(NT), 0, st, a);
  }
  return hipGetLastError();
}
#define FORGE_INSTANTIATE_FP8W(O, M, V) \
  template hipError_t combo_fused_fp8w<O, M, V>(const KArgs&, hipStream_t);

// Explicit instantiation of the launchers of one combination.
#define FORGE_INSTANTIATE(O, M, V)                                                  \
  template hipError_t combo_fused<O, M, V>(const KArgs&, int, int, hipStream_t);   \
  template hipError_t combo_group<O, M, V>(const GroupArgs&, int, hipStream_t);    \
  template hipError_t combo_step<O, M, V>(const KArgs&, int, hipStream_t);         \
  template hipError_t combo_fused_acc<O, M, V>(const KArgs&, int, hipStream_t);

}  // namespace forge
