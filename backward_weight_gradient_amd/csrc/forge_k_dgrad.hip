// The input gradient of a linear layer, dX = dY W (FORGE paper, Appendix A,
// Remark 1: it must be formed from the weight before the fused step
// overwrites it).  dY [BT, N], W [N, K], dX [BT, K], reduction over N in
// fp32.
//
// k_dgrad_bf16<TM> (bf16 dY and W, 16-byte aligned rows, N and K multiples
// of 8): one TM x 128 tile of dX per 256-thread workgroup (4 waves, 2 x 2
// arrangement of TM/2 x 64; TM = 64 when 128-token tiles would leave CUs
// idle, as for q/gate/up at BT = 512), v_mfma_f32_32x32x16_bf16 over chunks
// of 32 of the reduction index, both operands brought into a 4-stage LDS
// ring by
// buffer_load ... lds.  W's chunk (32 rows of W, 128 columns) has the
// reduction index as its row, like the weight-gradient operands, and is
// read with the transposing LDS read; dY's chunk (128 tokens, 32 reduction
// elements) has the reduction index along the row and is read 16 bytes per
// lane, its 64-byte rows XOR-swizzled in 16-byte units so that 16 lanes
// reading 16 consecutive rows cover all 64 banks.
//
// Split reduction (128-token tiles only): split s (the work index over the
// tiles, see xcd_work) takes the
// chunks [s c, min(nk, (s + 1) c)), c = ceil(nk / splits), and writes its
// fp32 partial tile to the workspace; k_dgrad_reduce then adds the splits'
// partials in split order (deterministic) and stores dX.  For the short-token,
// long-reduction layers this moves each W panel through L2 -> LDS once per
// 128 tokens instead of once per 64 on the same number of workgroups.
//
// k_dgrad_generic (any dtype combination, any alignment, and the E4M3 weight
// with block scales, decoded exactly): 64 x 64 tiles, fp32 FMA from an
// LDS-staged fp32 copy of both operands.

#include "forge_device.h"

#include <mutex>

namespace forge {

namespace {

constexpr int DG_TN = 32;                            // reduction elements per chunk
constexpr int DG_OPB = 8192;                         // bytes of W's chunk per stage (32 x 128 bf16)

// TM-token tiles with an S-stage ring (S - 1 chunks in flight).
template <int TM, int S>
struct DgShape {
  static constexpr int APB = TM * DG_TN * 2;         // bytes of dY's chunk per stage
  static constexpr int STAGE = APB + DG_OPB;
  static constexpr int ABLK = TM / 64;               // dY loads per wave per chunk (1 KiB each)
  static constexpr int LOADS = ABLK + 2;             // buffer loads per wave per chunk
  static constexpr int GP_ = TILE + 4;               // fp32 pitch of the staged output tile
  static constexpr int LDS = (S * STAGE > TM * GP_ * 4) ? S * STAGE : TM * GP_ * 4;
};

// Wait until at most `ahead` chunks' loads (LOADS each) are still in flight.
template <int LOADS, int K>
__device__ __forceinline__ void dg_wait_ahead(int ahead) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= K) wait_vmcnt<K * LOADS>();
    else dg_wait_ahead<LOADS, K - 1>(ahead);
  }
}

// Byte offset of (token row m, 16-byte segment s) in dY's chunk region.
__device__ __forceinline__ uint32_t dg_a_off(int m, int s) { return (uint32_t)(m * 64 + ((s ^ ((m >> 2) & 3)) << 4)); }

template <int TM, int S>
struct DgradLoader {
  using SH = DgShape<TM, S>;
  __amdgpu_buffer_rsrc_t rA, rB;
  uint32_t oobA, oobB;
  uint32_t aTok[SH::ABLK], aSeg[SH::ABLK];   // dY: byte offset of this lane's token row, 16-byte segment
  bool aOk[SH::ABLK];
  uint32_t bCol[2];            // W: byte offset of this lane's 8-column chunk
  int bRow[2];                 // W: row within the chunk
  bool bOk[2];
  int wave;

  // gtid: thread index within the 256 threads of one reduction group
  __device__ __forceinline__ void init(const DgArgs& g, int tok0, int col0, int gtid) {
    const int lane = gtid & 63;
    wave = gtid >> 6;
    oobA = (uint32_t)((uint64_t)g.BT * g.lddy * 2);
    oobB = (uint32_t)((uint64_t)g.N * g.ldw * 2);
    rA = make_rsrc(g.dY, oobA);
    rB = make_rsrc(g.W, oobB);
#pragma unroll
    for (int r = 0; r < SH::ABLK; ++r) {
      // dY: 1 KiB block = 16 token rows x 4 segments; lane -> (row, physical segment)
      const int blk = SH::ABLK * wave + r;
      const int m = blk * 16 + (lane >> 2);
      const int s = (lane & 3) ^ ((m >> 2) & 3);       // logical segment stored at this slot
      aOk[r] = tok0 + m < g.BT;
      aTok[r] = (uint32_t)((uint64_t)(tok0 + m) * g.lddy * 2);
      aSeg[r] = (uint32_t)(s * 16);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // W: 1 KiB block = 4 rows x 16 chunks of 8 columns, rows XOR-swizzled as
      // the weight-gradient operands (MainBF16::off)
      const int blk = 2 * wave + r;
      const int t = blk * 4 + (lane >> 4);
      const int c = (lane & 15) ^ ((t & 3) << 2);
      bRow[r] = t;
      bOk[r] = col0 + c * 8 < g.K;
      bCol[r] = (uint32_t)(col0 + c * 8) * 2;
    }
  }

  // dY's chunk kc alone (ABLK loads per wave)
  __device__ __forceinline__ void issue_a(const DgArgs& g, int kc, char* stage) const {
    const int n0 = kc * DG_TN;
#pragma unroll
    for (int r = 0; r < SH::ABLK; ++r) {
      const uint32_t oa = (aOk[r] && n0 + (int)(aSeg[r] >> 1) < g.N) ? aTok[r] + (uint32_t)n0 * 2 + aSeg[r] : oobA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(stage + (SH::ABLK * wave + r) * 1024), 16, oa, 0, 0,
                                               0);
    }
  }

  __device__ __forceinline__ void issue(const DgArgs& g, int kc, char* stage) const {
    const int n0 = kc * DG_TN;
#pragma unroll
    for (int r = 0; r < SH::ABLK; ++r) {
      const uint32_t oa = (aOk[r] && n0 + (int)(aSeg[r] >> 1) < g.N) ? aTok[r] + (uint32_t)n0 * 2 + aSeg[r] : oobA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(stage + (SH::ABLK * wave + r) * 1024), 16, oa, 0, 0,
                                               0);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int n = n0 + bRow[r];
      const uint32_t ob = (bOk[r] && n < g.N) ? (uint32_t)n * (uint32_t)(g.ldw * 2) + bCol[r] : oobB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(stage + SH::APB + (2 * wave + r) * 1024), 16, ob, 0,
                                               0, 0);
    }
  }
};

__device__ __forceinline__ u32x4 ds_read_16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

// Wait until at most N LDS reads are outstanding; the k-step's fragments
// are threaded through the statement so that their uses stay after it.
template <int N>
__device__ __forceinline__ void dg_wait(u32x4 (&a)[2], u32x2 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]) : "i"(N));
}
template <int N>
__device__ __forceinline__ void dg_wait(u32x4 (&a)[1], u32x2 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]) : "i"(N));
}

}  // namespace

// Workgroup L of T goes to XCD L % 8 (round-robin dispatch).  Give XCD x the
// x-th contiguous block of the work order (token tile fastest, then feature
// tile, then split): with 8 splits each XCD's L2 then serves one split's
// slice of the reduction, read from HBM once; with fewer, each XCD holds a
// run of feature tiles for both token tiles.
__device__ __forceinline__ int xcd_work(int L, int T) {
  const int q = T >> 3, r = T & 7, x = L & 7, slot = L >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
}

// KG reduction groups of 4 waves per workgroup (at most 4: 1024 threads): group k takes the chunks
// k, k + KG, k + 2 KG, ... through a ring of its own (chunks past the end
// read zero, so every group runs the same iterations and barriers), and the
// groups' partial tiles are added through LDS in a fixed order.  KG = 2 and
// 4 serve the short-token layers, whose few tiles would otherwise leave one
// 4-wave workgroup per CU with every per-chunk latency exposed.
template <int TM, int S, int KG>
__global__ void __launch_bounds__(NT * KG, KG == 1 ? 2 : 1) k_dgrad_bf16(const DgArgs g) {
  static_assert(KG >= 1 && KG <= 4, "at most 1024 threads per workgroup");
  using SH = DgShape<TM, S>;
  constexpr int BI = TM / 64;                        // 32-row MFMA blocks per wave
  constexpr int RINGS = KG * S * SH::STAGE;
  __shared__ __attribute__((aligned(16))) char lds[RINGS > SH::LDS ? RINGS : SH::LDS];
  // W panels are shared by the token tiles of one column: those run together
  const int tiles_m = (g.BT + TM - 1) / TM, tiles = tiles_m * ((g.K + TILE - 1) / TILE);
  const int w = xcd_work((int)blockIdx.x, (int)gridDim.x);
  const int tile = w % tiles, sp = w / tiles;
  const int tj = tile / tiles_m, ti = tile - tj * tiles_m;
  const int tok0 = ti * TM, col0 = tj * TILE;
  const int kg = (int)threadIdx.x / NT, gtid = (int)threadIdx.x - kg * NT;
  const int lane = gtid & 63, wave = gtid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  char* ring = lds + kg * S * SH::STAGE;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)ring;
  f32x16 acc[BI][2];
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  const int nk = (g.N + DG_TN - 1) / DG_TN;
  // this workgroup's chunks: c0 + kg + KG j, j < nj (a split range only with KG = 1)
  const int cps = (nk + g.splits - 1) / g.splits;
  const int c0 = KG == 1 ? sp * cps : 0;
  const int nj = KG == 1 ? max(0, min(cps, nk - c0)) : (nk + KG - 1) / KG;
  // this lane's fragment offsets within a stage: dY rows m(bi), 16-byte
  // segment 2 ks + lane / 32 (its swizzle differs between the two k-steps);
  // W (the weight-gradient mainloop's transposing-read fragments) per
  // 32-column block bj, the hi half 4 rows = 1024 bytes and the second
  // k-step 16 rows = 4096 bytes on
  uint32_t aofs[2][BI], bofs[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int bi = 0; bi < BI; ++bi) aofs[ks][bi] = dg_a_off(wr * (TM / 2) + bi * 32 + (lane & 31), 2 * ks + (lane >> 5));
  {
    const int t = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int f = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) bofs[bj] = (uint32_t)(SH::APB + MainBF16::off(t, wc * 64 + bj * 32 + f));
  }
  DgradLoader<TM, S> ld;
  ld.init(g, tok0, col0, gtid);
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (k < nj) ld.issue(g, c0 + kg + KG * k, ring + k * SH::STAGE);
  for (int j = 0; j < nj; ++j) {
    dg_wait_ahead<SH::LOADS, S - 2>(min(S - 2, nj - 1 - j));   // chunk j of this group landed
    bar();
    if (j + S - 1 < nj) ld.issue(g, c0 + kg + KG * (j + S - 1), ring + ((j + S - 1) % S) * SH::STAGE);
    const uint32_t cur = lds0 + (uint32_t)((j % S) * SH::STAGE);
    // both k-steps' fragments are requested first; the first k-step's MFMAs
    // run while the second's reads land
    u32x4 af[2][BI];
    u32x2 bf[2][4];
    uint32_t pb[2];
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) pb[bj] = cur + bofs[bj];
#pragma unroll
    for (int bi = 0; bi < BI; ++bi) af[0][bi] = ds_read_16(cur + aofs[0][bi]);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      bf[0][2 * bj] = tr_read_at<0>(pb[bj]);
      bf[0][2 * bj + 1] = tr_read_at<1024>(pb[bj]);
    }
#pragma unroll
    for (int bi = 0; bi < BI; ++bi) af[1][bi] = ds_read_16(cur + aofs[1][bi]);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      bf[1][2 * bj] = tr_read_at<4096>(pb[bj]);
      bf[1][2 * bj + 1] = tr_read_at<5120>(pb[bj]);
    }
    dg_wait<BI + 4>(af[0], bf[0]);
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[0][bi]),
                                                              frag_join(bf[0][2 * bj], bf[0][2 * bj + 1]),
                                                              acc[bi][bj], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // the wait below stays after these MFMAs
    dg_wait<0>(af[1], bf[1]);
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[1][bi]),
                                                              frag_join(bf[1][2 * bj], bf[1][2 * bj + 1]),
                                                              acc[bi][bj], 0, 0, 0);
  }
  wait_vmcnt<0>();
  bar();
  // lane l, register 4j+i of a 32 x 32 block holds row 8j + 4(l/32) + i, column l % 32
  float* sG = reinterpret_cast<float*>(lds);
  auto g_at = [&](int bi, int bj, int e) -> float& {
    const int r = wr * (TM / 2) + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    const int c = wc * 64 + bj * 32 + (lane & 31);
    return sG[r * SH::GP_ + c];
  };
  // group 0's partial + group 1's + ... in that order, through LDS
  for (int k = 1; k < KG; ++k) {
    if (kg == k) {
#pragma unroll
      for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int e = 0; e < 16; ++e) g_at(bi, bj, e) = acc[bi][bj][e];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[bi][bj][e] = acc[bi][bj][e] + g_at(bi, bj, e);
    }
    __syncthreads();
  }
  // stage the fp32 tile
  if (kg == 0) {
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 16; ++e) g_at(bi, bj, e) = acc[bi][bj][e];
  }
  __syncthreads();
  if (kg != 0) return;
  // write out: pass s, thread t -> row s*16 + t/16, two 4-column segments 64
  // apart; a split writes its fp32 partial to its [BT, K] slice of ws
  const int cl = 4 * (gtid & 15);
  const bool part = g.splits > 1;
  const bool vec = part || g.vec_out != 0;
  const int ofmt = part ? FMT_F32 : g.dx_fmt;
#pragma unroll
  for (int s = 0; s < TM / 16; ++s) {
    const int rl = s * 16 + (gtid >> 4);
    const int p = tok0 + rl;
    if (p >= g.BT) continue;
    char* rowp = part ? reinterpret_cast<char*>(g.ws + ((int64_t)sp * g.BT + p) * g.K)
                      : static_cast<char*>(g.dX) + (int64_t)p * g.ldx * (g.dx_fmt == FMT_F32 ? 4 : 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Seg sg;
      sg.q = col0 + 64 * h + cl;
      sg.nv = max(0, min(4, g.K - sg.q));
      sg.ok = sg.nv > 0;
      if (!sg.ok) continue;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sG[rl * SH::GP_ + 64 * h + cl + i];
      if (ofmt == FMT_F32) st4<FMT_F32, false>(rowp + (int64_t)sg.q * 4, sg, vec, x, 0, 0, 0);
      else st4<FMT_BF16, false>(rowp + (int64_t)sg.q * 2, sg, vec, x, 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// k_dgrad_wide (split path, long reduction): one 256 x 256 tile of dX per
// workgroup of 8 waves in a 2 x 4 arrangement of 128 tokens x 64 features
// (8 accumulator blocks per wave, two waves per SIMD, one workgroup per CU),
// the shape of the weight-gradient wide kernel.  Per 32-element reduction
// chunk a stage holds dY's 256 token rows x 64 B (swizzled in 16-byte units,
// dg_a_off) and W's 32 rows x 256 columns (the weight-gradient layout, read
// with the transposing LDS read): 32 KiB, 4 stages.  Per token and feature
// the tile moves half the L2 -> LDS bytes of the 128 x 128 tile.  Splits of
// the reduction write fp32 partials, which k_dgrad_reduce adds in split order.
// ---------------------------------------------------------------------------
namespace {
constexpr int DW_W = 256;                  // tile edge: tokens x features
constexpr int DW_S = 4;                    // ring stages (3 chunks in flight)
constexpr int DW_NW = 8;                   // waves
constexpr int DW_APB = DW_W * DG_TN * 2;   // dY's chunk: 256 token rows x 64 B = 16 KiB
constexpr int DW_BROWB = DW_W * 2;         // a row of W's chunk: 256 features
constexpr int DW_BPB = DG_TN * DW_BROWB;   // 16 KiB
constexpr int DW_STAGE = DW_APB + DW_BPB;
constexpr int DW_LOADS = 4;                // buffer loads per thread per chunk (2 dY, 2 W)
static_assert(DW_S * DW_STAGE <= 160 * 1024, "one workgroup per CU");

// byte offset of (row t, feature f) in W's chunk region, 64-byte XOR swizzle
__device__ __forceinline__ uint32_t dw_b_off(int t, int f) {
  return (uint32_t)(t * DW_BROWB + ((f * 2) ^ ((t & 3) << 6)));
}

template <int OFF>
__device__ __forceinline__ u32x4 ds_read_16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

template <int N>
__device__ __forceinline__ void dw_wait(u32x4 (&a)[4], u32x2 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
               : "i"(N));
}

// The fragments of one k-step: dY blocks bi (16-byte reads at 32-row =
// 2048-byte steps from pa), W blocks bj (transposing reads, hi half 4 rows =
// 2048 bytes on, the second k-step 16 rows = 8192 bytes on).
template <int KS>
__device__ __forceinline__ void dw_reads(uint32_t pa, uint32_t pb0, uint32_t pb1, u32x4 (&a)[4], u32x2 (&b)[4]) {
  a[0] = ds_read_16_at<0>(pa);
  a[1] = ds_read_16_at<2048>(pa);
  a[2] = ds_read_16_at<4096>(pa);
  a[3] = ds_read_16_at<6144>(pa);
  b[0] = tr_read_at<8192 * KS>(pb0);
  b[1] = tr_read_at<8192 * KS + 2048>(pb0);
  b[2] = tr_read_at<8192 * KS>(pb1);
  b[3] = tr_read_at<8192 * KS + 2048>(pb1);
}

__device__ __forceinline__ void dw_mfma(f32x16 (&acc)[4][2], const u32x4 (&a)[4], const u32x2 (&b)[4]) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[bi]),
                                                            frag_join(b[2 * bj], b[2 * bj + 1]), acc[bi][bj], 0, 0,
                                                            0);
}
}  // namespace

__global__ void __launch_bounds__(DW_NW * 64, 1) k_dgrad_wide(const DgArgs g) {
  __shared__ __attribute__((aligned(16))) char lds[DW_S * DW_STAGE];
  const int tiles_m = (g.BT + DW_W - 1) / DW_W, tiles_n = (g.K + DW_W - 1) / DW_W;
  const int w = xcd_work((int)blockIdx.x, (int)gridDim.x);
  const int tile = w % (tiles_m * tiles_n), sp = w / (tiles_m * tiles_n);
  const int tj = tile / tiles_m, ti = tile - tj * tiles_m;
  const int tok0 = ti * DW_W, col0 = tj * DW_W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 2, wc = wave & 3;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)lds;
  f32x16 acc[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
  // this split's chunks: [c0, c0 + nj)
  const int nk = (g.N + DG_TN - 1) / DG_TN;
  const int cps = (nk + g.splits - 1) / g.splits;
  const int c0 = sp * cps;
  const int nj = max(0, min(cps, nk - c0));
  // loads: instruction (wave, r) fills KiB NW r + wave of each region;
  // dY: 16 token rows x 4 segments per KiB, W: 2 rows x 32 chunks of 8 features
  const uint32_t oobA = (uint32_t)((uint64_t)g.BT * g.lddy * 2);
  const uint32_t oobB = (uint32_t)((uint64_t)g.N * g.ldw * 2);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.dY, oobA), rB = make_rsrc(g.W, oobB);
  uint32_t aTok[2], aSeg[2], bCol[2];
  int bRow[2];
  bool aOk[2], bOk[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int blk = DW_NW * r + wave;
    const int m = blk * 16 + (lane >> 2);
    const int sgl = (lane & 3) ^ ((m >> 2) & 3);        // logical 16-byte segment stored at this slot
    aOk[r] = tok0 + m < g.BT;
    aTok[r] = (uint32_t)((uint64_t)(tok0 + m) * g.lddy * 2);
    aSeg[r] = (uint32_t)(sgl * 16);
    const int t = blk * 2 + (lane >> 5);
    const int c = (lane & 31) ^ ((t & 3) << 2);          // logical 8-feature chunk stored at this slot
    bRow[r] = t;
    bOk[r] = col0 + c * 8 < g.K;
    bCol[r] = (uint32_t)(col0 + c * 8) * 2;
  }
  const auto issue = [&](int kc, char* stage) {
    const int n0 = kc * DG_TN;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t oa = (aOk[r] && n0 + (int)(aSeg[r] >> 1) < g.N) ? aTok[r] + (uint32_t)n0 * 2 + aSeg[r] : oobA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(stage + (DW_NW * r + wave) * 1024), 16, oa, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int n = n0 + bRow[r];
      const uint32_t ob = (bOk[r] && n < g.N) ? (uint32_t)n * (uint32_t)(g.ldw * 2) + bCol[r] : oobB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(stage + DW_APB + (DW_NW * r + wave) * 1024), 16, ob,
                                               0, 0, 0);
    }
  };
  // this lane's fragment offsets within a stage: dY rows wr 128 + lane % 32
  // (+ 32 bi), 16-byte segment 2 ks + lane / 32 (its swizzle differs between
  // the k-steps); W as in the weight-gradient mainloop, per 32-feature block bj
  uint32_t aofs[2], bofs[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) aofs[ks] = dg_a_off(wr * 128 + (lane & 31), 2 * ks + (lane >> 5));
  {
    const int t = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int f = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) bofs[bj] = DW_APB + dw_b_off(t, wc * 64 + bj * 32 + f);
  }
#pragma unroll
  for (int k = 0; k < DW_S - 1; ++k)
    if (k < nj) issue(c0 + k, lds + k * DW_STAGE);
  for (int j = 0; j < nj; ++j) {
    dg_wait_ahead<DW_LOADS, DW_S - 2>(min(DW_S - 2, nj - 1 - j));   // chunk j landed
    bar();                                                          // ... for all waves; stage j - 1 free
    if (j + DW_S - 1 < nj) issue(c0 + j + DW_S - 1, lds + ((j + DW_S - 1) % DW_S) * DW_STAGE);
    const uint32_t cur = lds0 + (uint32_t)((j % DW_S) * DW_STAGE);
    u32x4 a0[4], a1[4];
    u32x2 b0[4], b1[4];
    const uint32_t pb0 = cur + bofs[0], pb1 = cur + bofs[1];
    dw_reads<0>(cur + aofs[0], pb0, pb1, a0, b0);
    dw_reads<1>(cur + aofs[1], pb0, pb1, a1, b1);
    dw_wait<8>(a0, b0);
    dw_mfma(acc, a0, b0);
    __builtin_amdgcn_sched_barrier(0);   // the wait below stays after these MFMAs
    dw_wait<0>(a1, b1);
    dw_mfma(acc, a1, b1);
  }
  wait_vmcnt<0>();
  // lane l, register 4j + i of a 32 x 32 block holds row 8j + 4 (l / 32) + i,
  // column l % 32: 32 lanes store 32 consecutive columns of a row
  const bool part = g.splits > 1;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = tok0 + wr * 128 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = col0 + wc * 64 + bj * 32 + (lane & 31);
        if (tok >= g.BT || col >= g.K) continue;
        const float x = acc[bi][bj][e];
        if (part) g.ws[((int64_t)sp * g.BT + tok) * g.K + col] = x;
        else if (g.dx_fmt == FMT_F32) static_cast<float*>(g.dX)[(int64_t)tok * g.ldx + col] = x;
        else static_cast<uint16_t*>(g.dX)[(int64_t)tok * g.ldx + col] = (uint16_t)bf16_rne_bits(x);
      }
}

// dX = sum over s = 0 .. splits - 1 (at most 8) of ws[s] (in that order), 4 elements per
// thread (K % 8 == 0 on the split path: a 4-element group never crosses a row).
__global__ void __launch_bounds__(NT) k_dgrad_reduce(const DgArgs g) {
  const int64_t n4 = (int64_t)g.BT * g.K / 4;
  const int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (q >= n4) return;
  const f32x4* ws = reinterpret_cast<const f32x4*>(g.ws);
  f32x4 acc = ws[q];
  for (int s = 1; s < g.splits; ++s) {
    const f32x4 t = ws[(int64_t)s * n4 + q];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = acc[i] + t[i];
  }
  const int64_t e = 4 * q;
  const int p = (int)(e / g.K);
  Seg sg;
  sg.q = (int)(e - (int64_t)p * g.K);
  sg.nv = 4;
  sg.ok = true;
  float x[4] = {acc[0], acc[1], acc[2], acc[3]};
  const bool vec = g.vec_out != 0;
  char* rowp = static_cast<char*>(g.dX) + (int64_t)p * g.ldx * (g.dx_fmt == FMT_F32 ? 4 : 2);
  if (g.dx_fmt == FMT_F32) st4<FMT_F32, false>(rowp + (int64_t)sg.q * 4, sg, vec, x, 0, 0, 0);
  else st4<FMT_BF16, false>(rowp + (int64_t)sg.q * 2, sg, vec, x, 0, 0, 0);
}

namespace {
constexpr int DGG_T = 64;    // output tile edge of the generic kernel
constexpr int DGG_R = 16;    // reduction elements per step

__device__ __forceinline__ float ld_elem(const void* base, int fmt, int64_t i) {
  if (fmt == FMT_F32) return static_cast<const float*>(base)[i];
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
}

// W[n][col] as the step stores it: an E4M3 weight decodes to
// fp32(E4M3 value of the code * its block's scale), exactly the value the
// fused step reads back.
__device__ __forceinline__ float ld_w(const DgArgs& g, int n, int col) {
  const int64_t i = (int64_t)n * g.ldw + col;
  if (g.w_fmt == FMT_E4M3) {
    const int code = (int)static_cast<const uint8_t*>(g.W)[i];
    const float v = __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0];
    const int bsh = __builtin_ctz((unsigned)g.wblock);
    return v * g.wsc[(int64_t)n * (g.K >> bsh) + (col >> bsh)];
  }
  return ld_elem(g.W, g.w_fmt, i);
}
}  // namespace

__global__ void __launch_bounds__(NT) k_dgrad_generic(const DgArgs g) {
  __shared__ float sa[DGG_R][DGG_T + 1];   // dY^T chunk: [reduction][token]
  __shared__ float sb[DGG_R][DGG_T + 1];   // W chunk: [reduction][column]
  const int tiles_k = (g.K + DGG_T - 1) / DGG_T;
  const int ti = (int)blockIdx.x / tiles_k, tj = (int)blockIdx.x - ti * tiles_k;
  const int tok0 = ti * DGG_T, col0 = tj * DGG_T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // 16 x 16 threads, 4 x 4 outputs each
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int n0 = 0; n0 < g.N; n0 += DGG_R) {
    for (int e = threadIdx.x; e < DGG_R * DGG_T; e += NT) {
      const int r = e / DGG_T, c = e - r * DGG_T;
      const int n = n0 + r;
      const int tok = tok0 + c, col = col0 + c;
      sa[r][c] = (n < g.N && tok < g.BT) ? ld_elem(g.dY, g.in_fmt, (int64_t)tok * g.lddy + n) : 0.f;
      sb[r][c] = (n < g.N && col < g.K) ? ld_w(g, n, col) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < DGG_R; ++r) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sa[r][ty * 4 + i];
        b[i] = sb[r][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = tok0 + ty * 4 + i;
    if (tok >= g.BT) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = col0 + tx * 4 + j;
      if (col >= g.K) continue;
      const int64_t o = (int64_t)tok * g.ldx + col;
      if (g.dx_fmt == FMT_F32) static_cast<float*>(g.dX)[o] = acc[i][j];
      else static_cast<uint16_t*>(g.dX)[o] = (uint16_t)bf16_rne_bits(acc[i][j]);
    }
  }
}

// ------------------------------------------------------------------------
// dX from an E4M3 weight with block scales on the matrix cores.  Each chunk
// of 16 reduction elements is staged in LDS as fp32: dY widened from bf16
// (exact), the weight decoded exactly to the value the step stores (E4M3
// value of the code x its block's scale, one fp32 product); then
// v_mfma_f32_32x32x2_f32 accumulates in fp32, a sum of fp32 products in a
// fixed order per element (within the fp32 summation bound like the plain
// kernel).  One TM x 128 dX tile per 256-thread workgroup (TM = 64: 4 waves
// in a 2 x 2 arrangement of 32 x 64; TM = 32, when 64-token tiles would not
// give every CU two workgroups: 1 x 4 of 32 x 32), register-staged double
// buffering.  LDS rows are padded so that the two half-waves of a fragment
// read (reduction rows k and k + 1) fall 32 banks apart.  bf16 dY, any
// leading dimensions, ragged BT, N and K (K a multiple of the block, >= 32).
// ------------------------------------------------------------------------
namespace {
constexpr int F8_TN = 128, F8_R = 16;
constexpr int F8_BP = 160;                 // LDS row pitch of W's chunk in floats (rows k, k + 1: 32 banks apart)

// TM-token tiles (64 or 32): waves in a (TM / 32) x (4 / (TM / 32)) arrangement of 32-token parts.
template <int TM>
struct Fp8wShape {
  static constexpr int WR = TM / 32;                 // wave rows
  static constexpr int WCN = 4 / WR;                 // wave columns
  static constexpr int BJ = F8_TN / (32 * WCN);      // 32-column blocks per wave
  static constexpr int AE = TM * F8_R / NT;          // dY elements staged per thread (4 or 2)
  static constexpr int AP = TM % 64 == 32 ? TM : TM + 32;   // LDS row pitch of dY's chunk: 32 banks mod 64
};

template <int TM>
struct Fp8wStage {
  float a[Fp8wShape<TM>::AE];   // dY[tok][n .. n + AE - 1] of this thread, widened
  float b[8];                   // W[n][col .. col + 7] of this thread, decoded
};

template <int TM>
__device__ __forceinline__ void f8_load(const DgArgs& g, int tok0, int col0, int n0, Fp8wStage<TM>& st) {
  using SH = Fp8wShape<TM>;
  constexpr int PER = F8_R / SH::AE;                 // threads per token row
  const int t = threadIdx.x;
  {   // dY: token row t / PER, reduction elements AE (t % PER) ..
    const int tok = tok0 + t / PER, n = n0 + SH::AE * (t % PER);
    const uint16_t* p = static_cast<const uint16_t*>(g.dY) + (int64_t)tok * g.lddy + n;
#pragma unroll
    for (int i = 0; i < SH::AE; ++i)
      st.a[i] = (tok < g.BT && n + i < g.N) ? __uint_as_float((uint32_t)p[i] << 16) : 0.f;
  }
  {   // W: reduction row t / 16, columns 8 (t % 16) .. + 7 (one block: the block is >= 32)
    const int n = n0 + (t >> 4), col = col0 + 8 * (t & 15);
    if (n < g.N && col < g.K) {
      const uint8_t* p = static_cast<const uint8_t*>(g.W) + (int64_t)n * g.ldw + col;
      uint32_t w0, w1;
      if ((reinterpret_cast<uintptr_t>(p) & 7) == 0) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
        w0 = w[0];
        w1 = w[1];
      } else {
        w0 = p[0] | (p[1] << 8) | (p[2] << 16) | ((uint32_t)p[3] << 24);
        w1 = p[4] | (p[5] << 8) | (p[6] << 16) | ((uint32_t)p[7] << 24);
      }
      const int bsh = __builtin_ctz((unsigned)g.wblock);
      const float sc = g.wsc[(int64_t)n * (g.K >> bsh) + (col >> bsh)];
      e4m3_unpack4(w0, st.b);
      e4m3_unpack4(w1, st.b + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.b[i] *= sc;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) st.b[i] = 0.f;
    }
  }
}

template <int TM>
__device__ __forceinline__ void f8_store(const Fp8wStage<TM>& st, float* sA, float* sB) {
  using SH = Fp8wShape<TM>;
  constexpr int PER = F8_R / SH::AE;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < SH::AE; ++i) sA[(SH::AE * (t % PER) + i) * SH::AP + t / PER] = st.a[i];
  float* b = sB + (t >> 4) * F8_BP + 8 * (t & 15);
  *reinterpret_cast<f32x4*>(b) = f32x4{st.b[0], st.b[1], st.b[2], st.b[3]};
  *reinterpret_cast<f32x4*>(b + 4) = f32x4{st.b[4], st.b[5], st.b[6], st.b[7]};
}
}  // namespace

template <int TM>
__global__ void __launch_bounds__(NT) k_dgrad_fp8w(const DgArgs g) {
  using SH = Fp8wShape<TM>;
  __shared__ __attribute__((aligned(16))) float sA[2][F8_R * SH::AP];
  __shared__ __attribute__((aligned(16))) float sB[2][F8_R * F8_BP];
  const int tiles_k = (g.K + F8_TN - 1) / F8_TN;
  const int ti = (int)blockIdx.x / tiles_k, tj = (int)blockIdx.x - ti * tiles_k;
  const int tok0 = ti * TM, col0 = tj * F8_TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave / SH::WCN, wc = wave % SH::WCN;
  f32x16 acc[SH::BJ];
#pragma unroll
  for (int bj = 0; bj < SH::BJ; ++bj)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[bj][e] = 0.f;
  const int nk = (g.N + F8_R - 1) / F8_R;
  Fp8wStage<TM> st;
  if (nk > 0) {
    f8_load<TM>(g, tok0, col0, 0, st);
    f8_store<TM>(st, sA[0], sB[0]);
  }
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    if (kc + 1 < nk) f8_load<TM>(g, tok0, col0, (kc + 1) * F8_R, st);
    const float* A = sA[cur];
    const float* B = sB[cur];
#pragma unroll
    for (int kk = 0; kk < F8_R / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      const float fa = A[k * SH::AP + wr * 32 + (lane & 31)];
#pragma unroll
      for (int bj = 0; bj < SH::BJ; ++bj) {
        const float fb = B[k * F8_BP + wc * (32 * SH::BJ) + bj * 32 + (lane & 31)];
        acc[bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa, fb, acc[bj], 0, 0, 0);
      }
    }
    if (kc + 1 < nk) f8_store<TM>(st, sA[cur ^ 1], sB[cur ^ 1]);
    __syncthreads();
  }
  // lane l, register 4j + i of a 32 x 32 block: row 8j + 4(l / 32) + i, column l % 32
#pragma unroll
  for (int bj = 0; bj < SH::BJ; ++bj)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tok = tok0 + wr * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int col = col0 + wc * (32 * SH::BJ) + bj * 32 + (lane & 31);
      if (tok >= g.BT || col >= g.K) continue;
      const int64_t o = (int64_t)tok * g.ldx + col;
      if (g.dx_fmt == FMT_F32) static_cast<float*>(g.dX)[o] = acc[bj][e];
      else static_cast<uint16_t*>(g.dX)[o] = (uint16_t)bf16_rne_bits(acc[bj][e]);
    }
}

// ---------------------------------------------------------------------------
// k_dgrad_fp8w3<TM> (bf16 dY with 16-byte aligned rows and N % 8 == 0, E4M3
// W with 16-byte aligned rows and K % 16 == 0, fp32 block scales): dX on the
// bf16 matrix cores.  A weight element decodes to w = fp32(code * scale),
// the value the fused step reads back, and w splits exactly into three bf16
// terms: h = w with its low 16 bits cleared, m = (w - h) likewise, l =
// w - h - m (8 significant bits each; every subtraction is exact).  So dX =
// dY h + dY m + dY l with exact products and fp32 accumulation: three MFMAs
// per fragment pair, the fp32 kernel's work at the bf16 rate.  Tiles of TM
// tokens x 128 columns; 4 waves side by side, each all TM tokens x 32
// columns.  Per 32-row chunk a ring stage holds dY's chunk (as
// k_dgrad_bf16), W's raw 32 x 128 bytes (16-byte segments XOR-swizzled by
// row) and the chunk's scales (block-major), all by buffer_load ... lds.
// Each lane takes its B fragment's 8 codes (8 rows of one column) with the
// 8-bit transposing LDS read and its 8 rows' scales, and forms the three
// bf16 fragments in registers.  KG reduction groups of 4 waves (each its
// own ring, chunks g, g + KG, ...) are added through LDS in a fixed order at
// the end: KG = 2 for 64-token tiles, whose few workgroups would otherwise
// leave one 4-wave workgroup per CU.
// ---------------------------------------------------------------------------
namespace {
constexpr int F3_S = 4;                       // ring stages
template <int TM>
struct F3Shape {
  static constexpr int APB = TM * DG_TN * 2;  // dY's chunk
  static constexpr int RAW = APB;             // W's chunk, 32 rows x 128 bytes
  static constexpr int SCL = RAW + 4096;      // its scales: slot b * 32 + r (block b of the tile, row r);
  static constexpr int STAGE = SCL + 1024;    // 256 slots, 64 loaded by each wave (slots past 4 blocks read zero)
  static constexpr int LOADS = TM / 64 + 2;   // buffer loads per wave per chunk
};
static_assert(2 * F3_S * F3Shape<128>::STAGE <= 160 * 1024, "two workgroups per CU");

// the high halves of two fp32 patterns as one bf16 pair (a low, b high)
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// LDS accesses of this kernel are written out (the buffer_load ... lds
// writes are invisible to the compiler's own wait insertion); every read's
// result is threaded through an explicit wait before its use.
template <int OFF>
__device__ __forceinline__ u32x2 tr8_read_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// The three bf16 fragments of 8 codes (rows k .. k + 7 of one column) with
// the scales of those rows.
__device__ __forceinline__ void f3_split8(u32x2 raw, const float (&sc)[8], bf16x8 (&t)[3]) {
  float x[8];
  e4m3_unpack4(raw[0], x);
  e4m3_unpack4(raw[1], x + 4);
  uint32_t hb[8], mb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = x[e] * sc[e];                           // fp32(code * scale)
    hb[e] = __float_as_uint(v) & 0xFFFF0000u;
    const float r1 = v - __uint_as_float(hb[e]);
    mb[e] = __float_as_uint(r1) & 0xFFFF0000u;
    lb[e] = __float_as_uint(r1 - __uint_as_float(mb[e]));  // low 16 bits zero
  }
  t[0] = __builtin_bit_cast(bf16x8, u32x4{hi_pair(hb[0], hb[1]), hi_pair(hb[2], hb[3]), hi_pair(hb[4], hb[5]),
                                          hi_pair(hb[6], hb[7])});
  t[1] = __builtin_bit_cast(bf16x8, u32x4{hi_pair(mb[0], mb[1]), hi_pair(mb[2], mb[3]), hi_pair(mb[4], mb[5]),
                                          hi_pair(mb[6], mb[7])});
  t[2] = __builtin_bit_cast(bf16x8, u32x4{hi_pair(lb[0], lb[1]), hi_pair(lb[2], lb[3]), hi_pair(lb[4], lb[5]),
                                          hi_pair(lb[6], lb[7])});
}

// One k-step's operands: dY's BI fragments, the B codes, the 8 scales.
template <int BI>
struct F3Frag {
  u32x4 a[BI];
  u32x2 raw;
  u32x4 s0, s1;
};
template <int KS, int BI>
__device__ __forceinline__ void f3_reads(uint32_t cur, const uint32_t (&aofs)[2][BI], uint32_t braw, uint32_t bscl,
                                         F3Frag<BI>& f) {
#pragma unroll
  for (int bi = 0; bi < BI; ++bi) f.a[bi] = ds_read_16(cur + aofs[KS][bi]);
  f.raw = tr8_read_at<KS * 2048>(cur + braw);
  f.s0 = ds_read_16_at<KS * 64>(cur + bscl);
  f.s1 = ds_read_16_at<KS * 64 + 16>(cur + bscl);
}
template <int N, int BI>
__device__ __forceinline__ void f3_wait(F3Frag<BI>& f) {
  if constexpr (BI == 2)
    asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.raw), "+v"(f.s0), "+v"(f.s1) : "i"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%7)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.raw), "+v"(f.s0), "+v"(f.s1)
                 : "i"(N));
}
template <int BI>
__device__ __forceinline__ void f3_mfma(f32x16 (&acc)[BI], const F3Frag<BI>& f) {
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = __uint_as_float(f.s0[i]);
    sc[4 + i] = __uint_as_float(f.s1[i]);
  }
  bf16x8 t[3];
  f3_split8(f.raw, sc, t);
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
      acc[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[bi]), t[k], acc[bi], 0, 0, 0);
}
}  // namespace

template <int TM, int KG>
__global__ void __launch_bounds__(NT * KG, 2) k_dgrad_fp8w3(const DgArgs g) {
  using SH = F3Shape<TM>;
  constexpr int S = F3_S, BI = TM / 32;
  static_assert(BI == 2 || BI == 4, "64- or 128-token tiles");
  static_assert(KG == 1 || KG * S * SH::STAGE >= TM * TILE * 4, "the groups' partial tiles fit the rings");
  __shared__ __attribute__((aligned(16))) char lds[KG * S * SH::STAGE];
  const int tiles_m = (g.BT + TM - 1) / TM;
  const int w = xcd_work((int)blockIdx.x, (int)gridDim.x);
  const int tj = w / tiles_m, ti = w - tj * tiles_m;
  const int tok0 = ti * TM, col0 = tj * TILE;
  const int kg = (int)threadIdx.x / NT, tid = (int)threadIdx.x - kg * NT, lane = tid & 63, wave = tid >> 6;
  char* const ring = lds + kg * S * SH::STAGE;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)ring;
  f32x16 acc[BI];
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[bi][e] = 0.f;
  const int nk = (g.N + DG_TN - 1) / DG_TN;
  const int nj = (nk + KG - 1) / KG;   // this group's chunks kg + KG jj, jj < nj (past the end: zeros)
  DgradLoader<TM, S> ld;
  ld.init(g, tok0, col0, tid);
  // raw W: wave v, lane l -> row r = 8 v + l / 8 at 16-byte position
  // l % 8, holding the row's segment (l % 8) ^ (r % 8)
  const int bsh = __builtin_ctz((unsigned)g.wblock);
  const int bpt = TILE >> bsh;                              // blocks of the tile per row: 1, 2 or 4
  const int64_t spr = g.K >> bsh;                           // scales per row of W
  const uint32_t oobW = (uint32_t)((uint64_t)g.N * g.ldw);
  const uint32_t oobS = (uint32_t)((uint64_t)g.N * spr * 4);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W, oobW), rS = make_rsrc(g.wsc, oobS);
  const int wrow = 8 * wave + (lane >> 3);
  const int wcol = col0 + 16 * ((lane & 7) ^ (lane >> 3));
  const bool wOk = wcol < g.K;
  // scales: slot q = 64 v + l -> block q / 32 of the tile, row q % 32
  const int q = 64 * wave + lane, sblk = q >> 5, srow = q & 31;
  const bool sOk = sblk < bpt && (col0 >> bsh) + sblk < spr;
  const auto issue = [&](int kc, char* stage) {
    ld.issue_a(g, kc, stage);
    const int n = kc * DG_TN + wrow;
    const uint32_t ow = (wOk && n < g.N) ? (uint32_t)n * (uint32_t)g.ldw + (uint32_t)wcol : oobW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void*)(stage + SH::RAW + wave * 1024), 16, ow, 0, 0, 0);
    const int ns = kc * DG_TN + srow;
    const uint32_t os = (sOk && ns < g.N) ? (uint32_t)(((int64_t)ns * spr + (col0 >> bsh) + sblk) * 4) : oobS;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(stage + SH::SCL + wave * 256), 4, os, 0, 0, 0);
  };
  // fragment offsets within a stage.  dY: rows bi 32 + lane % 32, segment
  // 2 ks + lane / 32 (as k_dgrad_bf16).  B: in 16-lane group G = lane / 16
  // the 8-bit transposing read gives lane j byte b from byte j % 8 of the
  // 8 bytes that lane 2 b + j / 8 of the group addresses; lane s of the
  // group therefore addresses row 8 (lane / 32) + s / 2 (+ 16 in k-step 1),
  // columns 32 wave + 16 (G % 2) + 8 (s % 2) .. + 7, so that lane l gets
  // rows 8 (l / 32) .. + 7 of column 32 wave + l % 32: the MFMA's B layout.
  uint32_t aofs[2][BI];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int bi = 0; bi < BI; ++bi) aofs[ks][bi] = dg_a_off(bi * 32 + (lane & 31), 2 * ks + (lane >> 5));
  uint32_t braw, bscl;
  {
    const int sl = lane & 15, grp = lane >> 4;
    const int r = 8 * (lane >> 5) + (sl >> 1);
    const int c = 32 * wave + 16 * (grp & 1) + 8 * (sl & 1);
    braw = (uint32_t)(SH::RAW + r * 128 + ((((c >> 4) ^ (r & 7)) << 4) | (c & 15)));
    const int tb = (32 * wave + (lane & 31)) >> bsh;         // this lane's block of the tile
    bscl = (uint32_t)(SH::SCL + (tb * 32 + 8 * (lane >> 5)) * 4);
  }
  // every chunk issues its loads (past the end they read zero), so the
  // vector-memory counts are the same in every iteration
#pragma unroll
  for (int k = 0; k < S - 1; ++k) issue(kg + KG * k, ring + k * SH::STAGE);
  for (int j = 0; j < nj; ++j) {
    wait_vmcnt<(S - 2) * SH::LOADS>();   // chunk j landed (this wave's loads)
    bar();                               // ... every wave's; stage j - 1 free
    issue(kg + KG * (j + S - 1), ring + ((j + S - 1) % S) * SH::STAGE);
    const uint32_t cur = lds0 + (uint32_t)((j % S) * SH::STAGE);
    F3Frag<BI> f0, f1;
    f3_reads<0, BI>(cur, aofs, braw, bscl, f0);
    f3_reads<1, BI>(cur, aofs, braw, bscl, f1);
    f3_wait<BI + 3, BI>(f0);
    f3_mfma<BI>(acc, f0);
    __builtin_amdgcn_sched_barrier(0);
    f3_wait<0, BI>(f1);
    f3_mfma<BI>(acc, f1);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();
  if constexpr (KG > 1) {
    // group 0's partial + group 1's + ... in that order, through LDS
    // (lane l, register 4j + i of a 32 x 32 block: row 8j + 4 (l / 32) + i, column l % 32)
    float* sP = reinterpret_cast<float*>(lds);
    const auto at = [&](int bi, int e) -> float& {
      return sP[(bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * TILE + 32 * wave + (lane & 31)];
    };
    bar();   // every group's rings are idle
    for (int k = 1; k < KG; ++k) {
      if (kg == k) {
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
          for (int e = 0; e < 16; ++e) at(bi, e) = acc[bi][e];
      }
      __syncthreads();
      if (kg == 0) {
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[bi][e] = acc[bi][e] + at(bi, e);
      }
      __syncthreads();
    }
    if (kg != 0) return;
  }
  // lane l, register 4j + i of a 32 x 32 block holds row 8j + 4 (l / 32) + i, column l % 32
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tok = tok0 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int col = col0 + 32 * wave + (lane & 31);
      if (tok >= g.BT || col >= g.K) continue;
      const int64_t o = (int64_t)tok * g.ldx + col;
      if (g.dx_fmt == FMT_F32) static_cast<float*>(g.dX)[o] = acc[bi][e];
      else static_cast<uint16_t*>(g.dX)[o] = (uint16_t)bf16_rne_bits(acc[bi][e]);
    }
}

// fast (aligned operands): the bf16 matrix-core kernel, 128-token tiles when
// those give every CU a workgroup, else 64; otherwise the fp32 kernel, with
// 32-token tiles when 64-token tiles would not give every CU two workgroups.
hipError_t launch_dgrad_fp8w(const DgArgs& g, bool fast, hipStream_t st) {
  if (g.BT == 0 || g.K == 0) return hipSuccess;
  if (g.in_fmt != FMT_BF16 || g.w_fmt != FMT_E4M3 || g.wblock < 32) return launch_dgrad(g, false, st);
  if (fast) {
    const int64_t tk = (g.K + TILE - 1) / TILE;
    const int64_t t128 = ((g.BT + 127) / 128) * tk;
    if (t128 >= 256)
      hipLaunchKernelGGL((k_dgrad_fp8w3<128, 1>), dim3((unsigned)t128), dim3(NT), 0, st, g);
    else
      hipLaunchKernelGGL((k_dgrad_fp8w3<64, 2>), dim3((unsigned)(((g.BT + 63) / 64) * tk)), dim3(2 * NT), 0, st, g);
    return hipGetLastError();
  }
  const int64_t tk = (g.K + F8_TN - 1) / F8_TN;
  const int64_t t64 = ((g.BT + 63) / 64) * tk;
  if (t64 >= 512) {
    hipLaunchKernelGGL(k_dgrad_fp8w<64>, dim3((unsigned)t64), dim3(NT), 0, st, g);
  } else {
    hipLaunchKernelGGL(k_dgrad_fp8w<32>, dim3((unsigned)(((g.BT + 31) / 32) * tk)), dim3(NT), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_dgrad(const DgArgs& g, bool fast, hipStream_t st) {
  if (g.BT == 0 || g.K == 0) return hipSuccess;
  if (g.splits < 1 || g.splits > 8) return hipErrorInvalidValue;   // k_dgrad_reduce holds at most 8 partials
  if (fast) {
    // 128-token tiles, two workgroups per CU; when those would not give every
    // CU a workgroup (short token axis, few columns), 64-token tiles, up to
    // three workgroups per CU (measured: a deeper ring does not help them --
    // with 4 MFMAs per wave and chunk the per-chunk overhead dominates)
    const int64_t t128 = (int64_t)((g.BT + 127) / 128) * g.tiles_k;
    const int64_t t64 = (int64_t)((g.BT + 63) / 64) * g.tiles_k;
    if (g.splits > 1 && dgrad_plan(g.BT, g.N, g.K).wide) {
      const unsigned t256 = (unsigned)(((g.BT + DW_W - 1) / DW_W) * ((g.K + DW_W - 1) / DW_W));
      hipLaunchKernelGGL(k_dgrad_wide, dim3(t256 * (unsigned)g.splits), dim3(DW_NW * 64), 0, st, g);
      const int64_t n4 = (int64_t)g.BT * g.K / 4;
      hipLaunchKernelGGL(k_dgrad_reduce, dim3((unsigned)((n4 + NT - 1) / NT)), dim3(NT), 0, st, g);
    } else if (g.splits > 1) {
      hipLaunchKernelGGL((k_dgrad_bf16<128, 4, 1>), dim3((unsigned)t128 * (unsigned)g.splits), dim3(NT), 0, st, g);
      const int64_t n4 = (int64_t)g.BT * g.K / 4;
      hipLaunchKernelGGL(k_dgrad_reduce, dim3((unsigned)((n4 + NT - 1) / NT)), dim3(NT), 0, st, g);
    } else if (t128 >= 256) {
      hipLaunchKernelGGL((k_dgrad_bf16<128, 4, 1>), dim3((unsigned)t128), dim3(NT), 0, st, g);
    } else if (t64 < 512 && g.N >= 8 * DG_TN) {
      // the reduction in 4 groups of 4 waves (3-stage rings, 144 KiB of LDS)
      // up to 128 chunks, else in 2 (measured at BT 512: q / o_proj 33 -> 29
      // us with 4 groups, gate_proj unsplit 106 -> 110 us)
      if (g.N <= 128 * DG_TN)
        hipLaunchKernelGGL((k_dgrad_bf16<64, 3, 4>), dim3((unsigned)t64), dim3(4 * NT), 0, st, g);
      else
        hipLaunchKernelGGL((k_dgrad_bf16<64, 4, 2>), dim3((unsigned)t64), dim3(2 * NT), 0, st, g);
    } else {
      hipLaunchKernelGGL((k_dgrad_bf16<64, 4, 1>), dim3((unsigned)t64), dim3(NT), 0, st, g);
    }
  } else {
    const unsigned tiles = (unsigned)(((g.BT + DGG_T - 1) / DGG_T) * ((g.K + DGG_T - 1) / DGG_T));
    hipLaunchKernelGGL(k_dgrad_generic, dim3(tiles), dim3(NT), 0, st, g);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Allocation-free split dX (for callers that cannot allocate device memory):
// the fp32 partials go to this file-scope device array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy from the
// first use on that device until the process ends; its contents are left
// from the last call, which is harmless here because every split writes its
// whole [BT, K] slice before the reduction reads it.  Calls that overlap on
// one GPU share the array and race.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address is resolved once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to the kernels.
// ------------------------------------------------------------------------
static __device__ __align__(256) float scratch[DGRAD_SCRATCH_BYTES / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch` by device ordinal, once resolved

// The device address of this device's `scratch`, `dev` being the device the
// stream belongs to (the current device for the null stream).
hipError_t scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_dgrad_scratch(DgArgs g, bool fast, hipStream_t st) {
  if (fast && g.splits > 1) {
    if ((int64_t)g.splits * g.BT * g.K * 4 > (int64_t)DGRAD_SCRATCH_BYTES) return hipErrorInvalidValue;
    void* p = nullptr;
    const hipError_t e = scratch_address(st, &p);
    if (e != hipSuccess) return e;
    g.ws = static_cast<float*>(p);
  }
  return launch_dgrad(g, fast, st);
}

}  // namespace forge
