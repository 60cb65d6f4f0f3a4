// Kernels shared by every optimizer: the unfused baseline's GEMM (G to HBM)
// and the stochastic-rounding test hook.
#include "forge_device.h"

#include <algorithm>

namespace forge {

// The device stochastic rounding on its own, element i with flat index i:
// thread t rounds the pair 2t, 2t + 1 through the fused epilogue's pair
// function (its RNE half masked off); a last unpaired element uses the same
// function with a zero partner that is not stored.
__global__ void k_debug_sr(const float* __restrict__ in, uint16_t* __restrict__ out, uint32_t n, uint32_t key) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t i0 = 2ull * t;
  if (i0 >= n) return;
  const bool two = i0 + 1 < n;
  const uint32_t w = bf16x2_store(in[i0], two ? in[i0 + 1] : 0.f, 0xFFFFFFFFu, key, t * GOLDEN);
  out[i0] = (uint16_t)(w & 0xFFFFu);
  if (two) out[i0 + 1] = (uint16_t)(w >> 16);
}

// The device E4M3 rounding on its own, through the same four-value packing
// the fused epilogue uses: thread i encodes elements 4i .. 4i+3 (zeros past
// the end, which are not stored).
__global__ void k_debug_e4m3(const float* __restrict__ in, uint8_t* __restrict__ out, uint32_t n) {
  const uint64_t i0 = 4ull * (blockIdx.x * (uint64_t)blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  float y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = i0 + k < n ? in[i0 + k] : 0.f;
  const uint32_t w = e4m3_pack4(y[0], y[1], y[2], y[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) out[i0 + k] = (uint8_t)((w >> (8 * k)) & 0xFFu);
}

// The FP8 weight store's stochastic rounding on its own, through the same
// four-value packing: thread i rounds elements 4i .. 4i+3 with the SR bits
// of flat indices 4i .. 4i+3 under `key` (zeros past the end, not stored).
__global__ void k_debug_e4m3_sr(const float* __restrict__ in, uint8_t* __restrict__ out, uint32_t n, uint32_t key) {
  const uint64_t i0 = 4ull * (blockIdx.x * (uint64_t)blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  float y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = i0 + k < n ? in[i0 + k] : 0.f;
  // i0 is even: two hash pairs, as in the fused FP8 weight store
  const uint32_t jmul = (uint32_t)(i0 >> 1) * GOLDEN;
  const uint32_t h0 = sr_pair(key, jmul), h1 = sr_pair(key, jmul + GOLDEN);
  const uint32_t r[4] = {h0, h0 << 16, h1, h1 << 16};
  const uint32_t w = e4m3_sr_pack4(y, r);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) out[i0 + k] = (uint8_t)((w >> (8 * k)) & 0xFFu);
}

// Exhaustive check of the block quantiser's quotients: for every fp32 a in
// [2^-64, 2^126) and QMAX in {127, 255, 448}, quot_by_q(a) against the IEEE
// a / QMAX and q_by_quot(a) against the IEEE QMAX / a.  Workgroup b writes
// its mismatch counts (a/127, 127/a, a/255, 255/a, a/448, 448/a) and the
// number of a values it checked to counts[8 b .. 8 b + 6].
__global__ void __launch_bounds__(256) k_debug_quotients(unsigned long long* __restrict__ counts) {
  constexpr uint32_t LO = 0x1F800000u, HI = 0x7E800000u;   // 2^-64, 2^126
  __shared__ unsigned long long part[7];
  if (threadIdx.x < 7) part[threadIdx.x] = 0ull;
  __syncthreads();
  unsigned long long bad[6] = {0, 0, 0, 0, 0, 0}, seen = 0;
  const uint32_t stride = gridDim.x * blockDim.x;   // HI + stride < 2^32: no wrap
  for (uint32_t u = LO + blockIdx.x * blockDim.x + threadIdx.x; u < HI; u += stride) {
    const float a = __uint_as_float(u);
    ++seen;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float q = k == 0 ? 127.f : k == 1 ? 255.f : 448.f;
      const float rq = k == 0 ? 1.f / 127.f : k == 1 ? 1.f / 255.f : 1.f / 448.f;
      float qv = q;
      asm volatile("" : "+v"(qv));   // an opaque divisor: the division below is the IEEE one
      bad[2 * k] += __float_as_uint(quot_by_q(a, q, rq)) != __float_as_uint(a / qv);
      bad[2 * k + 1] += __float_as_uint(q_by_quot(q, a)) != __float_as_uint(qv / a);
    }
  }
#pragma unroll
  for (int k = 0; k < 6; ++k)
    if (bad[k]) atomicAdd(&part[k], bad[k]);
  atomicAdd(&part[6], seen);
  __syncthreads();
  if (threadIdx.x < 7) counts[8ull * blockIdx.x + threadIdx.x] = part[threadIdx.x];
}

// The fused epilogue's 8-bit block quantiser on its own: quantize_chunk with
// the epilogue's thread mapping (thread t of a 256-thread workgroup owns row
// t / 16 of a 16-row slab and the two 4-element segments at columns
// 4 (t % 16) and 64 + 4 (t % 16) of a 128-column tile).  in, codes: dense
// [rows, cols]; scales: dense [rows, cols / block].  cols % block == 0, so a
// segment is entirely inside or outside; rows past the end take no part.
template <int FMT, bool POSITIVE>
__global__ void __launch_bounds__(256) k_debug_quant(const float* __restrict__ in, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales, int rows, int cols, int block) {
  const int tiles_c = (cols + 127) / 128;
  const int rg = (int)blockIdx.x / tiles_c, ct = (int)blockIdx.x - rg * tiles_c;
  const int tid = threadIdx.x;
  const int p = rg * 16 + (tid >> 4);
  Seg sg[2];
  float x[8];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    sg[g].q = ct * 128 + 64 * g + 4 * (tid & 15);
    sg[g].nv = max(0, min(4, cols - sg[g].q));
    sg[g].ok = sg[g].nv > 0 && p < rows;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * g + i] = sg[g].ok ? in[(int64_t)p * cols + sg[g].q + i] : 0.f;
  }
  const int64_t prow = p < rows ? p : 0;   // a valid row for lanes that store nothing
  const int bsh = __builtin_ctz((unsigned)block);
  uint8_t* const cp[2] = {codes + prow * cols + sg[0].q, codes + prow * cols + sg[1].q};
  float* const sp[2] = {scales + prow * (cols / block) + (sg[0].q >> bsh),
                        scales + prow * (cols / block) + (sg[1].q >> bsh)};
  quantize_chunk<FMT, POSITIVE>(x, block, sg, cp, true, sp);
}

hipError_t launch_debug_quant(const float* in, uint8_t* codes, float* scales, int rows, int cols, int fmt,
                              bool positive, int block, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)(((rows + 15) / 16) * ((cols + 127) / 128))), b(256);
  if (fmt == FMT_S8 && !positive)
    hipLaunchKernelGGL((k_debug_quant<FMT_S8, false>), grid, b, 0, st, in, codes, scales, rows, cols, block);
  else if (fmt == FMT_U8 && positive)
    hipLaunchKernelGGL((k_debug_quant<FMT_U8, true>), grid, b, 0, st, in, codes, scales, rows, cols, block);
  else if (fmt == FMT_E4M3 && !positive)
    hipLaunchKernelGGL((k_debug_quant<FMT_E4M3, false>), grid, b, 0, st, in, codes, scales, rows, cols, block);
  else if (fmt == FMT_E4M3 && positive)
    hipLaunchKernelGGL((k_debug_quant<FMT_E4M3, true>), grid, b, 0, st, in, codes, scales, rows, cols, block);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_debug_e4m3_sr(const float* in, uint8_t* out, uint32_t n, uint32_t key, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t threads = (n + 3ull) / 4ull;
  hipLaunchKernelGGL(k_debug_e4m3_sr, dim3((unsigned)((threads + 255u) / 256u)), dim3(256), 0, st, in, out, n, key);
  return hipGetLastError();
}

hipError_t launch_debug_quotients(unsigned long long* counts, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_quotients, dim3(QUOTIENT_CHECK_BLOCKS), dim3(256), 0, st, counts);
  return hipGetLastError();
}

hipError_t launch_debug_e4m3(const float* in, uint8_t* out, uint32_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t threads = (n + 3ull) / 4ull;
  hipLaunchKernelGGL(k_debug_e4m3, dim3((unsigned)((threads + 255u) / 256u)), dim3(256), 0, st, in, out, n);
  return hipGetLastError();
}

// Streaming ceiling: dst = src in 16-byte non-temporal loads and stores.
// Each workgroup copies one contiguous chunk, four requests in flight per
// thread (measured on MI355X: 5.5-5.6 TB/s for 1 GiB, against 4.7 TB/s for
// a grid-stride walk and 5.1 TB/s for torch's copy).
__global__ void __launch_bounds__(256) k_debug_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   uint64_t n16) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;       // 16-byte elements per workgroup
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  const uint64_t stride = blockDim.x;
  uint64_t i = lo + threadIdx.x;
  for (; i + 3 * stride < hi; i += 4 * stride) {
    const u32x4 a = ld_nt<u32x4>(src + i), b = ld_nt<u32x4>(src + i + stride);
    const u32x4 c = ld_nt<u32x4>(src + i + 2 * stride), d = ld_nt<u32x4>(src + i + 3 * stride);
    st_nt<u32x4>(dst + i, a);
    st_nt<u32x4>(dst + i + stride, b);
    st_nt<u32x4>(dst + i + 2 * stride, c);
    st_nt<u32x4>(dst + i + 3 * stride, d);
  }
  for (; i < hi; i += stride) st_nt<u32x4>(dst + i, ld_nt<u32x4>(src + i));
}

// Matrix-core ceiling: every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 on register operands of ones, so each round adds
// exactly 16 to every accumulator element; thread t of workgroup b writes
// out[256 b + t] = the four accumulators' first elements summed = 64 iters.
__global__ void __launch_bounds__(256) k_debug_mfma(float* __restrict__ out, int iters) {
  bf16x8 one;
#pragma unroll
  for (int i = 0; i < 8; ++i) one[i] = (__bf16)1.0f;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, acc[j], 0, 0, 0);
  }
  out[(uint64_t)blockIdx.x * 256u + threadIdx.x] = acc[0][0] + acc[1][0] + acc[2][0] + acc[3][0];
}

// Streaming ceiling of the fused step's own state traffic: W bf16, m and v
// fp32 [N, K] read and written once (20 bytes per element) in 128 x 128
// tiles, one 256-thread workgroup per tile, tiles in row-major order, each
// thread one 4-element segment per row pass, 8 passes in flight, 16-byte
// (8-byte for W) non-temporal accesses -- the access pattern of the
// epilogue with no gradient and no arithmetic beyond a trivial update
// (m' = m + 1, v' = v + 1, W' = W with its bit pattern incremented), so that
// the kernel cannot be folded away.  Requires N % 128 == K % 128 == 0.
__global__ void __launch_bounds__(256) k_debug_state_stream(uint16_t* __restrict__ W, float* __restrict__ m,
                                                           float* __restrict__ v, int N, int K) {
  constexpr int PASSES = 16, RPP = 8, DEPTH = 8;    // 128 rows, 8 per pass (32 segments of 4 per row)
  const int tk = K / TILE;
  const int ti = (int)blockIdx.x / tk, tj = (int)blockIdx.x - ti * tk;
  const int t = threadIdx.x;
  const int64_t q = (int64_t)tj * TILE + 4 * (t & 31);
  const int64_t r0 = (int64_t)ti * TILE + (t >> 5);
  u32x2 pw[DEPTH];
  f32x4 pm[DEPTH], pv[DEPTH];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) {
    const int64_t o = (r0 + s * RPP) * K + q;
    pw[s] = ld_nt<u32x2>(W + o);
    pm[s] = ld_nt<f32x4>(m + o);
    pv[s] = ld_nt<f32x4>(v + o);
  }
#pragma unroll
  for (int s = 0; s < PASSES; ++s) {
    const int slot = s % DEPTH;
    u32x2 w = pw[slot];
    f32x4 mm = pm[slot], vv = pv[slot];
    const int64_t o = (r0 + s * RPP) * K + q;
    if (s + DEPTH < PASSES) {
      const int64_t on = (r0 + (s + DEPTH) * RPP) * K + q;
      pw[slot] = ld_nt<u32x2>(W + on);
      pm[slot] = ld_nt<f32x4>(m + on);
      pv[slot] = ld_nt<f32x4>(v + on);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mm[i] = mm[i] + 1.f;
      vv[i] = vv[i] + 1.f;
    }
    w[0] += 0x00010001u;
    w[1] += 0x00010001u;
    st_nt<u32x2>(W + o, w);
    st_nt<f32x4>(m + o, mm);
    st_nt<f32x4>(v + o, vv);
  }
}

hipError_t launch_debug_state_stream(uint16_t* W, float* m, float* v, int N, int K, hipStream_t st) {
  if (N == 0 || K == 0) return hipSuccess;
  hipLaunchKernelGGL(k_debug_state_stream, dim3((unsigned)((N / TILE) * (K / TILE))), dim3(256), 0, st, W, m, v, N,
                     K);
  return hipGetLastError();
}

hipError_t launch_debug_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const uint64_t n16 = bytes / 16u;
  const uint64_t threads = (n16 + 3u) / 4u;
  const unsigned blocks = (unsigned)std::min<uint64_t>((threads + 255u) / 256u, 16384u);
  hipLaunchKernelGGL(k_debug_copy, dim3(blocks), dim3(256), 0, st, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_debug_mfma(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_mfma, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

hipError_t launch_gemm(const KArgs& a, int in_fmt, hipStream_t st) {
  if (in_fmt == FMT_BF16 && a.dma_ok) hipLaunchKernelGGL((k_gemm<FMT_BF16, true>), tile_grid(a), dim3(NT), 0, st, a);
  else if (in_fmt == FMT_BF16) hipLaunchKernelGGL((k_gemm<FMT_BF16, false>), tile_grid(a), dim3(NT), 0, st, a);
  else if (in_fmt == FMT_F32) hipLaunchKernelGGL((k_gemm<FMT_F32, false>), tile_grid(a), dim3(NT), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_debug_sr(const float* in, uint16_t* out, uint32_t n, uint32_t key, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t threads = (n + 1ull) / 2ull;   // one pair per thread
  hipLaunchKernelGGL(k_debug_sr, dim3((unsigned)((threads + 255u) / 256u)), dim3(256), 0, st, in, out, n, key);
  return hipGetLastError();
}

}  // namespace forge
