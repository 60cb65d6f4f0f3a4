// Kernels shared by every optimizer: the unfused baseline's GEMM (G to HBM)
// and the stochastic-rounding test hook.
#include "forge_device.h"

namespace forge {

// The device stochastic rounding on its own: element i uses flat index i.
__global__ void k_debug_sr(const float* __restrict__ in, uint16_t* __restrict__ out, uint32_t n, uint32_t key) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint16_t)bf16_sr_bits(in[i], key, i);
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

hipError_t launch_debug_e4m3(const float* in, uint8_t* out, uint32_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t threads = (n + 3ull) / 4ull;
  hipLaunchKernelGGL(k_debug_e4m3, dim3((unsigned)((threads + 255u) / 256u)), dim3(256), 0, st, in, out, n);
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
  const unsigned blocks = (unsigned)((n + 255u) / 256u);
  hipLaunchKernelGGL(k_debug_sr, dim3(blocks), dim3(256), 0, st, in, out, n, key);
  return hipGetLastError();
}

}  // namespace forge
