// Test and measurement kernels of the W4A16 MoE library: dequantisation dump
// (same decoders as the GEMM kernels), workspace zero-fill, HBM stream read.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// One thread per 16-byte chunk (32 codes) of a packed [rows][cols] matrix.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ nib,
                                                 const uint8_t* __restrict__ sc, int rows,
                                                 int cols, uint16_t* __restrict__ out) {
  const int cpr = cols / 32;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * cpr) return;
  const int n = (int)(idx / cpr), c = (int)(idx % cpr);
  const uint4 w = *(const uint4*)(nib + (size_t)n * (cols / 2) + 16 * c);
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  uint4* dst = (uint4*)(out + (size_t)n * cols + 32 * c);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x8 v;
    if constexpr (FMT == MOE_SCALE_E8M0_G32)
      v = fp4x8_to_bf16x8(wd[d], e8m0_f32(sc[(size_t)n * (cols / 32) + c]));
    else
      v = fp4x8_scaled_to_bf16x8(wd[d], e4m3_f32(sc[(size_t)n * (cols / 16) + 2 * c + (d >> 1)]));
    dst[d] = __builtin_bit_cast(uint4, v);
  }
}

__global__ __launch_bounds__(256) void k_zero(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    ((uint4*)p)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < (bytes & 15)) p[16 * n16 + threadIdx.x] = 0;
}

// Plain read of n16 16-byte words, grid-strided; the grid is sized to the
// buffer (launch_stream_read).
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

// One wave spinning on the 100 MHz real-time counter until `ticks` have
// passed; the loop ends for any counter value, since the counter only grows.
__global__ __launch_bounds__(64) void k_delay(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(16);
}

}  // namespace

hipError_t launch_dequant(const uint8_t* nib, const uint8_t* sc, int rows, int cols, int fmt,
                          uint16_t* out, hipStream_t s) {
  const long long chunks = (long long)rows * (cols / 32);
  if (chunks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  if (fmt == MOE_SCALE_E4M3_G16)
    return launch_kernel(MOE_KERNEL_DEQUANT, k_dequant<MOE_SCALE_E4M3_G16>, dim3(grid), dim3(256), 0,
                         s, nib, sc, rows, cols, out);
  return launch_kernel(MOE_KERNEL_DEQUANT, k_dequant<MOE_SCALE_E8M0_G32>, dim3(grid), dim3(256), 0, s,
                       nib, sc, rows, cols, out);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  return launch_kernel(MOE_KERNEL_ZERO, k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint8_t*)p,
                       bytes);
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  // two 16-byte words per thread at least, 256 to 4096 workgroups
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>(4096, std::max<size_t>(256, (n16 + 511) / 512));
  return launch_kernel(MOE_KERNEL_STREAM_READ, k_stream_read, dim3(grid), dim3(256), 0, s,
                       (const uint4*)src, n16, sink);
}

hipError_t launch_delay(uint32_t microseconds, hipStream_t s) {
  return launch_kernel(MOE_KERNEL_DELAY, k_delay, dim3(1), dim3(64), 0, s,
                       (uint64_t)microseconds * 100u);
}

}  // namespace moe
