// Floor kernels for the decode path (measurement only).
//
// They answer how long the batch-1 decode kernels would take if they did no
// arithmetic at all.  Each one reads exactly the bytes its decode kernel
// reads, with the same grid, the same dependent load of the routing slot
// before the weights, and the same order of loads per lane, then folds
// everything it loaded into one word with XOR, which it stores where its
// decode kernel stores its results (h, out), so that the loads cannot be
// dropped and the same stores complete before the kernel ends.  Next to
// them: an empty kernel of a given grid (the launch alone), a read of a
// byte range in which every lane issues all of its 16-byte loads before it
// uses any (the cost of moving the same bytes with no dependent load in
// front of them), and a kernel of repeated grid-wide barriers (what a
// persistent kernel would pay per in-kernel dependency instead of a kernel
// boundary).
//
// The decode kernels they mirror are fixed to the LFM2.5-24B-A2B shape
// (hidden 2048, expert intermediate 1536, top-4, E8M0 per 32): "LFM2.5-24B-A2B
// -- Packed MXFP4 Inference", "Model and quantization".
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kH = 2048, kI = 1536, kK = 4;
constexpr uint32_t kNever = 0x9E3779B9u;  // the word no fold is compared against in practice

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Gate/up: 4 waves per workgroup, wave gw owns rows 2 nb, 2 nb + 1 of gate and
// of up of slot gw / 768; lane (li = lane % 16, q = lane / 16) loads one scale
// byte and one 16-byte chunk of its row for chunks li, li + 16, li + 32,
// li + 48; the workgroup loads the token's 4 KB of x (16 bytes per thread).
__global__ __launch_bounds__(256) void k_floor_gateup(const SlotRef* pre, const uint16_t* x,
                                                      uint16_t* hbuf) {
  asm volatile("" ::"s"(pre), "s"(x), "s"(hbuf));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  const int per_slot = kI / 2;
  const int nb = gw % per_slot, sj = gw / per_slot;
  const SlotRef sr = load_slot(pre + sj);
  __builtin_amdgcn_sched_barrier(0);
  const uint4 xv = ldg16(x + 8 * threadIdx.x);
  __builtin_amdgcn_sched_barrier(0);
  const int li = lane & 15, q = lane >> 4;
  const int n = nb * 2 + (q >> 1);
  const uint8_t* srow = sr.s + (size_t)(q & 1) * kI * (kH / 32) + (size_t)n * (kH / 32);
  const uint8_t* wrow = sr.w + (size_t)(q & 1) * kI * (kH / 2) + (size_t)n * (kH / 2);
  uint32_t sv[4];
  uint4 wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = ldg<uint8_t>(srow + li + 16 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = ldg16(wrow + 16 * (li + 16 * i));
  uint32_t acc = fold(xv);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc ^= sv[i] ^ fold(wv[i]);
  // the decode kernel's stores: h of rows n (lane 0) and n + 1 (lane 32)
  if (li == 0 && (q & 1) == 0) hbuf[(size_t)sj * kI + n] = (uint16_t)acc;
}

// Down: 256 workgroups of 8 output rows and 8 waves; wave w takes slot
// w % 4 and the 4 rows m0 + 4 (w / 4) + q (one load set), loads that slot's
// h (I BF16, 16 bytes per lane three times), the 4 coefficients and one
// residual value; lane (li, q) loads the scale byte and 16-byte chunk of
// its row for chunks li, li + 16, li + 32.
__global__ __launch_bounds__(512) void k_floor_down(const SlotRef* pre, const uint16_t* hbuf,
                                                    const uint16_t* rw, const uint16_t* residual,
                                                    uint16_t* out) {
  asm volatile("" ::"s"(pre), "s"(hbuf), "s"(rw), "s"(residual), "s"(out));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int js = wave & 3, st = wave >> 2;
  const int m0 = blockIdx.x * 8;
  const SlotRef sr = load_slot(pre + js);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < kK; ++j) acc ^= rw[j];
  acc ^= residual[m0 + tid % 8];
  uint4 hv[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) hv[u] = ldg16(hbuf + (size_t)js * kI + 8 * (lane + 64 * u));
  const int li = lane & 15, q = lane >> 4;
  const int row = m0 + 4 * st + q;
  const uint8_t* wd = sr.w + (size_t)kI * kH;
  const uint8_t* sd = sr.s + 2 * (size_t)kI * (kH / 32);
  uint32_t sv[3];
  uint4 wv[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) sv[i] = ldg<uint8_t>(sd + (size_t)row * (kI / 32) + li + 16 * i);
#pragma unroll
  for (int i = 0; i < 3; ++i) wv[i] = ldg16(wd + (size_t)row * (kI / 2) + 16 * (li + 16 * i));
#pragma unroll
  for (int u = 0; u < 3; ++u) acc ^= fold(hv[u]);
#pragma unroll
  for (int i = 0; i < 3; ++i) acc ^= sv[i] ^ fold(wv[i]);
  // the decode kernel's stores: one output value per row of the workgroup
  if (tid < 8) out[m0 + tid] = (uint16_t)acc;
}

// `nbar` grid-wide barriers in one kernel: thread 0 of every workgroup adds 1
// to a counter that starts at zero (relaxed, agent scope: the cheapest
// arrival) and spins until it reaches (i + 1) * gridDim.x.  The grid must be
// resident all at once (at most one workgroup per CU is launched).  Every
// spin is bounded: past kSpinLimit polls the workgroup sets bit 0 of
// counter[1] and returns, so the kernel ends whatever happens.
constexpr uint32_t kSpinLimit = 1u << 22;

__global__ __launch_bounds__(64) void k_grid_barrier(uint32_t* counter, int nbar) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int i = 0; i < nbar; ++i) {
    if (threadIdx.x == 0) {
      const uint32_t target = (uint32_t)(i + 1) * gridDim.x;
      __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t n = 0;
      while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++n > kSpinLimit) {
          bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (bad) break;
  }
  if (threadIdx.x == 0 && bad) atomicOr(counter + 1, 1u);
}

__global__ void k_empty(uint32_t never, uint32_t* sink) {
  if (blockIdx.x == never) sink[0] = 1u;
}

// Every lane issues its N loads (elements i, i + P, ..., i + (N - 1) P of the
// n16 16-byte words, P the grid's thread count) before it uses any of them.
template <int N>
__global__ __launch_bounds__(256) void k_read_burst(const uint4* __restrict__ src, size_t n16,
                                                    uint32_t never, uint32_t* sink) {
  const size_t P = (size_t)gridDim.x * 256;
  const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint4 v[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const size_t i = i0 + (size_t)j * P;
    v[j] = i < n16 ? ldg16(src + i) : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) acc ^= fold(v[j]);
  if (acc == never) sink[i0 & 4095] = acc;
}

template <int N>
hipError_t burst_n(const void* src, size_t n16, uint32_t* sink, hipStream_t s) {
  const size_t grid = (n16 + (size_t)256 * N - 1) / ((size_t)256 * N);
  return launch_kernel(MOE_KERNEL_READ_BURST, k_read_burst<N>, dim3((unsigned)grid), dim3(256), 0,
                       s, (const uint4*)src, n16, kNever, sink);
}

}  // namespace

bool decode_floor_supported(int H, int I, int K) { return H == kH && I == kI && K == kK; }

hipError_t launch_decode_floor(const SlotRef* pre, const uint16_t* x, uint16_t* hbuf,
                               const uint16_t* rw, const uint16_t* residual, uint16_t* out,
                               hipStream_t s) {
  hipError_t e = launch_kernel(MOE_KERNEL_FLOOR_GATE_UP, k_floor_gateup, dim3(kK * kI / 2 / 4),
                               dim3(256), 0, s, pre, x, hbuf);
  if (e != hipSuccess) return e;
  return launch_kernel(MOE_KERNEL_FLOOR_DOWN, k_floor_down, dim3(kH / 8), dim3(512), 0, s, pre,
                       (const uint16_t*)hbuf, rw, residual, out);
}

hipError_t launch_empty(int workgroups, int threads, uint32_t* sink, hipStream_t s) {
  return launch_kernel(MOE_KERNEL_EMPTY, k_empty, dim3(workgroups), dim3(threads), 0, s, kNever,
                       sink);
}

hipError_t launch_grid_barrier(int workgroups, int barriers, uint32_t* counter, hipStream_t s) {
  return launch_kernel(MOE_KERNEL_GRID_BARRIER, k_grid_barrier, dim3(workgroups), dim3(64), 0, s,
                       counter, barriers);
}

hipError_t launch_read_burst(const void* src, size_t bytes, int loads_per_lane, uint32_t* sink,
                             hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  switch (loads_per_lane) {
    case 1: return burst_n<1>(src, n16, sink, s);
    case 2: return burst_n<2>(src, n16, sink, s);
    case 4: return burst_n<4>(src, n16, sink, s);
    case 8: return burst_n<8>(src, n16, sink, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
