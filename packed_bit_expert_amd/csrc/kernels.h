// Kernel launchers of the W4A16 MoE library (host side of the HIP kernels).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One routing slot (token t, slot j) resolved to its expert: weight and scale
// bases and the two tensor scales (1 for E8M0).  ok = 0 marks a slot a device
// check rejected (its h and y are 0).
struct SlotRef {
  const uint8_t* w;
  const uint8_t* s;
  float tg, td;
  int32_t ok, pad;
};

// A resolved slot with one 32-byte vector load (device code).
__device__ __forceinline__ SlotRef load_slot(const SlotRef* p) {
  SlotRef r;
  const uint4* q = (const uint4*)p;
  const uint4 a = q[0], b = q[1];
  r.w = (const uint8_t*)(((uint64_t)a.y << 32) | a.x);
  r.s = (const uint8_t*)(((uint64_t)a.w << 32) | a.z);
  r.tg = __uint_as_float(b.x);
  r.td = __uint_as_float(b.y);
  r.ok = (int32_t)b.z;
  r.pad = 0;
  return r;
}

// Arguments of the per-token GEMV path (decode).  All pointers are device
// pointers; the dump pointers may be null.
struct DecodeArgs {
  const uint16_t* x;          // [T][H] BF16
  const int32_t* ids;         // [T][K]
  const uint16_t* rw;         // [T][K] BF16 routing coefficients
  const uint8_t* const* wtab; // [E] packed-nibble bases
  const uint8_t* const* stab; // [E] scale bases
  const float* tsc;           // [E][2] FP32 tensor scales (E4M3) or null
  const uint16_t* residual;   // [T][H] or null
  uint16_t* out;              // [T][H]
  uint16_t* hbuf;             // [T][K][I] workspace
  SlotRef* slots;             // [T][K] workspace: written by gate/up, read by down
  const SlotRef* pre;         // [T][K] already resolved slots, or null
  uint16_t *du, *dg, *dv, *dh, *dy;
  int* err;                   // device error word
  int T, H, I, K, E;
  uint32_t flags;
  float eps;
  uint64_t kmagic;            // floor(2^32 / K) + 1, set by the decode launcher
};

// Arguments of the sorted batched path.
struct BatchedArgs {
  const uint16_t* x;
  const int32_t* ids;
  const uint16_t* rw;
  const uint8_t* const* wtab;
  const uint8_t* const* stab;
  const float* tsc;
  const uint16_t* residual;
  uint16_t* out;
  uint16_t* hbuf;     // [T * K][I]
  uint16_t* ybuf;     // [T * K][H]
  uint8_t* hq;        // [T * K][mxfp4_row_bytes(I)]: h as MXFP4 rows (W4A4)
  uint16_t *du, *dg, *dv, *dh, *dy;
  int* err;
  uint16_t* ubuf;     // [T][H] the pre-normed input (MOE_FLAG_PRENORM)
  uint16_t* unext;    // [T][H] or null: where the combine writes the pre-norm of out
  uint8_t* xqbuf;     // [T][mxfp4_row_bytes(H)]: the pre-norm as MXFP4 rows (W4A4)
  const uint8_t* xq;  // set by the launcher: xqbuf when it holds this call's rows, else null
  bool x_normed;      // ubuf already holds the pre-norm of x (and xqbuf its MXFP4 rows under W4A4)
  int ncu;            // CUs of the device (set by the launcher)
  int T, H, I, K, E;
  uint32_t flags;
  float eps;
};

bool decode_supported(int H, int I);
bool batched_supported(int H, int I);

hipError_t launch_decode(const DecodeArgs& a, int fmt, hipStream_t s);
// Resolve n = L*T*K slots of consecutive layers: out[i] for ids[i] of layer
// i / (T*K), tables wtab/stab [L][E], tensor scales [L][E][2] or null.
hipError_t launch_resolve(const int32_t* ids, const uint8_t* const* wtab,
                          const uint8_t* const* stab, const float* tsc, int n, int per_layer,
                          int E, uint32_t flags, int* err, SlotRef* out, hipStream_t s);
hipError_t launch_batched(const BatchedArgs& a, int fmt, hipStream_t s);
hipError_t launch_sort(const int32_t* ids, int npairs, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* active, int32_t* nactive, int* err, uint32_t flags,
                       hipStream_t s);
// With u (not null) the combine also writes u = the pre-norm of out, and with
// uq (not null) u as MXFP4 rows as well.
hipError_t launch_combine(const uint16_t* y, const uint16_t* rw, const uint16_t* residual,
                          uint16_t* out, int T, int K, int H, hipStream_t s,
                          uint16_t* u = nullptr, float eps = 0.f, uint8_t* uq = nullptr);
hipError_t launch_prenorm(const uint16_t* x, uint16_t* u, int T, int H, float eps, hipStream_t s,
                          uint8_t* uq = nullptr);
hipError_t launch_dequant(const uint8_t* nib, const uint8_t* sc, int rows, int cols, int fmt,
                          uint16_t* out, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_delay(uint32_t microseconds, hipStream_t s);
// Measurement kernels: the decode kernels' loads without their arithmetic
// (hidden 2048, inter 1536, top-4, E8M0 only), an empty kernel, and a read in
// which every lane issues all of its loads up front.
bool decode_floor_supported(int H, int I, int K);
hipError_t launch_decode_floor(const SlotRef* pre, const uint16_t* x, uint16_t* hbuf,
                               const uint16_t* rw, const uint16_t* residual, uint16_t* out,
                               hipStream_t s);
hipError_t launch_empty(int workgroups, int threads, uint32_t* sink, hipStream_t s);
hipError_t launch_grid_barrier(int workgroups, int barriers, uint32_t* counter, hipStream_t s);
hipError_t launch_read_burst(const void* src, size_t bytes, int loads_per_lane, uint32_t* sink,
                             hipStream_t s);
bool router_supported(int H, int E, int K);
// logits [T][E] FP64 and count [T] (zero, left zero) workspace; ids [T][K];
// rw [T][K] BF16
// With slots set, the router also resolves the slots it selects (expert
// bases, tensor scales, base alignment under MOE_FLAG_CHECK_IDS) into the
// table the decode kernels read, so their first dependent load is the table
// entry, not the id and then the expert tables.
struct RouteResolve {
  const uint8_t* const* wtab = nullptr;
  const uint8_t* const* stab = nullptr;
  const float* tsc = nullptr;
  uint32_t flags = 0;
  int* err = nullptr;
  SlotRef* slots = nullptr;  // [T][K], or null: no resolution
};

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                        int E, int K, bool prenorm, float eps, double* logits, uint32_t* count,
                        int32_t* ids, uint16_t* rw, const RouteResolve& res, hipStream_t s);

// Kernel timing (moe_w4a16_timing_*): while the calling thread times
// launches, each launch gets a start and a stop event that the dispatch
// itself records (hipExtLaunchKernel), i.e. the kernel's own execution
// interval; otherwise both are null and the launch is an ordinary one.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents timing_begin(int kind, hipStream_t s);
void timing_end(const LaunchEvents& ev);

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t s, Args... args) {
  const LaunchEvents ev = timing_begin(kind, s);
  if (ev.start)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, ev.start, ev.stop, 0u, args...);
  else
    kernel<<<grid, block, shmem, s>>>(args...);
  timing_end(ev);
  return hipGetLastError();
}

// Records a result code and message as the calling thread's last error (what
// moe_w4a16_last_error returns); returns code.  MOE_OK clears the message.
int report(int code, const char* msg);

}  // namespace moe
