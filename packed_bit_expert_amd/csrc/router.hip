// Router of a GPU-resident MoE layer, on the device.
//
// "LFM2.5-24B-A2B -- Packed MXFP4 Inference", "GPU routing inside
// resident-layer graphs": the layer's graph holds the router projection,
// sigmoid scores, the expert bias where configured, dynamic top-k selection
// and the routing coefficients, recomputed on every replay, and the expert
// ids never go back to the host.  One launch per layer, one wave per
// (token, expert): logit[t][e] = sum_k u[k] * Wr[e][k] in FP64 (BF16 x BF16
// products are exact in FP64), u = x or its weightless RMS pre-norm; the
// token's last workgroup then selects: s = sigmoid(logit) in FP64, key
// c = s + bias, k rounds of a wave-wide (key desc, id asc) argmax, and
// w_j = bf16(s_j / sum of the selected s) in slot order.
// The top-k decision and the coefficients are taken in FP64, the precision
// the oracle uses; the two sides can differ only where keys tie to within
// FP64 rounding.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {


// One wave: the k-of-E selection of token t from its FP64 logits.
// Lane l holds experts l, l + 64, l + 128, l + 192 (E <= 256).
__device__ void router_select(const double* logits, const float* bias, int E, int K, int lane,
                              int32_t* ids, uint16_t* rw, const RouteResolve& res) {
  double s[4], c[4];
  bool taken[4];
  double l[4];
  float bv[4];
  // without a bias, a harmless read of the logits (its value is not used),
  // so that every load is unconditional and all are in flight together
  const float* bsrc = bias ? bias : (const float*)logits;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i < E ? lane + 64 * i : 0;
    l[i] = __hip_atomic_load(logits + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bv[i] = bsrc[e];
  }
  // with a slot table to fill, every expert's table entries are loaded now,
  // next to the logits, so that the winners' entries are at hand (a lane
  // holds those of its experts) instead of a round trip after the selection
  uint64_t tw[4] = {0, 0, 0, 0}, ts[4] = {0, 0, 0, 0};
  float tg[4] = {1.f, 1.f, 1.f, 1.f}, td[4] = {1.f, 1.f, 1.f, 1.f};
  if (res.slots) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (64 * i >= E) break;
      const int e = lane + 64 * i < E ? lane + 64 * i : 0;
      tw[i] = (uint64_t)res.wtab[e];
      ts[i] = (uint64_t)res.stab[e];
      if (res.tsc) {
        tg[i] = res.tsc[2 * e];
        td[i] = res.tsc[2 * e + 1];
      }
    }
  }
  uint64_t my_w = 0, my_sb = 0;  // lane j: slot j's expert bases and tensor scales
  float my_tg = 1.f, my_td = 1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    taken[i] = e >= E;
    s[i] = 0.0;
    c[i] = 0.0;
    if (e < E) {
      s[i] = 1.0 / (1.0 + exp(-l[i]));
      c[i] = s[i] + (bias ? (double)bv[i] : 0.0);
    }
  }
  double my_s = 0.0;  // lane j keeps slot j's score and expert
  int32_t my_e = 0;
  double sum = 0.0;
  for (int j = 0; j < K; ++j) {
    // this lane's best untaken expert: largest key, then smallest id
    double bc = -INFINITY, bs = 0.0;
    uint32_t be = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!taken[i] && (be == 0xFFFFFFFFu || c[i] > bc)) {
        bc = c[i];
        bs = s[i];
        be = (uint32_t)(lane + 64 * i);
      }
    // wave-wide argmax by butterfly; every lane ends with the same winner
#define MOE_ARGMAX_STEP(O)                                                                   \
  {                                                                                        \
    const double oc = xor_lane<O>(bc, lane), os = xor_lane<O>(bs, lane);                   \
    const uint32_t oe = xor_lane_u32<O>(be, lane);                                         \
    if (oe != 0xFFFFFFFFu && (be == 0xFFFFFFFFu || oc > bc || (oc == bc && oe < be))) {    \
      bc = oc;                                                                             \
      bs = os;                                                                             \
      be = oe;                                                                             \
    }                                                                                      \
  }
    MOE_ARGMAX_STEP(32) MOE_ARGMAX_STEP(16) MOE_ARGMAX_STEP(8) MOE_ARGMAX_STEP(4)
    MOE_ARGMAX_STEP(2) MOE_ARGMAX_STEP(1)
#undef MOE_ARGMAX_STEP
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((uint32_t)(lane + 64 * i) == be) taken[i] = true;
    if (lane == j) {
      my_s = bs;
      my_e = (int32_t)be;
    }
    if (res.slots) {  // the winner's entries, from the lane that holds them
      // (be is the same in every lane after the butterfly)
      const int src = __builtin_amdgcn_readfirstlane((int)(be & 63u));
      const int reg = __builtin_amdgcn_readfirstlane((int)(be >> 6));
      uint64_t w = tw[0], sb = ts[0];
      float g = tg[0], d = td[0];
#pragma unroll
      for (int i = 1; i < 4; ++i)
        if (reg == i) {
          w = tw[i];
          sb = ts[i];
          g = tg[i];
          d = td[i];
        }
      const uint64_t ww = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(w >> 32), src) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, src);
      const uint64_t ss = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(sb >> 32), src) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sb, src);
      const float gg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), src));
      const float dd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), src));
      if (lane == j) {
        my_w = ww;
        my_sb = ss;
        my_tg = gg;
        my_td = dd;
      }
    }
    sum += bs;  // slot order, as the oracle sums
  }
  if (lane < K) {
    ids[lane] = my_e;
    rw[lane] = f64_to_bf16(my_s / sum);
    if (res.slots) {
      // the ids are in range by construction; under MOE_FLAG_CHECK_IDS a
      // misaligned expert base rejects the slot, as the decode kernels do
      SlotRef r;
      r.w = (const uint8_t*)my_w;
      r.s = (const uint8_t*)my_sb;
      r.tg = my_tg;
      r.td = my_td;
      r.ok = 1;
      r.pad = 0;
      if ((res.flags & MOE_FLAG_CHECK_IDS) && ((my_w | my_sb) & 15u)) {
        if (res.err) atomicOr(res.err, kErrAlign);
        r.tg = r.td = 1.f;
        r.ok = 0;
      }
      res.slots[lane] = r;
    }
  }
}

// grid (T, ceil(E / 4)), 256 threads: wave w of workgroup y computes the
// logit of expert 4y + w.  x goes to LDS (one 16-byte piece per thread for
// H = 2048) and is pre-normed there once per workgroup in FP64; lane l of a
// wave holds the router-row pieces l, l + 64, ... (H a multiple of 512, at
// most 2048: at most 4 pieces), loaded before x is waited for.  The
// workgroup's logits leave together as device-coherent stores; once they
// have been stored, the workgroup counts itself in with a release atomic,
// and the token's last workgroup to finish takes an acquire fence and
// selects, reading the logits with device-coherent loads -- an atomic count
// that nobody waits on.  count[T] starts at 0 and is left at 0.
template <bool PRENORM>
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ x,
                                                const uint16_t* __restrict__ wr,
                                                const float* __restrict__ bias, int H, int E,
                                                int K, float eps, double* logits, uint32_t* count,
                                                int32_t* __restrict__ ids,
                                                uint16_t* __restrict__ rw, RouteResolve res) {
  // every argument fetched in one scalar batch
  asm volatile("" ::"s"(x), "s"(wr), "s"(bias), "s"(H), "s"(E), "s"(K), "s"(eps), "s"(logits),
               "s"(count), "s"(ids), "s"(rw));
  __shared__ __attribute__((aligned(16))) uint16_t us[2048];
  __shared__ double red[4], lgs[4];
  __shared__ int last;
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.y * 4 + wave;
  const int npc = H / 8 / 64;
  const uint16_t* xt = x + (size_t)t * H;
  const uint16_t* row = wr + (size_t)(e < E ? e : 0) * H;
  const bool xpiece = tid < H / 8;
  const uint4 xv = xpiece ? ldg16(xt + 8 * tid) : make_uint4(0u, 0u, 0u, 0u);
  uint4 wv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) wv[p] = p < npc ? ldg16(row + 8 * (lane + 64 * p)) : make_uint4(0u, 0u, 0u, 0u);
  if (!PRENORM && xpiece) *(uint4*)(us + 8 * tid) = xv;

  if (PRENORM) {  // FP64, once per workgroup, the same order as the layer's gate/up kernel
    double ss = sumsq8_bf16(xv);
    ss = seg_finish<32, double>(ss, lane);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double rs = rsqrt_f64((red[0] + red[1] + red[2] + red[3]) / (double)H + (double)eps);
    // rescaled from the registers (the FP32 path with its exact-rounding
    // guard, as in the layer's kernels), stored once
    const uint4 uv = scale8_bf16(xv, rs);
    if (xpiece) *(uint4*)(us + 8 * tid) = uv;
  }
  __syncthreads();

  double acc = 0.0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (p >= npc) break;
    const uint4 uv = *(const uint4*)(us + 8 * (lane + 64 * p));
    const uint32_t a4[4] = {wv[p].x, wv[p].y, wv[p].z, wv[p].w}, b4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = fma((double)__uint_as_float(a4[q] << 16), (double)__uint_as_float(b4[q] << 16), acc);
      acc = fma((double)__uint_as_float(a4[q] & 0xFFFF0000u),
                (double)__uint_as_float(b4[q] & 0xFFFF0000u), acc);
    }
  }
  acc = seg_finish<32, double>(acc, lane);
  if (lane == 0) lgs[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    for (int w = 0; w < 4; ++w)
      if ((int)blockIdx.y * 4 + w < E)
        __hip_atomic_store(logits + (size_t)t * E + blockIdx.y * 4 + w, lgs[w], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // The count is a release operation at agent scope, so the logit stores
    // above happen before it for every workgroup that reads the count; the
    // workgroup that reads the final value takes an agent-scope acquire
    // fence after it (fence synchronisation: its read of the count, part of
    // every earlier workgroup's release sequence, is sequenced before the
    // fence).  The workgroup barrier below then orders the selecting wave's
    // logit loads after that acquire.
    const uint32_t prev = __hip_atomic_fetch_add(count + t, 1u, __ATOMIC_RELEASE,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last = prev == gridDim.y - 1;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(count + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!last || wave != 0) return;
  // router_select reads the logits with device-coherent loads
  RouteResolve rt = res;
  if (rt.slots) rt.slots += (size_t)t * K;
  router_select(logits + (size_t)t * E, bias, E, K, lane, ids + (size_t)t * K, rw + (size_t)t * K,
                rt);
}

}  // namespace

bool router_supported(int H, int E, int K) {
  return H > 0 && H % 512 == 0 && H <= 2048 && E >= 1 && E <= 256 && K >= 1 && K <= 8 && K <= E;
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                        int E, int K, bool prenorm, float eps, double* logits, uint32_t* count,
                        int32_t* ids, uint16_t* rw, const RouteResolve& res, hipStream_t s) {
  // at most kRouterCounters tokens per launch: their counters sit at a fixed
  // place of the workspace, so a workspace reused with another cfg still
  // finds them at zero; launches on one stream run one after the other
  for (int t0 = 0; t0 < T; t0 += kRouterCounters) {
    const int n = T - t0 < kRouterCounters ? T - t0 : kRouterCounters;
    const dim3 grid(n, (E + 3) / 4);
    const uint16_t* xc = x + (size_t)t0 * H;
    double* lc = logits + (size_t)t0 * E;
    int32_t* ic = ids + (size_t)t0 * K;
    uint16_t* rc = rw + (size_t)t0 * K;
    RouteResolve rs = res;
    if (rs.slots) rs.slots += (size_t)t0 * K;
    const hipError_t e =
        prenorm ? launch_kernel(MOE_KERNEL_ROUTER, k_router<true>, grid, dim3(256), 0, s, xc, wr,
                                bias, H, E, K, eps, lc, count, ic, rc, rs)
                : launch_kernel(MOE_KERNEL_ROUTER, k_router<false>, grid, dim3(256), 0, s, xc, wr,
                                bias, H, E, K, eps, lc, count, ic, rc, rs);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
