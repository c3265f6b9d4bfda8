// Per-token GEMV path (decode, T = 1) of the grouped top-k W4A16 MoE FFN.
//
// "LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Grouped top-4 expert
// execution": all selected experts are processed together -- grouped packed
// GEMV for gate and up, activation and multiplication, grouped packed GEMV
// for down, and a fused routing-weighted combine that keeps the sequential
// BF16 multiply/add rounding.  The weights are decoded in registers during the
// dot products; nothing is expanded to BF16 in memory ("Model and
// quantization": packed GEMV kernels with FP32 accumulation and BF16 outputs).
//
// CDNA4 mapping.  Every lane streams 16-byte chunks (32 E2M1 codes = exactly
// one E8M0 block, or two E4M3 blocks) with one dwordx4 load, so one wave
// instruction reads 1 KiB of contiguous weights.  All chunk loads of a wave
// are issued before any arithmetic.  Codes become BF16 pairs with
// v_cvt_scalef32_pk_bf16_fp4 (the E8M0 scale folded into the conversion) and
// meet the activations in v_dot2_f32_bf16: two VALU instructions per pair of
// weights.  Row sums are finished with a multi-value butterfly across lanes.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Row mapping shared by both GEMVs.  A row of K = 32*C weights is C 16-byte
// chunks; LPR lanes share a row, each holding CPL chunks (lane li of the row
// takes chunks li, li + LPR, ...), so a wave covers RPS = 64 / LPR rows per
// load set of CPL loads.  Every load instruction still reads contiguous
// 16*LPR-byte runs of RPS rows.  A lane sums its CPL chunks in registers, so
// the cross-lane reduction spans only LPR lanes.
template <int C>
struct RowMap {
  static constexpr int LPR = (C % 16 == 0) ? 16 : 8;
  static_assert(C % LPR == 0, "rows must be a multiple of 8 chunks (256 values)");
  static constexpr int CPL = C / LPR;
  static constexpr int RPS = 64 / LPR;
};

// gate/up: K = H; NS load sets per wave (4 weight loads per lane in total:
// at H = 2048 one set, 2 rows of gate and 2 of up per wave, 3,072 waves per
// layer -- twice as many waves with half the work each finish sooner after
// their data lands than 8 loads per lane did); rows of a set alternate gate n,
// up n, gate n+1, up n+1, ... so the partner matrix of a row sits LPR lanes
// away.
template <int H>
struct GuShape {
  static constexpr int C = H / 32;
  using M = RowMap<C>;
  static constexpr int NS = 4 / M::CPL > 0 ? 4 / M::CPL : 1;
  static constexpr int RW = NS * M::RPS / 2;  // n rows (of gate and of up) per wave
  static_assert(NS <= M::LPR && (NS & (NS - 1)) == 0, "load sets per wave");
};

// down: K = I; a workgroup owns ROWS = NS * RPS output rows for every slot
// (one wave per slot), so the combine is finished in the same workgroup.
template <int I>
struct DnShape {
  static constexpr int C = I / 32;
  using M = RowMap<C>;
  static constexpr int NS = M::RPS >= 8 ? 1 : 8 / M::RPS;
  static constexpr int ROWS = NS * M::RPS;
  static_assert(NS <= M::LPR && (NS & (NS - 1)) == 0, "load sets per wave");
};

template <int FMT>
constexpr int group_of() { return FMT == MOE_SCALE_E4M3_G16 ? 16 : 32; }

template <int FMT>
__device__ __forceinline__ uint32_t load_chunk_scale(const uint8_t* srow, int c) {
  if constexpr (FMT == MOE_SCALE_E8M0_G32) return ldg<uint8_t>(srow + c);
  else return ldg<uint16_t>(srow + 2 * c);
}

__device__ __forceinline__ void unpack16(const uint16_t* p, bf16x2 (&xp)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = ldg16(p + 8 * q);
    xp[4 * q + 0] = __builtin_bit_cast(bf16x2, w.x);
    xp[4 * q + 1] = __builtin_bit_cast(bf16x2, w.y);
    xp[4 * q + 2] = __builtin_bit_cast(bf16x2, w.z);
    xp[4 * q + 3] = __builtin_bit_cast(bf16x2, w.w);
  }
}

__device__ __forceinline__ void unpack16_lds(const uint16_t* p, bf16x2 (&xp)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = ((const uint4*)p)[q];
    xp[4 * q + 0] = __builtin_bit_cast(bf16x2, w.x);
    xp[4 * q + 1] = __builtin_bit_cast(bf16x2, w.y);
    xp[4 * q + 2] = __builtin_bit_cast(bf16x2, w.z);
    xp[4 * q + 3] = __builtin_bit_cast(bf16x2, w.w);
  }
}

// Resolves slot i of ids/wtab/stab to its expert.  With MOE_FLAG_CHECK_IDS an
// out-of-range id or a misaligned base marks the slot bad (ok = 0) and, when
// err is not null, sets the matching device error bit.
__device__ __forceinline__ SlotRef resolve_slot(const int32_t* ids, const uint8_t* const* wtab,
                                                const uint8_t* const* stab, const float* tsc,
                                                int i, int E, uint32_t flags, int* err) {
  SlotRef r;
  r.pad = 0;
  r.tg = r.td = 1.f;
  const int e = ids[i];
  if ((flags & MOE_FLAG_CHECK_IDS) && (e < 0 || e >= E)) {
    if (err) atomicOr(err, kErrBadId);
    r.w = r.s = nullptr;
    r.ok = 0;
    return r;
  }
  r.w = wtab[e];
  r.s = stab[e];
  r.ok = 1;
  if ((flags & MOE_FLAG_CHECK_IDS) && ((((uintptr_t)r.w) | ((uintptr_t)r.s)) & 15u)) {
    if (err) atomicOr(err, kErrAlign);
    r.ok = 0;
  }
  if (tsc && r.ok) {
    r.tg = tsc[2 * e];
    r.td = tsc[2 * e + 1];
  }
  return r;
}

// Slots of consecutive layers resolved in one pass (the layer-stack path):
// the per-layer kernels then need one dependent load before streaming.
__global__ __launch_bounds__(256) void k_resolve(const int32_t* ids, const uint8_t* const* wtab,
                                                 const uint8_t* const* stab, const float* tsc,
                                                 int n, int per_layer, int E, uint32_t flags,
                                                 int* err, SlotRef* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int l = i / per_layer;
  out[i] = resolve_slot(ids + (size_t)l * per_layer, wtab + (size_t)l * E, stab + (size_t)l * E,
                        tsc ? tsc + (size_t)l * E * 2 : nullptr, i - l * per_layer, E, flags, err);
}

__device__ __forceinline__ SlotRef load_slot(const SlotRef* p) {
  // one 32-byte vector load
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

// Grouped gate/up GEMV + silu(g) * v.  A 256-thread workgroup is four
// independent waves, each owning RW rows of gate and of up of one (token,
// slot).  All loads of a wave are issued before any arithmetic; the
// activation slices come first because vmcnt retires loads in issue order.
// With PRENORM the workgroup stages x in LDS and computes the weightless RMS
// pre-norm once (FP64) for its four waves.  A rejected slot reads a harmless
// valid address and writes zeros, so the code after the loads is
// straight-line and each chunk waits only for its own load.
template <int H, int FMT, bool PRENORM, bool DUMP>
__global__ __launch_bounds__(256) void k_dec_gateup(DecodeArgs a) {
  // every argument the first loads depend on, fetched in one scalar batch
  // (the compiler would otherwise fetch them in dependent rounds near use)
  asm volatile("" ::"s"(a.x), "s"(a.pre), "s"(a.slots), "s"(a.hbuf), "s"(a.T), "s"(a.I),
               "s"(a.K), "s"(a.eps));
  using S = GuShape<H>;
  using M = typename S::M;
  constexpr int LPR = M::LPR, CPL = M::CPL, RPS = M::RPS, NS = S::NS, RW = S::RW;
  constexpr int G = group_of<FMT>();
  __shared__ __attribute__((aligned(16))) uint16_t xs[PRENORM ? H : 8];
  __shared__ double red[4];
  const int I = a.I;
  const int per_slot = (I + RW - 1) / RW;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  // all waves of a workgroup belong to one token (per_slot * K is a multiple of 4)
  const int nb = gw % per_slot, sj = gw / per_slot;
  const bool live = sj < a.T * a.K;
  const int sjc = live ? sj : a.T * a.K - 1;
  const int t = sjc / a.K, j = sjc - t * a.K;

  // 0. the slot's expert (one 32-byte load of the pre-resolved table; without
  // one the load reads the workspace table, a harmless valid address, and
  // the slot is resolved below), then the activations, so that both are in
  // flight together
  SlotRef sr = load_slot(a.pre ? a.pre + sjc : a.slots);
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* xt = a.x + (size_t)t * H;
  bf16x2 xp[CPL][16];
  constexpr int XPT = PRENORM ? (H / 8 + 255) / 256 : 1;  // 16-byte pieces of x per thread
  uint4 xraw[XPT];
  if constexpr (PRENORM) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int k8 = threadIdx.x + 256 * u;
      xraw[u] = k8 < H / 8 ? ldg16(xt + 8 * k8) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!a.pre) {
    sr = resolve_slot(a.ids, a.wtab, a.stab, a.tsc, sjc, a.E, a.flags,
                      (nb == 0 && lane == 0 && live) ? a.err : nullptr);
    if (nb == 0 && lane == 0 && live) a.slots[sj] = sr;
  }
  const bool ok = __builtin_amdgcn_readfirstlane(sr.ok) != 0;
  const uint8_t* wbase = ok ? sr.w : (const uint8_t*)a.slots;
  const uint8_t* sbase = ok ? sr.s : (const uint8_t*)a.slots;
  const size_t mat_nib = ok ? (size_t)I * (H / 2) : 0, mat_sc = ok ? (size_t)I * (H / G) : 0;
  const size_t row_nib = ok ? H / 2 : 0, row_sc = ok ? H / G : 0;
  const int li = lane % LPR, q = lane / LPR;
  const int n0 = nb * RW;

  // 1. loads: activations first (vmcnt retires loads in issue order, so the
  // pre-norm or the first chunk can start while the weights stream), then
  // scale bytes, then weights
  if constexpr (!PRENORM) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) unpack16(xt + 32 * (li + LPR * i), xp[i]);
  }
  uint4 wv[NS][CPL];
  uint32_t sv[NS][CPL];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int n = min(n0 + st * (RPS / 2) + (q >> 1), I - 1);  // a ragged last wave re-reads row I-1
    const uint8_t* srow = sbase + (q & 1) * mat_sc + (size_t)n * row_sc;
#pragma unroll
    for (int i = 0; i < CPL; ++i) sv[st][i] = load_chunk_scale<FMT>(srow, ok ? li + LPR * i : 0);
  }
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int n = min(n0 + st * (RPS / 2) + (q >> 1), I - 1);
    const uint8_t* wrow = wbase + (q & 1) * mat_nib + (size_t)n * row_nib;
#pragma unroll
    for (int i = 0; i < CPL; ++i) wv[st][i] = ldg16(wrow + (ok ? 16 * (li + LPR * i) : 0));
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. pre-norm once per workgroup (FP64), then the slices from LDS
  if constexpr (PRENORM) {
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int k8 = threadIdx.x + 256 * u;
      if (k8 >= H / 8) break;
      const uint4 v = xraw[u];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double lo = __uint_as_float(w4[k] << 16), hi = __uint_as_float(w4[k] & 0xFFFF0000u);
        ss += lo * lo + hi * hi;
      }
    }
    ss = seg_finish<32, double>(ss, lane);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double rs = 1.0 / sqrt((red[0] + red[1] + red[2] + red[3]) / (double)H + (double)a.eps);
    // each thread rescales the pieces it holds in registers and stores them once
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int k8 = threadIdx.x + 256 * u;
      if (k8 >= H / 8) break;
      const uint32_t w4[4] = {xraw[u].x, xraw[u].y, xraw[u].z, xraw[u].w};
      uint32_t o4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = f64_to_bf16((double)__uint_as_float(w4[k] << 16) * rs);
        const uint32_t hi = f64_to_bf16((double)__uint_as_float(w4[k] & 0xFFFF0000u) * rs);
        o4[k] = lo | (hi << 16);
      }
      *(uint4*)(xs + 8 * k8) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CPL; ++i) unpack16_lds(xs + 32 * (li + LPR * i), xp[i]);
    if constexpr (DUMP) {
      if (a.du && nb < 4 && j == 0 && live)
        for (int k = threadIdx.x; k < H; k += 256) a.du[(size_t)t * H + k] = xs[k];
    }
  } else if constexpr (DUMP) {
    if (a.du && nb == 0 && j == 0 && live)
      for (int k = lane; k < H; k += 64) a.du[(size_t)t * H + k] = xt[k];
  }
  if (!live) return;

  // 3. dot products (a lane sums its CPL chunks), one butterfly over LPR lanes
  double p[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    p[st] = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) p[st] += chunk_dot<FMT>(wv[st][i], sv[st][i], xp[i]);
  }
  const double tot = seg_reduce<NS, LPR>(p, lane);
  const double oth = xor_lane<LPR>(tot, lane);  // the same n of the other matrix
  const int v = li / (LPR / NS);             // load set whose sum this lane holds
  const int n = n0 + v * (RPS / 2) + (q >> 1);
  if ((li % (LPR / NS)) == 0 && (q & 1) == 0 && n < I) {
    const double tg = (double)sr.tg;
    uint16_t gb = f64_to_bf16(tot * tg), ub = f64_to_bf16(oth * tg);
    uint16_t h = silu_mul_bf16(gb, ub);
    if (!ok) gb = ub = h = 0;
    const size_t o = (size_t)sj * I + n;
    a.hbuf[o] = h;
    if constexpr (DUMP) {
      if (a.dg) a.dg[o] = gb;
      if (a.dv) a.dv[o] = ub;
      if (a.dh) a.dh[o] = h;
    }
  }
}

// Grouped down GEMV for ROWS output rows of every slot (one wave per slot),
// then the slot-order BF16 combine (+ residual) of those rows.  The token's h
// (all k slots, k * I BF16) is read once per workgroup into LDS; every lane
// then takes its slices from there instead of re-reading them from L2.
template <int H, int I, int FMT, bool DUMP>
__global__ __launch_bounds__(256) void k_dec_down(DecodeArgs a) {
  // every argument the first loads depend on, fetched in one scalar batch
  asm volatile("" ::"s"(a.pre), "s"(a.slots), "s"(a.hbuf), "s"(a.rw), "s"(a.residual),
               "s"(a.out), "s"(a.T), "s"(a.K));
  using D = DnShape<I>;
  using M = typename D::M;
  constexpr int LPR = M::LPR, CPL = M::CPL, RPS = M::RPS, NS = D::NS, ROWS = D::ROWS;
  constexpr int G = group_of<FMT>();
  constexpr int HPT = (I + 255) / 256;  // 16-byte pieces of h per thread for k <= 8
  __shared__ uint16_t ys[8][ROWS];
  __shared__ __attribute__((aligned(16))) uint16_t hs[8 * I];

  const int nblk = H / ROWS;
  const int mb = blockIdx.x % nblk, t = blockIdx.x / nblk;
  const int m0 = mb * ROWS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane % LPR, q = lane / LPR;
  const SlotRef* slots = a.pre ? a.pre : a.slots;

  // 1. loads, in this order: the wave's first slot (its weights depend on
  // it), the combine's operands, the token's h, then the slot's scales and
  // weights.  Everything is unconditional with clamped indices, so the loads
  // go out back to back and each value is waited for only where it is used.
  // A wave without a slot (k < 4) works on the last one and discards it.
  const int j0 = min(wave, a.K - 1);
  const SlotRef sr0 = load_slot(slots + t * a.K + j0);
  uint16_t rwv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rwv[j] = a.rw[t * a.K + min(j, a.K - 1)];
  // (without a residual the load reads a harmless valid address, unused)
  const uint16_t resv = *(a.residual ? a.residual + (size_t)t * H + m0 + tid % ROWS : a.rw);
  const int npc = a.K * I / 8;
  const uint16_t* ht = a.hbuf + (size_t)t * a.K * I;
  uint4 hv[HPT];
#pragma unroll
  for (int u = 0; u < HPT; ++u) hv[u] = ldg16(ht + 8 * min(tid + 256 * u, npc - 1));

  // scales and weights of slot j (a rejected slot reads a harmless valid
  // address, the slot table)
  auto issue = [&](const SlotRef& sr, uint4 (&wv)[NS][CPL], uint32_t (&sv)[NS][CPL]) {
    const bool ok = __builtin_amdgcn_readfirstlane(sr.ok) != 0;
    const uint8_t* wd = ok ? sr.w + (size_t)I * H : (const uint8_t*)slots;  // after gate and up
    const uint8_t* sd = ok ? sr.s + 2 * (size_t)I * (H / G) : (const uint8_t*)slots;
    const size_t row_nib = ok ? I / 2 : 0, row_sc = ok ? I / G : 0;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        sv[st][i] = load_chunk_scale<FMT>(sd + (size_t)(m0 + st * RPS + q) * row_sc,
                                          ok ? li + LPR * i : 0);
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        wv[st][i] = ldg16(wd + (size_t)(m0 + st * RPS + q) * row_nib + (ok ? 16 * (li + LPR * i) : 0));
  };
  // y rows of slot j into ys (the dot products, one butterfly over LPR lanes)
  auto finish = [&](int j, const SlotRef& sr, const uint4 (&wv)[NS][CPL],
                    const uint32_t (&sv)[NS][CPL]) {
    const bool ok = __builtin_amdgcn_readfirstlane(sr.ok) != 0;
    bf16x2 hp[CPL][16];
#pragma unroll
    for (int i = 0; i < CPL; ++i) unpack16_lds(hs + j * I + 32 * (li + LPR * i), hp[i]);
    double p[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      p[st] = 0.0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) p[st] += chunk_dot<FMT>(wv[st][i], sv[st][i], hp[i]);
    }
    const double tot = seg_reduce<NS, LPR>(p, lane);
    if ((li % (LPR / NS)) == 0) {
      const int r = (li / (LPR / NS)) * RPS + q;
      const uint16_t y = ok ? f64_to_bf16(tot * (double)sr.td) : (uint16_t)0;
      ys[j][r] = y;
      if constexpr (DUMP) {
        if (a.dy) a.dy[((size_t)t * a.K + j) * H + m0 + r] = y;
      }
    }
  };

  uint4 wv[NS][CPL];
  uint32_t sv[NS][CPL];
  issue(sr0, wv, sv);
  __builtin_amdgcn_sched_barrier(0);
  // 2. h into LDS (its loads are older than the weights, so only they are
  // waited for here), then the first slot's rows
#pragma unroll
  for (int u = 0; u < HPT; ++u)
    if (tid + 256 * u < npc) *(uint4*)(hs + 8 * (tid + 256 * u)) = hv[u];
  lds_barrier();
  if (wave < a.K) finish(wave, sr0, wv, sv);
  // 3. slots 4..k-1 (k > 4), one more per wave
  for (int j = wave + 4; j < a.K; j += 4) {
    const SlotRef sr = load_slot(slots + t * a.K + j);
    issue(sr, wv, sv);
    finish(j, sr, wv, sv);
  }
  __syncthreads();
  if (tid < ROWS) {
    const int m = m0 + tid;
    uint16_t acc = 0;  // +0
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < a.K) acc = combine_step(acc, rwv[j], ys[j][tid]);
    if (a.residual) acc = residual_add(resv, acc);
    a.out[(size_t)t * H + m] = acc;
  }
}

template <int H, int I, int FMT, bool PRENORM, bool DUMP>
hipError_t launch_variant(const DecodeArgs& a, hipStream_t s) {
  // the pre-norm is shared by the four waves of a workgroup: they must belong
  // to one token
  if (PRENORM && ((I / GuShape<H>::RW) * a.K) % 4 != 0) return hipErrorInvalidValue;
  const int waves = a.T * a.K * ((I + GuShape<H>::RW - 1) / GuShape<H>::RW);
  const hipError_t e = launch_kernel(MOE_KERNEL_DECODE_GATE_UP, k_dec_gateup<H, FMT, PRENORM, DUMP>,
                                     dim3((waves + 3) / 4), dim3(256), 0, s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(MOE_KERNEL_DECODE_DOWN, k_dec_down<H, I, FMT, DUMP>,
                       dim3(a.T * (H / DnShape<I>::ROWS)), dim3(256), 0, s, a);
}

template <int H, int I, int FMT>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
  const bool pre = (a.flags & MOE_FLAG_PRENORM) != 0;
  const bool dump = a.du || a.dg || a.dv || a.dh || a.dy;
  if (pre) return dump ? launch_variant<H, I, FMT, true, true>(a, s)
                       : launch_variant<H, I, FMT, true, false>(a, s);
  return dump ? launch_variant<H, I, FMT, false, true>(a, s)
              : launch_variant<H, I, FMT, false, false>(a, s);
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, hipStream_t s) {
  if (a.H == 2048 && a.I == 1536) return launch_shape<2048, 1536, FMT>(a, s);
  if (a.H == 1024 && a.I == 768) return launch_shape<1024, 768, FMT>(a, s);
  if (a.H == 512 && a.I == 256) return launch_shape<512, 256, FMT>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int H, int I) {
  return (H == 2048 && I == 1536) || (H == 1024 && I == 768) || (H == 512 && I == 256);
}

hipError_t launch_resolve(const int32_t* ids, const uint8_t* const* wtab,
                          const uint8_t* const* stab, const float* tsc, int n, int per_layer,
                          int E, uint32_t flags, int* err, SlotRef* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const hipError_t e = launch_kernel(MOE_KERNEL_RESOLVE, k_resolve, dim3((n + 255) / 256), dim3(256),
                                     0, s, ids, wtab, stab, tsc, n, per_layer, E, flags, err, out);
  return e;
}

hipError_t launch_decode(const DecodeArgs& a, int fmt, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return fmt == MOE_SCALE_E4M3_G16 ? launch_fmt<MOE_SCALE_E4M3_G16>(a, s)
                                   : launch_fmt<MOE_SCALE_E8M0_G32>(a, s);
}

}  // namespace moe
