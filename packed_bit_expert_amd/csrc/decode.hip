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
  // waves per slot: where a slot's rows take two load sets, two waves share
  // them (one set each), so that two waves per SIMD overlap their streams
  static constexpr int SPW = NS >= 2 ? 2 : 1;
  static constexpr int NSW = NS / SPW;  // load sets per wave
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

// LDS staging of activations in 80-byte segments: each 32-value (64-byte)
// segment of x or h is followed by 16 bytes of padding.  Every lane reads
// one segment piece by piece, 16 lanes of a row reading 16 consecutive
// segments with one instruction; at a 64-byte stride those 16 addresses
// fall into two 16-byte bank slots of every 128 bytes (an 8-way conflict),
// at 80 bytes they take 8 distinct slots of 128 bytes and 16 of 256.
constexpr int kSeg = 40;  // BF16 values per staged segment (32 + 8 padding)

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
  // Every table read comes before the error atomics (at a clamped index), so
  // the compiler knows nothing in this kernel has written those words yet and
  // reads them with scalar loads when the slot index is uniform: a vector
  // load here would leave a register pending where the path without this
  // call joins, and the compiler then waits for every load in flight (the
  // activations included) before the weight loads can go out.
  SlotRef r;
  r.pad = 0;
  const int e = ids[i];
  const int ec = min(max(e, 0), E - 1);
  r.w = wtab[ec];
  r.s = stab[ec];
  r.tg = tsc ? tsc[2 * ec] : 1.f;
  r.td = tsc ? tsc[2 * ec + 1] : 1.f;
  r.ok = 1;
  if ((flags & MOE_FLAG_CHECK_IDS) && (e < 0 || e >= E)) {
    if (err) atomicOr(err, kErrBadId);
    r.w = r.s = nullptr;
    r.tg = r.td = 1.f;
    r.ok = 0;
    return r;
  }
  if ((flags & MOE_FLAG_CHECK_IDS) && ((((uintptr_t)r.w) | ((uintptr_t)r.s)) & 15u)) {
    if (err) atomicOr(err, kErrAlign);
    r.tg = r.td = 1.f;
    r.ok = 0;
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

// Grouped gate/up GEMV + silu(g) * v.  A 256-thread workgroup is four
// waves of one (token, slot), each owning RW rows of gate and of up; their
// row sums meet in LDS at the end, where wave 0 finishes the workgroup's
// rows.  All loads of a wave are issued before any arithmetic; the
// activation slices come first because vmcnt retires loads in issue order.
// With PRENORM the workgroup stages x in LDS and computes the weightless RMS
// pre-norm once (FP64) for its four waves.  A rejected slot reads a harmless
// valid address and writes zeros, so the code after the loads is
// straight-line and each chunk waits only for its own load.
// The arguments its first loads depend on come first and one by one: the
// library is built with kernarg preloading (-amdgpu-kernarg-preload-count),
// so on gfx950 they arrive in SGPRs with the wave instead of through scalar
// loads of the kernarg segment; the rest stay in DecodeArgs.
template <int H, int I, int FMT, bool PRENORM, bool DUMP>
__global__ __launch_bounds__(256) void k_dec_gateup(const SlotRef* pre, SlotRef* slots_ws,
                                                    const uint16_t* x, uint64_t kmagic, int T,
                                                    int K, int E, uint32_t flags, DecodeArgs a) {
  using S = GuShape<H>;
  using M = typename S::M;
  constexpr int LPR = M::LPR, CPL = M::CPL, RPS = M::RPS, NS = S::NS, RW = S::RW;
  constexpr int G = group_of<FMT>();
  __shared__ __attribute__((aligned(16))) uint16_t xs[PRENORM ? (H / 32) * kSeg : 8];
  __shared__ double red[4];
  // The wave's slot and token, in scalar registers and without a division
  // by a run-time value: these indices stand in front of the first load.
  constexpr int per_slot = (I + RW - 1) / RW;
  static_assert(per_slot % 4 == 0, "the waves of a workgroup share one slot");
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  // all waves of a workgroup belong to one token (per_slot * K is a multiple of 4)
  const int nb = gw % per_slot, sj = gw / per_slot;
  const bool live = sj < T * K;
  const int sjc = live ? sj : T * K - 1;
  const int t = (int)(((uint64_t)(uint32_t)sjc * kmagic) >> 32), j = sjc - t * K;

  // 0. the slot's expert (one 32-byte load of the pre-resolved table; without
  // one the load reads the workspace table, a harmless valid address, and
  // the slot is resolved below), then the activations, so that both are in
  // flight together
  // the pre-norm chain first, from the slot load on (raised after it, the
  // compiler reads the slot through the scalar cache instead, and the step
  // measured 0.8% slower)
  if constexpr (PRENORM) __builtin_amdgcn_s_setprio(2);
  SlotRef sr = load_slot(pre ? pre + sjc : slots_ws);
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* xt = x + (size_t)t * H;
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
  if (!pre) {
    sr = resolve_slot(a.ids, a.wtab, a.stab, a.tsc, sjc, E, flags,
                      (nb == 0 && lane == 0 && live) ? a.err : nullptr);
    if (nb == 0 && lane == 0 && live) slots_ws[sj] = sr;
  }
  const bool ok = __builtin_amdgcn_readfirstlane(sr.ok) != 0;
  const uint8_t* wbase = ok ? sr.w : (const uint8_t*)slots_ws;
  const uint8_t* sbase = ok ? sr.s : (const uint8_t*)slots_ws;
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
      ss += sumsq8_bf16(xraw[u]);
    }
    ss = seg_finish<32, double>(ss, lane);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double rs = rsqrt_f64((red[0] + red[1] + red[2] + red[3]) / (double)H + (double)a.eps);
    // each thread rescales the pieces it holds in registers and stores them once
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int k8 = threadIdx.x + 256 * u;
      if (k8 >= H / 8) break;
      *(uint4*)(xs + kSeg * (k8 >> 2) + 8 * (k8 & 3)) = scale8_bf16(xraw[u], rs);
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) unpack16_lds(xs + kSeg * (li + LPR * i), xp[i]);
    if constexpr (DUMP) {
      if (a.du && nb < 4 && j == 0 && live)
        for (int k = threadIdx.x; k < H; k += 256)
          a.du[(size_t)t * H + k] = xs[kSeg * (k >> 5) + (k & 31)];
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

  // 4. the workgroup's row sums meet in LDS and wave 0 finishes its 4 * RW
  // rows, one lane each: BF16 g and v, SiLU(g) * v, the h store.  Per wave
  // the epilogue would run with only RW lanes active; once per workgroup its
  // instructions are issued a quarter as often.  The four waves share the
  // slot (per_slot is a multiple of 4) and hold consecutive row blocks.
  __shared__ double rsum[4][NS][RPS];  // [wave][load set][q = matrix + 2 * row]
  if ((li % (LPR / NS)) == 0) rsum[wave][li / (LPR / NS)][q] = tot;
  lds_barrier();
  if (wave != 0 || lane >= 4 * RW) return;
  const int w = lane / RW, r = lane % RW;
  const int v = r / (RPS / 2), qh = r % (RPS / 2);
  const int n = (nb + w) * RW + r;
  if (n >= I) return;
  const double tg = (double)sr.tg;
  uint16_t gb = f64_to_bf16(rsum[w][v][2 * qh] * tg), ub = f64_to_bf16(rsum[w][v][2 * qh + 1] * tg);
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

// Grouped down GEMV for ROWS output rows of every slot (SPW waves per slot,
// one load set of rows each), then the slot-order BF16 combine (+ residual)
// of those rows.  Each wave stages its slot's h (I BF16) in LDS once; every
// lane then takes its slices from there instead of re-reading them from L2.
// Leading arguments as in k_dec_gateup (preloaded into SGPRs).  KMAX (4 or
// 8) bounds k, so that at top-4 no load or LDS slot is spent on slots 5..8.
template <int H, int I, int FMT, bool DUMP, int KMAX>
__global__ __launch_bounds__(256 * DnShape<I>::SPW) void k_dec_down(const SlotRef* pre, const SlotRef* slots_ws,
                                                  const uint16_t* rw, const uint16_t* hbuf,
                                                  const uint16_t* residual, int K, DecodeArgs a) {
  using D = DnShape<I>;
  using M = typename D::M;
  constexpr int LPR = M::LPR, CPL = M::CPL, RPS = M::RPS, ROWS = D::ROWS;
  constexpr int SPW = D::SPW, NS = D::NSW;  // this wave's load sets
  constexpr int G = group_of<FMT>();
  constexpr int HPW = (I / 8 + 63) / 64;  // 16-byte pieces of one slot's h per lane
  __shared__ uint16_t ys[KMAX][ROWS];
  // each wave stages the h of its own slot in its own region: no workgroup
  // barrier stands between a wave's loads and its dot products
  __shared__ __attribute__((aligned(16))) uint16_t hs[4 * SPW][(I / 32) * kSeg];

  const int nblk = H / ROWS;
  const int mb = blockIdx.x % nblk, t = blockIdx.x / nblk;
  const int m0 = mb * ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // a scalar: the slot indices
  const int js = wave % 4, r0 = (wave / 4) * NS * RPS;  // the wave's slot and first row
  const int li = lane % LPR, q = lane / LPR;
  const SlotRef* slots = pre ? pre : slots_ws;

  // 1. loads, in this order: the wave's first slot (its weights depend on
  // it), the combine's operands, the token's h, then the slot's scales and
  // weights.  Everything is unconditional with clamped indices, so the loads
  // go out back to back and each value is waited for only where it is used.
  // A wave without a slot (k < 4) works on the last one and discards it.
  const int j0 = min(js, K - 1);
  const SlotRef sr0 = load_slot(slots + t * K + j0);
  uint16_t rwv[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) rwv[j] = rw[t * K + min(j, K - 1)];
  // (without a residual the load reads a harmless valid address, unused)
  const uint16_t resv = *(residual ? residual + (size_t)t * H + m0 + tid % ROWS : rw);
  auto load_h = [&](int j, uint4 (&hv)[HPW]) {
    const uint16_t* hj = hbuf + ((size_t)t * K + j) * I;
#pragma unroll
    for (int u = 0; u < HPW; ++u) hv[u] = ldg16(hj + 8 * min(lane + 64 * u, I / 8 - 1));
  };
  // piece pc & 3 of segment pc >> 2 (I is a multiple of 32); the lanes of
  // the wave read what the others wrote only after the wave's LDS writes,
  // which LDS performs in order
  auto stage_h = [&](const uint4 (&hv)[HPW]) {
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int pc = lane + 64 * u;
      if (pc < I / 8) *(uint4*)(&hs[wave][0] + kSeg * (pc >> 2) + 8 * (pc & 3)) = hv[u];
    }
    __builtin_amdgcn_wave_barrier();
  };
  uint4 hv[HPW];
  load_h(j0, hv);

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
        sv[st][i] = load_chunk_scale<FMT>(sd + (size_t)(m0 + r0 + st * RPS + q) * row_sc,
                                          ok ? li + LPR * i : 0);
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        wv[st][i] = ldg16(wd + (size_t)(m0 + r0 + st * RPS + q) * row_nib + (ok ? 16 * (li + LPR * i) : 0));
  };
  // y rows of slot j into ys (the dot products, one butterfly over LPR lanes)
  auto finish = [&](int j, const SlotRef& sr, const uint4 (&wv)[NS][CPL],
                    const uint32_t (&sv)[NS][CPL]) {
    const bool ok = __builtin_amdgcn_readfirstlane(sr.ok) != 0;
    bf16x2 hp[CPL][16];
#pragma unroll
    for (int i = 0; i < CPL; ++i) unpack16_lds(&hs[wave][0] + kSeg * (li + LPR * i), hp[i]);
    double p[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      p[st] = 0.0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) p[st] += chunk_dot<FMT>(wv[st][i], sv[st][i], hp[i]);
    }
    const double tot = seg_reduce<NS, LPR>(p, lane);
    if ((li % (LPR / NS)) == 0) {
      const int r = r0 + (li / (LPR / NS)) * RPS + q;
      const uint16_t y = ok ? f64_to_bf16(tot * (double)sr.td) : (uint16_t)0;
      ys[j][r] = y;
      if constexpr (DUMP) {
        if (a.dy) a.dy[((size_t)t * K + j) * H + m0 + r] = y;
      }
    }
  };

  uint4 wv[NS][CPL];
  uint32_t sv[NS][CPL];
  issue(sr0, wv, sv);
  __builtin_amdgcn_sched_barrier(0);
  // 2. the slot's h into the wave's LDS region (its loads are older than the
  // weights, so only they are waited for here), then the slot's rows
  stage_h(hv);
  if (js < K) finish(js, sr0, wv, sv);
  // 3. slots 4..k-1 (k > 4), one more per wave
  if constexpr (KMAX > 4) {
    for (int j = js + 4; j < K; j += 4) {
      const SlotRef sr = load_slot(slots + t * K + j);
      load_h(j, hv);
      issue(sr, wv, sv);
      stage_h(hv);
      finish(j, sr, wv, sv);
    }
  }
  __syncthreads();
  if (tid < ROWS) {
    const int m = m0 + tid;
    uint16_t acc = 0;  // +0
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < K) acc = combine_step(acc, rwv[j], ys[j][tid]);
    if (residual) acc = residual_add(resv, acc);
    a.out[(size_t)t * H + m] = acc;
  }
}

template <int H, int I, int FMT, bool PRENORM, bool DUMP>
hipError_t launch_variant(const DecodeArgs& a0, hipStream_t s) {
  // the pre-norm is shared by the four waves of a workgroup: they must belong
  // to one token
  if (PRENORM && ((I / GuShape<H>::RW) * a0.K) % 4 != 0) return hipErrorInvalidValue;
  if (a0.I != I || a0.H != H || a0.K < 1) return hipErrorInvalidValue;
  DecodeArgs a = a0;
  // floor(s / K) = (s * kmagic) >> 32 for every slot index s < 2^29 (kmagic =
  // floor(2^32 / K) + 1 = (2^32 + e) / K with 0 < e <= K, so the product
  // exceeds s / K by less than s * K / (K 2^32) < 1 / K)
  a.kmagic = (uint64_t)((1ull << 32) / (uint64_t)a.K) + 1;
  const int waves = a.T * a.K * ((I + GuShape<H>::RW - 1) / GuShape<H>::RW);
  const hipError_t e = launch_kernel(MOE_KERNEL_DECODE_GATE_UP, k_dec_gateup<H, I, FMT, PRENORM, DUMP>,
                                     dim3((waves + 3) / 4), dim3(256), 0, s, a.pre, a.slots, a.x,
                                     a.kmagic, a.T, a.K, a.E, a.flags, a);
  if (e != hipSuccess) return e;
  if (a.K <= 4)
    return launch_kernel(MOE_KERNEL_DECODE_DOWN, k_dec_down<H, I, FMT, DUMP, 4>,
                         dim3(a.T * (H / DnShape<I>::ROWS)), dim3(256 * DnShape<I>::SPW), 0, s, a.pre,
                         (const SlotRef*)a.slots, a.rw, (const uint16_t*)a.hbuf, a.residual, a.K, a);
  return launch_kernel(MOE_KERNEL_DECODE_DOWN, k_dec_down<H, I, FMT, DUMP, 8>,
                       dim3(a.T * (H / DnShape<I>::ROWS)), dim3(256 * DnShape<I>::SPW), 0, s, a.pre,
                       (const SlotRef*)a.slots, a.rw, (const uint16_t*)a.hbuf, a.residual, a.K, a);
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
