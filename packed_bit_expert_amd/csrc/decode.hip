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

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// gate/up: K = H.  One row has C chunks; a wave covers RW rows of gate and of
// up (8 chunk loads per lane); C divides 64, so a lane always meets the same
// activation chunk (lane % C) and keeps it in 16 registers.
template <int H>
struct GuShape {
  static constexpr int C = H / 32;
  static_assert(C >= 8 && C <= 64 && (C & (C - 1)) == 0, "gate/up rows of 8..64 chunks");
  static constexpr int RW = 256 / C;
  static constexpr int RWG = 4 * RW;  // rows per 256-thread workgroup
};

// down: K = I.  A pattern of L loads per lane covers R whole rows (the chunk a
// lane meets repeats every L loads); P patterns give ROWS rows per wave.  A
// workgroup owns ROWS output rows for every slot (one wave per slot), so the
// combine is finished in the same workgroup.
template <int I>
struct DnShape {
  static constexpr int C = I / 32;
  static constexpr int L = C / gcd_c(C, 64);
  static constexpr int R = 64 * L / C;
  static constexpr int P = R >= 8 ? 1 : 8 / R;
  static constexpr int ROWS = R * P;
  static constexpr int NL = L * P;
  static_assert(ROWS <= 64 && (ROWS & (ROWS - 1)) == 0, "rows per wave");
};

template <int FMT>
constexpr int group_of() { return FMT == MOE_SCALE_E4M3_G16 ? 16 : 32; }

template <int FMT>
__device__ __forceinline__ uint32_t load_chunk_scale(const uint8_t* srow, int c) {
  if constexpr (FMT == MOE_SCALE_E8M0_G32) return srow[c];
  else return *(const uint16_t*)(srow + 2 * c);
}

__device__ __forceinline__ void unpack16(const uint16_t* p, bf16x2 (&xp)[16]) {
  const uint4* v = (const uint4*)p;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = v[q];
    xp[4 * q + 0] = __builtin_bit_cast(bf16x2, w.x);
    xp[4 * q + 1] = __builtin_bit_cast(bf16x2, w.y);
    xp[4 * q + 2] = __builtin_bit_cast(bf16x2, w.z);
    xp[4 * q + 3] = __builtin_bit_cast(bf16x2, w.w);
  }
}

// Resolves slot (t, j) to its expert's bases; with MOE_FLAG_CHECK_IDS an
// out-of-range id or a misaligned base marks the slot bad (its h and y are 0).
__device__ __forceinline__ bool resolve_expert(const DecodeArgs& a, int t, int j, int& e,
                                               const uint8_t*& wb, const uint8_t*& sb,
                                               bool report) {
  e = a.ids[t * a.K + j];
  wb = nullptr;
  sb = nullptr;
  if (a.flags & MOE_FLAG_CHECK_IDS) {
    if (e < 0 || e >= a.E) {
      if (report) atomicOr(a.err, kErrBadId);
      e = 0;
      return false;
    }
    wb = a.wtab[e];
    sb = a.stab[e];
    if ((((uintptr_t)wb) | ((uintptr_t)sb)) & 15u) {
      if (report) atomicOr(a.err, kErrAlign);
      return false;
    }
    return true;
  }
  wb = a.wtab[e];
  sb = a.stab[e];
  return true;
}

// Grouped gate/up GEMV + silu(g) * u for one (token, slot, row block).
template <int H, int FMT>
__global__ __launch_bounds__(256) void k_dec_gateup(DecodeArgs a) {
  using S = GuShape<H>;
  constexpr int C = S::C, RW = S::RW, RWG = S::RWG, G = group_of<FMT>();
  __shared__ __attribute__((aligned(16))) uint16_t xs[H];
  __shared__ double red[4];

  const int I = a.I;
  const int nblk = (I + RWG - 1) / RWG;
  int b = blockIdx.x;
  const int nb = b % nblk;
  b /= nblk;
  const int j = b % a.K, t = b / a.K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  int e;
  const uint8_t *wb, *sb;
  const bool ok = resolve_expert(a, t, j, e, wb, sb, tid == 0 && nb == 0);

  // 1. issue every weight load of this wave
  const int n0 = nb * RWG + wave * RW;
  const size_t mat_nib = (size_t)I * (H / 2), mat_sc = (size_t)I * (H / G);
  uint4 wv[8];
  uint32_t sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int f = 64 * i + lane;
    const int r = f / (2 * C), mat = (f / C) & 1, c = f % C;
    const int n = n0 + r;
    wv[i] = make_uint4(0u, 0u, 0u, 0u);
    sv[i] = 0u;
    if (ok && n < I) {
      wv[i] = *(const uint4*)(wb + mat * mat_nib + (size_t)n * (H / 2) + 16 * c);
      sv[i] = load_chunk_scale<FMT>(sb + mat * mat_sc + (size_t)n * (H / G), c);
    }
  }

  // 2. stage x (or its weightless RMS pre-norm, in FP64) in LDS
  const uint16_t* xt = a.x + (size_t)t * H;
  const bool prenorm = (a.flags & MOE_FLAG_PRENORM) != 0;
  double ss = 0.0;
  for (int k8 = tid; k8 < H / 8; k8 += 256) {
    const uint4 v = *(const uint4*)(xt + 8 * k8);
    *(uint4*)(xs + 8 * k8) = v;
    if (prenorm) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = __uint_as_float(w4[q] << 16), hi = __uint_as_float(w4[q] & 0xFFFF0000u);
        ss += lo * lo + hi * hi;
      }
    }
  }
  if (prenorm) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double den = sqrt((red[0] + red[1] + red[2] + red[3]) / (double)H + (double)a.eps);
    for (int k = tid; k < H; k += 256) xs[k] = f64_to_bf16((double)bf2f(xs[k]) / den);
  }
  __syncthreads();
  if (a.du && nb == 0 && j == 0)
    for (int k = tid; k < H; k += 256) a.du[(size_t)t * H + k] = xs[k];

  bf16x2 xp[16];
  unpack16(xs + 32 * (lane % C), xp);

  // 3. dot products, then one butterfly for all 8 chunk sums
  double p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = chunk_dot<FMT>(wv[i], sv[i], xp);
  const double tot = seg_reduce<8, C>(p, lane);
  const double oth = __shfl_xor(tot, C == 64 ? 8 : C);  // the same row of the other matrix

  const int s = lane / C;
  const int v = (lane % C) / (C / 8);
  const int mat = (C == 64) ? (v & 1) : (s & 1);
  const int r = (C == 64) ? (v >> 1) : (32 / C) * v + (s >> 1);
  const int n = n0 + r;
  if ((lane % (C / 8)) == 0 && mat == 0 && n < I) {
    double tg = 1.0;
    if constexpr (FMT == MOE_SCALE_E4M3_G16) tg = ok ? (double)a.tsc[2 * e] : 0.0;
    uint16_t gb = f64_to_bf16(tot * tg), ub = f64_to_bf16(oth * tg);
    uint16_t h = silu_mul_bf16(gb, ub);
    if (!ok) gb = ub = h = 0;
    const size_t o = ((size_t)t * a.K + j) * I + n;
    a.hbuf[o] = h;
    if (a.dg) a.dg[o] = gb;
    if (a.dv) a.dv[o] = ub;
    if (a.dh) a.dh[o] = h;
  }
}

// Grouped down GEMV for ROWS output rows of every slot, then the slot-order
// BF16 combine (+ residual) of those rows.
template <int H, int I, int FMT>
__global__ __launch_bounds__(256) void k_dec_down(DecodeArgs a) {
  using D = DnShape<I>;
  constexpr int C = D::C, L = D::L, R = D::R, ROWS = D::ROWS, NL = D::NL, G = group_of<FMT>();
  __shared__ uint16_t ys[8][ROWS];

  const int nblk = H / ROWS;
  const int mb = blockIdx.x % nblk, t = blockIdx.x / nblk;
  const int m0 = mb * ROWS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int j = wave; j < a.K; j += 4) {
    int e;
    const uint8_t *wb, *sb;
    const bool ok = resolve_expert(a, t, j, e, wb, sb, false);
    const uint8_t* wd = ok ? wb + (size_t)I * H : nullptr;              // after gate and up
    const uint8_t* sd = ok ? sb + 2 * (size_t)I * (H / G) : nullptr;
    uint4 wv[NL];
    uint32_t sv[NL];
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int pl = q / L, ql = q % L;
      const int f = 64 * ql + lane;
      const int m = m0 + pl * R + f / C, c = f % C;
      wv[q] = make_uint4(0u, 0u, 0u, 0u);
      sv[q] = 0u;
      if (ok) {
        wv[q] = *(const uint4*)(wd + (size_t)m * (I / 2) + 16 * c);
        sv[q] = load_chunk_scale<FMT>(sd + (size_t)m * (I / G), c);
      }
    }
    const uint16_t* hj = a.hbuf + ((size_t)t * a.K + j) * I;
    bf16x2 hp[L][16];
#pragma unroll
    for (int ql = 0; ql < L; ++ql) unpack16(hj + 32 * ((64 * ql + lane) % C), hp[ql]);

    double acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = 0.0;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int pl = q / L, ql = q % L;
      const double part = chunk_dot<FMT>(wv[q], sv[q], hp[ql]);
      const int rr = (64 * ql + lane) / C;
      const int lo = (64 * ql) / C, hi = (64 * ql + 63) / C;  // rows this load can touch
#pragma unroll
      for (int r = lo; r <= hi; ++r) acc[pl * R + r] += (rr == r) ? part : 0.0;
    }
    const double tot = seg_reduce<ROWS, 64>(acc, lane);
    if ((lane % (64 / ROWS)) == 0) {
      const int v = lane / (64 / ROWS);
      double td = 1.0;
      if constexpr (FMT == MOE_SCALE_E4M3_G16) td = ok ? (double)a.tsc[2 * e + 1] : 0.0;
      const uint16_t y = ok ? f64_to_bf16(tot * td) : (uint16_t)0;
      ys[j][v] = y;
      if (a.dy) a.dy[((size_t)t * a.K + j) * H + m0 + v] = y;
    }
  }
  __syncthreads();
  if (tid < ROWS) {
    const int m = m0 + tid;
    uint16_t acc = 0;  // +0
    for (int j = 0; j < a.K; ++j) acc = combine_step(acc, a.rw[t * a.K + j], ys[j][tid]);
    if (a.residual) acc = residual_add(a.residual[(size_t)t * H + m], acc);
    a.out[(size_t)t * H + m] = acc;
  }
}

template <int H, int I, int FMT>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
  const int g1 = a.T * a.K * ((I + GuShape<H>::RWG - 1) / GuShape<H>::RWG);
  k_dec_gateup<H, FMT><<<g1, 256, 0, s>>>(a);
  const int g2 = a.T * (H / DnShape<I>::ROWS);
  k_dec_down<H, I, FMT><<<g2, 256, 0, s>>>(a);
  return hipGetLastError();
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

hipError_t launch_decode(const DecodeArgs& a, int fmt, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return fmt == MOE_SCALE_E4M3_G16 ? launch_fmt<MOE_SCALE_E4M3_G16>(a, s)
                                   : launch_fmt<MOE_SCALE_E8M0_G32>(a, s);
}

}  // namespace moe
