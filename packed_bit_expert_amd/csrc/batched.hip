// Sorted batched path (concurrency-32 decode and S=64 prefill chunks).
//
// "visible-cx/LFM2.5-8B-A1B-CoreAI", "Provenance": the batched switch-GLU
// serves S=64 by sorting (token, expert) pairs, so each selected expert's
// packed weights are read once per call for all of its tokens.  Here:
//   1. k_sort: stable counting sort of the T*k pairs by expert, on device
//      (no id or count ever reaches the host: "GPU routing inside
//      resident-layer graphs" of the MXFP4 card);
//   2. k_bat_gemm<MODE 0>: per (expert, 128-row tile) workgroup, the expert's
//      token rows are staged in LDS, packed gate and up rows are dequantised
//      to BF16 MFMA operands in registers (exact, no BF16 copy in memory),
//      v_mfma_f32_16x16x32_bf16 accumulates in FP32, and the epilogue writes
//      h = bf16(silu(bf16 g) * bf16 u) per pair;
//   3. k_bat_gemm<MODE 1>: the same for down, writing y per (token, slot);
//   4. k_combine: the slot-order BF16 combine per token (+ residual).
// At these sizes the work is still HBM-bound (12-15 flop per weight byte
// against a BF16-MFMA ridge near 312): MFMA removes the multiply-adds from
// the VALU, which is left with the dequantisation.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBT = 512;  // threads per GEMM workgroup (8 waves)
constexpr int kBN = 128;  // output rows per GEMM workgroup (16 per wave)
constexpr int kKS = 256;  // contraction elements per step (64 per lane group)

// ---------------------------------------------------------------------------
// 1. stable counting sort of (token, slot) pairs by expert
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sort(const int32_t* __restrict__ ids, int npairs, int E,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm,
                                              int32_t* __restrict__ active,
                                              int32_t* __restrict__ nactive, int* err,
                                              uint32_t flags) {
  extern __shared__ int32_t sh[];  // cnt[E], base[E]
  int32_t* cnt = sh;
  int32_t* base = sh + E;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int p = tid; p < npairs; p += 256) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else bad = true;
  }
  if (bad && (flags & MOE_FLAG_CHECK_IDS)) atomicOr(err, kErrBadId);
  __syncthreads();
  if (tid == 0) {
    int run = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      offsets[e] = run;
      counts[e] = cnt[e];
      if (cnt[e] > 0 && active) active[na++] = e;
      run += cnt[e];
    }
    offsets[E] = run;
    if (nactive) *nactive = na;
  }
  __syncthreads();
  if (tid < 64) {
    // pairs in order, 64 at a time; equal experts within a chunk are ranked
    // by lane, so the scatter is stable
    for (int p0 = 0; p0 < npairs; p0 += 64) {
      const int p = p0 + lane;
      const int e = p < npairs ? ids[p] : -1;
      bool todo = e >= 0 && e < E;
      uint64_t pending = __ballot(todo);
      while (pending) {
        const int leader = __builtin_ctzll(pending);
        const int e0 = __shfl(e, leader);
        const uint64_t mask = __ballot(todo && e == e0);
        const int b0 = base[e0];
        if (todo && e == e0) {
          const uint64_t below = mask & ((1ull << lane) - 1ull);
          perm[b0 + __popcll(below)] = p;
          todo = false;
        }
        if (lane == leader) base[e0] = b0 + __popcll(mask);
        pending = __ballot(todo);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2./3. grouped GEMM on bf16 MFMA
// ---------------------------------------------------------------------------
// Lane (n = lane % 16, g = lane / 16) of a wave loads 32 contiguous bytes (64
// codes) of its weight row per K step: K indices [ks*256 + 64g, +64).  Dword d
// of that holds K = ks*256 + 64g + 8d + [0, 8), which is the lane's 8-element
// B operand of MFMA number d; the A operand (token rows in LDS) is read at the
// same K indices, so every MFMA pairs A and B on identical K (the order of
// the K terms inside the FP32 sum is the only freedom used).
struct Step {
  uint4 w[2][2];  // [matrix][half]
  uint32_t s[2];  // scale bytes of the 64 codes
};

template <int FMT, int NMAT>
__device__ __forceinline__ void load_step(Step& st, const uint8_t* const (&wrow)[2],
                                          const uint8_t* const (&srow)[2], int ks, int g) {
#pragma unroll
  for (int mt = 0; mt < NMAT; ++mt) {
    const uint8_t* src = wrow[mt] + ks * (kKS / 2) + 32 * g;
    st.w[mt][0] = ldg16(src);
    st.w[mt][1] = ldg16(src + 16);
    if constexpr (FMT == MOE_SCALE_E8M0_G32)
      st.s[mt] = ldg<uint16_t>(srow[mt] + ks * (kKS / 32) + 2 * g);
    else
      st.s[mt] = ldg<uint32_t>(srow[mt] + ks * (kKS / 16) + 4 * g);
  }
}

template <int FMT>
__device__ __forceinline__ bf16x8 step_operand(const Step& st, int mt, int d) {
  const uint4& h = st.w[mt][d >> 2];
  const uint32_t w = (d & 3) == 0 ? h.x : (d & 3) == 1 ? h.y : (d & 3) == 2 ? h.z : h.w;
  if constexpr (FMT == MOE_SCALE_E8M0_G32)
    return fp4x8_to_bf16x8(w, e8m0_f32((st.s[mt] >> (8 * (d >> 2))) & 255u));
  else
    return fp4x8_scaled_to_bf16x8(w, e4m3_f32((st.s[mt] >> (8 * (d >> 1))) & 255u));
}

// MFMAs chained in FP32 before their sum is added to the FP64 accumulators.
// A short chain of exact BF16 products is exact in FP32 unless it spans more
// than 24 bits, so the FP64 accumulation keeps the outputs correctly rounded
// to BF16 almost always (the same scheme as the decode path's runs of 8).
constexpr int kChain = 1;

template <int FMT, int NMAT>
__device__ __forceinline__ void step_mfma(const Step& st, const uint16_t* xs, int ldx, int ks,
                                          int ln, int g, bool two, double (&acc)[2][2][4]) {
  const uint16_t* arow0 = xs + ln * ldx + ks * kKS + 64 * g;
  const uint16_t* arow1 = arow0 + 16 * ldx;
#pragma unroll
  for (int d0 = 0; d0 < 8; d0 += kChain) {
    f32x4 part[NMAT][2];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) part[mt][0] = part[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = d0; d < d0 + kChain; ++d) {
      bf16x8 B[NMAT];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) B[mt] = step_operand<FMT>(st, mt, d);
      const bf16x8 A0 = *(const bf16x8*)(arow0 + 8 * d);
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
        part[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B[mt], part[mt][0], 0, 0, 0);
      if (two) {
        const bf16x8 A1 = *(const bf16x8*)(arow1 + 8 * d);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
          part[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B[mt], part[mt][1], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[mt][0][i] += (double)part[mt][0][i];
        acc[mt][1][i] += (double)part[mt][1][i];
      }
  }
}

// MODE 0: A = x rows (pre-normed if asked), B = gate and up -> h.
// MODE 1: A = h rows, B = down -> y.
template <int FMT, int MODE>
__global__ __launch_bounds__(kBT) void k_bat_gemm(BatchedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  constexpr int NMAT = MODE == 0 ? 2 : 1;
  constexpr int G = FMT == MOE_SCALE_E4M3_G16 ? 16 : 32;
  const int Kd = MODE == 0 ? a.H : a.I;
  const int Nd = MODE == 0 ? a.I : a.H;
  const int ntiles = Nd / kBN;
  const int ai = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
  if (ai >= *a.nactive) return;
  const int e = a.active[ai];
  const int M = a.counts[e], off = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, g = lane >> 4;
  const int n = tile * kBN + wave * 16 + ln;  // this lane's output row (B column)
  const int ldx = Kd + 8;                     // +16 B per row: conflict-free A reads

  const uint8_t* wb = a.wtab[e];
  const uint8_t* sb = a.stab[e];
  const bool aligned = ((((uintptr_t)wb) | ((uintptr_t)sb)) & 15u) == 0;
  if ((a.flags & MOE_FLAG_CHECK_IDS) && !aligned) {
    if (tid == 0) atomicOr(a.err, kErrAlign);
    return;
  }
  const size_t rowb = (size_t)Kd / 2, rows = (size_t)Kd / G;
  const uint8_t* wrow[2];
  const uint8_t* srow[2];
  if (MODE == 0) {
    wrow[0] = wb + n * rowb;
    wrow[1] = wrow[0] + (size_t)a.I * rowb;
    srow[0] = sb + n * rows;
    srow[1] = srow[0] + (size_t)a.I * rows;
  } else {
    wrow[0] = wrow[1] = wb + (size_t)a.I * a.H + n * rowb;
    srow[0] = srow[1] = sb + 2 * (size_t)a.I * (a.H / G) + n * rows;
  }
  double tscale = 1.0;
  if constexpr (FMT == MOE_SCALE_E4M3_G16) tscale = (double)a.tsc[2 * e + MODE];
  const int nks = Kd / kKS;

  for (int mc0 = 0; mc0 < M; mc0 += a.mc) {
    const int mcnt = min(a.mc, M - mc0);
    __syncthreads();
    // stage the chunk's A rows (zero rows pad the last M tile)
    const int k8s = Kd / 8;
    for (int idx = tid; idx < a.mc * k8s; idx += kBT) {
      const int r = idx / k8s, k8 = idx - r * k8s;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < mcnt) {
        const int pair = a.perm[off + mc0 + r];
        const uint16_t* src = MODE == 0 ? a.x + (size_t)(pair / a.K) * Kd : a.hbuf + (size_t)pair * Kd;
        v = ldg16(src + 8 * k8);
      }
      *(uint4*)(xs + r * ldx + 8 * k8) = v;
    }
    __syncthreads();
    if (MODE == 0) {
      const bool prenorm = (a.flags & MOE_FLAG_PRENORM) != 0;
      for (int r = wave; r < mcnt; r += kBT / 64) {
        uint16_t* row = xs + r * ldx;
        if (prenorm) {
          double ss = 0.0;
          for (int k = lane; k < Kd; k += 64) {
            const double f = bf2f(row[k]);
            ss += f * f;
          }
          ss = seg_finish<32, double>(ss, lane);
          const double den = sqrt(ss / (double)Kd + (double)a.eps);
          for (int k = lane; k < Kd; k += 64) row[k] = f64_to_bf16((double)bf2f(row[k]) / den);
        }
        if (a.du && tile == 0) {
          const int t = a.perm[off + mc0 + r] / a.K;
          for (int k = lane; k < Kd; k += 64) a.du[(size_t)t * Kd + k] = row[k];
        }
      }
      if (prenorm) __syncthreads();
    }

    double acc[2][2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][q][i] = 0.0;
    const bool two = mcnt > 16;
    Step cur, nxt;
    load_step<FMT, NMAT>(cur, wrow, srow, 0, g);
    nxt = cur;
    for (int ks = 0; ks < nks; ++ks) {
      if (ks + 1 < nks) load_step<FMT, NMAT>(nxt, wrow, srow, ks + 1, g);
      step_mfma<FMT, NMAT>(cur, xs, ldx, ks, ln, g, two, acc);
      cur = nxt;
    }

    // epilogue: lane holds D[m = 4g + i][n] of each M tile
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * q + 4 * g + i;
        if (m >= mcnt) continue;
        const int pair = a.perm[off + mc0 + m];
        if (MODE == 0) {
          const uint16_t gb = f64_to_bf16(acc[0][q][i] * tscale);
          const uint16_t ub = f64_to_bf16(acc[1][q][i] * tscale);
          const uint16_t h = silu_mul_bf16(gb, ub);
          const size_t o = (size_t)pair * a.I + n;
          a.hbuf[o] = h;
          if (a.dg) a.dg[o] = gb;
          if (a.dv) a.dv[o] = ub;
          if (a.dh) a.dh[o] = h;
        } else {
          const uint16_t y = f64_to_bf16(acc[0][q][i] * tscale);
          const size_t o = (size_t)pair * a.H + n;
          a.ybuf[o] = y;
          if (a.dy) a.dy[o] = y;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4. slot-order combine: 8 consecutive outputs per thread
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y,
                                                 const uint16_t* __restrict__ rw,
                                                 const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out, int K, int H) {
  const int t = blockIdx.y;
  const int m8 = blockIdx.x * 256 + threadIdx.x;
  if (8 * m8 >= H) return;
  uint16_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < K; ++j) {
    const uint16_t w = rw[t * K + j];
    const uint4 v = *(const uint4*)(y + ((size_t)t * K + j) * H + 8 * m8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = combine_step(acc[2 * q], w, (uint16_t)(w4[q] & 0xFFFFu));
      acc[2 * q + 1] = combine_step(acc[2 * q + 1], w, (uint16_t)(w4[q] >> 16));
    }
  }
  if (residual) {
    const uint4 v = *(const uint4*)(residual + (size_t)t * H + 8 * m8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = residual_add((uint16_t)(w4[q] & 0xFFFFu), acc[2 * q]);
      acc[2 * q + 1] = residual_add((uint16_t)(w4[q] >> 16), acc[2 * q + 1]);
    }
  }
  uint4 o;
  o.x = acc[0] | ((uint32_t)acc[1] << 16);
  o.y = acc[2] | ((uint32_t)acc[3] << 16);
  o.z = acc[4] | ((uint32_t)acc[5] << 16);
  o.w = acc[6] | ((uint32_t)acc[7] << 16);
  *(uint4*)(out + (size_t)t * H + 8 * m8) = o;
}

template <typename KernelT>
hipError_t allow_lds(KernelT kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int FMT>
hipError_t launch_batched_fmt(const BatchedArgs& a, hipStream_t s) {
  hipError_t err = launch_sort(a.ids, a.T * a.K, a.E, a.counts, a.offsets, a.perm, a.active,
                               a.nactive, a.err, a.flags, s);
  if (err != hipSuccess) return err;
  const size_t lds0 = (size_t)a.mc * (a.H + 8) * 2, lds1 = (size_t)a.mc * (a.I + 8) * 2;
  static bool attrs_set = false;  // benign race: every caller sets the same values
  if (!attrs_set) {
    if ((err = allow_lds(k_bat_gemm<FMT, 0>, 160 * 1024)) != hipSuccess) return err;
    if ((err = allow_lds(k_bat_gemm<FMT, 1>, 160 * 1024)) != hipSuccess) return err;
    attrs_set = true;
  }
  k_bat_gemm<FMT, 0><<<a.E * (a.I / kBN), kBT, lds0, s>>>(a);
  k_bat_gemm<FMT, 1><<<a.E * (a.H / kBN), kBT, lds1, s>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(a.ybuf, a.rw, a.residual, a.out, a.T, a.K, a.H, s);
}

}  // namespace

bool batched_supported(int H, int I) {
  return H > 0 && I > 0 && H % kKS == 0 && I % kKS == 0 && H <= 4096 && I <= 4096;
}

int batched_chunk_tokens(int H, int I) {
  const int kmax = H > I ? H : I;
  return (size_t)32 * (kmax + 8) * 2 <= 160 * 1024 ? 32 : 16;
}

hipError_t launch_sort(const int32_t* ids, int npairs, int E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* active, int32_t* nactive, int* err, uint32_t flags,
                       hipStream_t s) {
  k_sort<<<1, 256, (size_t)2 * E * sizeof(int32_t), s>>>(ids, npairs, E, counts, offsets, perm,
                                                         active, nactive, err, flags);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const uint16_t* rw, const uint16_t* residual,
                          uint16_t* out, int T, int K, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((H / 8 + 255) / 256, T);
  k_combine<<<grid, 256, 0, s>>>(y, rw, residual, out, K, H);
  return hipGetLastError();
}

hipError_t launch_batched(const BatchedArgs& a, int fmt, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return fmt == MOE_SCALE_E4M3_G16 ? launch_batched_fmt<MOE_SCALE_E4M3_G16>(a, s)
                                   : launch_batched_fmt<MOE_SCALE_E8M0_G32>(a, s);
}

}  // namespace moe
