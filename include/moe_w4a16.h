/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) grouped top-k W4A16 MoE FFN.
 *
 * The operation ("LFM2.5-24B-A2B -- Packed MXFP4 Inference", sections "Model
 * and quantization" and "What was optimized / Grouped top-4 expert
 * execution"): for every token t and routing slot j with expert e = ids[t][j],
 *
 *     u      = x[t], or the weightless RMS pre-norm of x[t] (MOE_FLAG_PRENORM)
 *     g      = bf16(Wg_e u)          grouped gate GEMV, FP32 accumulation
 *     v      = bf16(Wu_e u)          grouped up GEMV
 *     h      = bf16(silu(g) * v)     activation and multiplication
 *     y_j    = bf16(Wd_e h)          grouped down GEMV
 *     out[t] = sequential BF16 combine over slots 0..k-1 of bf16(w[t][j] * y_j),
 *              each product and each add rounded to BF16 separately, starting
 *              from +0; then, with a residual, out = bf16(residual + out).
 *
 * Expert weights stay packed: E2M1 FP4 values two per byte with one E8M0
 * scale per 32 values (MOE_SCALE_E8M0_G32, the MXFP4 card's format; codes
 * 1..254, i.e. 2^-126 .. 2^127, are supported and decode exactly, including
 * to BF16 subnormals and infinities; code 0 (2^-127) and the NaN code 255
 * are outside the supported input range), or one
 * E4M3FN scale per 16 values plus an FP32 per-expert tensor scale shared by
 * gate and up and a second one for down (MOE_SCALE_E4M3_G16, the NVFP4
 * weight-only variant of "primitive-ai/LFM2.5-24B-A2B-NVFP4A16", section
 * "What's quantized to what").  Activations and outputs are BF16.
 *
 * Packed layout (the only layout; one expert):
 *   packed_weights[e] -> gate [I][H/2] | up [I][H/2] | down [H][I/2]  bytes
 *   scales[e]         -> gate [I][H/G] | up [I][H/G] | down [H][I/G]  bytes
 * Matrices are [out][in], row-major.  Byte i of a row holds element 2i in bits
 * 0..3 and element 2i+1 in bits 4..7.  The scale of element (n, k) is byte
 * k / G of row n (G = 32 for E8M0, 16 for E4M3FN).  The two bases may point
 * into one contiguous buffer per expert (nibbles then scales: the "expert
 * triplet as one contiguous byte buffer" of the MXFP4 card's "Bounded pinned
 * RAM expert cache").  Every base must be 16-byte aligned (256 recommended).
 *
 * Pointer tables.  packed_weights and scales are DEVICE arrays of E device
 * pointers, built once per layer by the caller and kept ("Direct reads from
 * GPU-resident weights": resident experts are read in place through
 * persistent device pointer tables, with no staging copy).  Kernels read the
 * tables and expert_ids on the device, so both may change between calls or
 * between replays of a captured HIP graph without re-capture ("GPU routing
 * inside resident-layer graphs": selection is recomputed on every replay and
 * ids are never copied back to the CPU).  The library never reads device data
 * on the host and never synchronises in a forward call.
 *
 * Ownership.  The caller owns every buffer: inputs, tables, weights, outputs
 * and the workspace.  The library allocates and frees nothing in the calls
 * below and keeps no device state between calls.  All device work is
 * enqueued on cfg->stream (a hipStream_t; NULL = the default stream) and the
 * call returns without waiting.  Calls that share a workspace must be
 * ordered (same stream, or synchronised); distinct workspaces and streams
 * may run concurrently.
 *
 * Errors.  Every int-returning function returns MOE_OK (0) or a negative
 * MOE_ERR_* code.  Argument checks read only host values (cfg fields and
 * pointer values), run before anything is enqueued, and leave nothing
 * enqueued on failure.  moe_w4a16_last_error() gives a message for the
 * calling thread's last failure.  Invalid expert ids or misaligned expert
 * bases inside the device tables cannot be seen on the host: they are
 * undefined behaviour unless MOE_FLAG_CHECK_IDS is set, in which case the
 * kernels skip the bad slot, write an error word into the workspace and
 * moe_w4a16_device_status() reports it.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_W4A16_ABI_VERSION 1

/* return codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)          /* null pointer, bad enum, T < 0, aliasing, ... */
#define MOE_ERR_UNSUPPORTED_SHAPE (-2)    /* hidden / inter / top_k / experts not supported */
#define MOE_ERR_MISALIGNED (-3)           /* a pointer breaks its documented alignment */
#define MOE_ERR_WORKSPACE_TOO_SMALL (-4)  /* workspace_bytes < moe_w4a16_workspace_bytes() */
#define MOE_ERR_ABI_MISMATCH (-5)         /* cfg->abi_version != MOE_W4A16_ABI_VERSION */
#define MOE_ERR_HIP (-6)                  /* a HIP runtime call failed (text in last_error) */
#define MOE_ERR_DEVICE_CHECK (-7)         /* a device-side check (MOE_FLAG_CHECK_IDS) failed */

/* scale formats */
#define MOE_SCALE_E8M0_G32 0  /* E8M0 2^(e-127), one per 32 values along K (MXFP4) */
#define MOE_SCALE_E4M3_G16 1  /* E4M3FN, one per 16 values, times an FP32 tensor scale */

/* flags */
#define MOE_FLAG_PRENORM (1u << 0)        /* u = bf16(x * rsqrt(mean(x^2) + prenorm_eps)) */
#define MOE_FLAG_FORCE_DECODE (1u << 1)   /* use the per-token GEMV path for any T */
#define MOE_FLAG_FORCE_BATCHED (1u << 2)  /* use the sorted MFMA path even at T = 1 */
#define MOE_FLAG_CHECK_IDS (1u << 3)      /* device-side id / alignment checks */
/* Serial expert execution, the ablation of the grouped engine ("LFM2.5-24B-A2B
 * -- Packed MXFP4 Inference", "Grouped top-4 expert execution": the original
 * runner executed each selected expert separately).  T = 1 on the decode path
 * only: every slot j runs its own gate/up and down launches, which write y_j,
 * and one combine launch follows (2k + 1 launches per layer instead of 2).
 * Same device functions, so the results equal the grouped path's bit for bit. */
#define MOE_FLAG_SERIAL (1u << 4)
/* W4A4: the expert activations are 4-bit as well ("primitive-ai/LFM2.5-24B-
 * A2B-NVFP4A16", "Why this quant": the W4A4 builds quantise the expert
 * activations too and run on FP4 matrix hardware).  u and every h are
 * quantised to MXFP4 before the GEMV that reads them: per block of 32 along
 * K, E8M0 scale X = 2^(floor(log2 max|v|) - 2) (exponent clamped to
 * -127..127; a zero block takes 2^-127) and E2M1 elements nearest to v / X,
 * ties to the even code, saturating at 6, sign kept (the weights' own
 * format, with the OCP MX conversion rule).  Both operands then go to the
 * gfx950 block-scaled FP4 MFMA.  Needs MOE_SCALE_E8M0_G32; runs the sorted
 * batched kernels for every T (not with FORCE_DECODE or SERIAL).  The
 * results are the oracle's W4A4 layer, not the W4A16 one. */
#define MOE_FLAG_W4A4 (1u << 5)

typedef struct moe_w4a16_cfg {
  int32_t abi_version;         /* MOE_W4A16_ABI_VERSION */
  int32_t num_tokens;          /* T >= 0; T = 0 is a no-op */
  int32_t hidden;              /* H; see moe_w4a16_shape_supported() */
  int32_t inter;               /* I, the expert intermediate size */
  int32_t num_experts;         /* E, 1..1024 */
  int32_t top_k;               /* k, 1..8 */
  int32_t scale_fmt;           /* MOE_SCALE_* */
  uint32_t flags;              /* MOE_FLAG_* */
  const float* tensor_scales;  /* device [E][2] FP32 {gate_up, down}: required for
                                  E4M3, must be NULL for E8M0 */
  const void* residual;        /* optional device BF16 [T][H]; may alias x */
  float prenorm_eps;           /* used with MOE_FLAG_PRENORM */
  int32_t reserved0;
  void* workspace;             /* device, 256-byte aligned, see below */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t or NULL */
} moe_w4a16_cfg;

/* Debug dumps: device BF16 buffers, each optional (NULL = not written). */
typedef struct moe_w4a16_dump {
  void* u;  /* [T][H]     activation fed to gate/up (after the pre-norm) */
  void* g;  /* [T][k][I]  gate outputs */
  void* v;  /* [T][k][I]  up outputs */
  void* h;  /* [T][k][I]  silu(g) * v */
  void* y;  /* [T][k][H]  down outputs, before the combine */
} moe_w4a16_dump;

/* MOE_W4A16_ABI_VERSION of the loaded library. */
int moe_w4a16_abi_version(void);

/* Message of the calling thread's last failed call ("" if none). */
const char* moe_w4a16_last_error(void);

/* 1 if (hidden, inter) is supported for the given token count and flags
 * (both must be multiples of 256 and at most 16384; the one-launch decode
 * path used at T = 1 is compiled for hidden/inter pairs (2048, 1536),
 * (1024, 768) and (512, 256); other pairs fall back to the batched path). */
int moe_w4a16_shape_supported(int32_t hidden, int32_t inter);

/* Workspace bytes needed by moe_w4a16_forward / _forward_debug /
 * _stack_forward with this cfg (it depends on T, H, I, E, k and flags).
 * Returns 0 for an invalid cfg. */
size_t moe_w4a16_workspace_bytes(const moe_w4a16_cfg* cfg);

/* Zero-fill a workspace on `stream` (a kernel, not a memset node, so it can
 * be captured).  A workspace must be zeroed once before its first use.  Its
 * control words (the device error word and the router's per-token counters)
 * sit at fixed offsets at its start, whatever the cfg, and every call leaves
 * the counters at zero again, so one workspace zeroed once may serve calls
 * of different cfgs (each at least moe_w4a16_workspace_bytes of its cfg). */
int moe_w4a16_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * One MoE layer: out = combine(experts(x)) (+ residual), all in BF16.
 *   x          device BF16 [T][H], 16-byte aligned
 *   expert_ids device int32 [T][k]; duplicates within a token are allowed
 *              (each slot is computed on its own)
 *   route_w    device BF16 [T][k] routing coefficients
 *   packed_weights, scales   device tables [E] of device pointers (layout above)
 *   out        device BF16 [T][H], 16-byte aligned, must not overlap x
 * T = 1 uses the decode path (one gate/up GEMV launch for all k experts,
 * then one down GEMV launch that also does the combine); T > 1 uses the
 * batched path (grouped BF16-MFMA GEMMs whose workgroups group the
 * (token, slot) pairs by expert on the device, then the combine).
 */
int moe_w4a16_forward(const void* x, const int32_t* expert_ids, const void* route_w,
                      const void* const* packed_weights, const void* const* scales,
                      void* out, const moe_w4a16_cfg* cfg);

/* moe_w4a16_forward that also writes the intermediates named in `dump`
 * (device pointers; dump may be NULL).  Same kernels, same results. */
int moe_w4a16_forward_debug(const void* x, const int32_t* expert_ids, const void* route_w,
                            const void* const* packed_weights, const void* const* scales,
                            void* out, const moe_w4a16_cfg* cfg, const moe_w4a16_dump* dump);

/*
 * moe_w4a16_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, the same kernels and the same results, with
 * cfg->workspace and cfg->workspace_bytes ignored.  The workspace is a
 * file-scope device array of the library, 4 MiB (4,194,304 bytes) on each
 * GPU it runs on, held until the process ends; the call allocates and frees
 * nothing.  A call whose moe_w4a16_workspace_bytes(cfg) exceeds 4 MiB (at
 * hidden 2048 / inter 1536 / 64 experts / top-4: more than 77 tokens) fails
 * with MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued;
 * MOE_FLAG_CHECK_IDS is rejected (MOE_ERR_INVALID_ARG: its error word would
 * have no reader).  Every call on one GPU shares that GPU's array, and no
 * part of it needs to start at zero (each call writes every region before it
 * reads it), but calls that overlap in time on one GPU -- on different
 * streams, or from different threads without ordering -- race on it.
 */
int moe_w4a16_forward_noalloc(const void* x, const int32_t* expert_ids, const void* route_w,
                              const void* const* packed_weights, const void* const* scales,
                              void* out, const moe_w4a16_cfg* cfg);

/*
 * L chained MoE layers (the 38-layer MoE stack of LFM2.5-24B-A2B, "Model and
 * quantization": 40 layers of which 38 are MoE), batch T:
 *     h_0 = x;  h_{l+1} = bf16(h_l + MoE_l(prenorm(h_l)));  out = h_L
 * with the weightless pre-norm always applied (cfg->prenorm_eps) and the
 * residual always the layer input (cfg->residual and MOE_FLAG_PRENORM are
 * ignored).  Layer l uses expert_ids + l*T*k, route_w + l*T*k (BF16),
 * packed_weights + l*E, scales + l*E and, for E4M3, tensor_scales + l*E*2.
 *   x, out      device BF16 [T][H]; out must not overlap x
 *   expert_ids  device int32 [L][T][k]; route_w device BF16 [L][T][k]
 *   packed_weights, scales   device tables [L][E]
 *   tensor_scales            device FP32 [L][E][2] (E4M3) or NULL (E8M0)
 * At T = 1 every layer is two decode launches (the routing slots of up to 64
 * layers are resolved to expert addresses by one extra launch); otherwise
 * each layer is one batched sequence (gate/up GEMM, down GEMM, combine),
 * whose combine also writes the next layer's pre-normed input into the
 * workspace, so only the first layer has a pre-norm launch.
 */
int moe_w4a16_stack_forward(int32_t num_layers, const void* x, const int32_t* expert_ids,
                            const void* route_w, const void* const* packed_weights,
                            const void* const* scales, const float* tensor_scales, void* out,
                            const moe_w4a16_cfg* cfg);

/*
 * The layer's router on the device ("LFM2.5-24B-A2B -- Packed MXFP4
 * Inference", "GPU routing inside resident-layer graphs": router projection,
 * sigmoid scores, expert bias where configured, dynamic top-k, routing
 * coefficients; nothing returns to the host):
 *   u        = x[t], or its weightless RMS pre-norm with MOE_FLAG_PRENORM
 *   logit[e] = sum_k u[k] * router_w[e][k]      (FP64)
 *   s[e] = sigmoid(logit[e]);  key c[e] = s[e] + expert_bias[e]
 *   expert_ids[t][0..k-1] = the k largest keys, descending; equal keys to
 *                           the smaller id
 *   route_w[t][j] = bf16(s[ids[t][j]] / sum over the k selected s)
 *   x           device BF16 [T][H], 16-byte aligned
 *   router_w    device BF16 [E][H], 16-byte aligned
 *   expert_bias device FP32 [E], or NULL (no bias)
 *   expert_ids  device int32 [T][k] (written);  route_w device BF16 [T][k] (written)
 * Uses cfg->num_tokens, hidden, num_experts (<= 256), top_k, flags, prenorm_eps,
 * workspace (the moe_w4a16_workspace_bytes of the cfg) and stream.
 */
int moe_w4a16_route(const void* x, const void* router_w, const float* expert_bias,
                    int32_t* expert_ids, void* route_w, const moe_w4a16_cfg* cfg);

/* moe_w4a16_route, then moe_w4a16_forward with the ids and coefficients it
 * wrote (both stay on the device; the buffers are the caller's). */
int moe_w4a16_forward_routed(const void* x, const void* router_w, const float* expert_bias,
                             const void* const* packed_weights, const void* const* scales,
                             void* out, int32_t* expert_ids, void* route_w,
                             const moe_w4a16_cfg* cfg);

/* moe_w4a16_stack_forward with the routing of every layer computed on the
 * device from that layer's pre-normed input: layer l routes with
 * router_w + l*E*H (BF16 [L][E][H]) and expert_bias + l*E (FP32 [L][E], or
 * NULL), writing expert_ids + l*T*k and route_w + l*T*k ([L][T][k]), then
 * runs its experts.  Each layer's routing depends on the previous layer's
 * output, as in the model. */
int moe_w4a16_stack_forward_routed(int32_t num_layers, const void* x, const void* router_w,
                                   const float* expert_bias, const void* const* packed_weights,
                                   const void* const* scales, const float* tensor_scales,
                                   void* out, int32_t* expert_ids, void* route_w,
                                   const moe_w4a16_cfg* cfg);

/*
 * Test hook: dequantise one packed [rows][cols] matrix to BF16 with the same
 * device decoders the GEMM kernels use.  E2M1 * E8M0 and E2M1 * E4M3FN are
 * exact in BF16, so the result is the exact dequantised value ("Model and
 * quantization": packed E2M1, E8M0 scale per 32 values).  No tensor scale is
 * applied.  nibbles [rows][cols/2], scales [rows][cols/G], out BF16
 * [rows][cols]; cols a multiple of 32, all device pointers.
 */
int moe_w4a16_dequant(const void* nibbles, const void* scales, int32_t rows, int32_t cols,
                      int32_t scale_fmt, void* out, void* stream);

/*
 * The order-preserving combine on its own ("Grouped top-4 expert execution":
 * the fused routing-weighted combination keeps the sequential BF16
 * multiply/add rounding), with the same device function the forward kernels
 * use: out[t][m] = fold over j = 0..k-1 of acc = bf16(acc + bf16(w[t][j] *
 * y[t][j][m])) from acc = +0, then bf16(residual[t][m] + acc) if residual.
 *   y device BF16 [T][k][H]; route_w BF16 [T][k]; residual BF16 [T][H] or NULL;
 *   out BF16 [T][H].
 */
int moe_w4a16_combine(const void* y, const void* route_w, const void* residual, void* out,
                      int32_t num_tokens, int32_t top_k, int32_t hidden, void* stream);

/*
 * The batched path's grouping step on its own: a stable counting sort of the
 * T*k (token, slot) pairs by expert id, on the device ("BatchedMetalSwitchGLU
 * serves S=64 by sorting (token, expert) pairs", visible-cx/LFM2.5-8B-A1B-CoreAI,
 * "Provenance").  counts [E], offsets [E+1] (offsets[0] = 0), perm [T*k] with
 * perm[i] = t*k + j, pairs of one expert contiguous and in (t, j) order.
 * All device int32 buffers; nothing is read back.  Ids outside [0, E) are
 * undefined behaviour (they are counted in no bin).
 */
int moe_w4a16_sort_pairs(const int32_t* expert_ids, int32_t num_tokens, int32_t top_k,
                         int32_t num_experts, int32_t* counts, int32_t* offsets, int32_t* perm,
                         void* stream);

/* Reads (and clears) the device error word of a workspace; synchronises
 * `stream`.  *host_code = 0 if no device check failed, else a bitmask:
 * 1 = expert id out of range, 2 = misaligned expert base.  Returns
 * MOE_ERR_DEVICE_CHECK when *host_code != 0. */
int moe_w4a16_device_status(void* workspace, int32_t* host_code, void* stream);

/* Measurement helper: stream-read `bytes` (multiple of 16) from device
 * memory `src` with 16-byte loads over the whole GPU (256 to 4096
 * workgroups, sized to the buffer) and write one word per workgroup to
 * `sink` (device, 4 * 4096 bytes), to measure the achievable HBM read
 * bandwidth next to the kernels above. */
int moe_w4a16_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * Measurement helpers for the floor of the batch-1 decode path (what the two
 * decode kernels of a layer would cost with no arithmetic).
 *
 * moe_w4a16_decode_floor: the launch sequence of moe_w4a16_stack_forward at
 *   T = 1 (same arguments, with `sink` in place of out: device, 16 KiB,
 *   16-byte aligned) in which each layer's two decode kernels are replaced
 *   by kernels with the same grid that resolve the same routing slots and
 *   issue the same loads in the same order -- the selected experts' nibbles
 *   and scales, x, h, the coefficients and the residual -- fold them with
 *   XOR (no dequantisation, no products, no reductions) and store the fold
 *   where the decode kernels store h (in the workspace) and the layer output
 *   (workspace buffers in turn, which the next layer reads as its input, as
 *   in the stack; the last layer's in `sink`).  Only the
 *   LFM2.5-24B-A2B shape (hidden 2048, inter 1536, top-4) with E8M0 scales;
 *   otherwise MOE_ERR_UNSUPPORTED_SHAPE.
 * moe_w4a16_empty_launch: one kernel of `workgroups` x `threads` (1..1024)
 *   threads that does nothing (it reads no memory; `sink` is a device word
 *   it never writes in practice).
 * moe_w4a16_read_burst: read `bytes` (a multiple of 16) at `src` (16-byte
 *   aligned) with bytes / (16 * 256 * loads_per_lane) workgroups of 256
 *   lanes, each lane issuing all of its `loads_per_lane` (1, 2, 4 or 8)
 *   16-byte loads before it uses any; `sink` as above.
 * moe_w4a16_grid_barrier: one kernel of `workgroups` (1 .. the device's CU
 *   count, so that all are resident at once) single-wave workgroups that
 *   pass `barriers` (0 .. 100000) grid-wide barriers: each workgroup adds 1
 *   to counter[0] (relaxed, agent scope) and polls it until every workgroup
 *   has arrived.  counter: device uint32 [2], zero on entry (counter[0] ends
 *   at workgroups * barriers; counter[1] gets bit 0 if a bounded poll gave
 *   up, so the kernel always ends).  Timing it with and without barriers
 *   gives the cost of one in-kernel grid dependency.
 */
int moe_w4a16_decode_floor(int32_t num_layers, const void* x, const int32_t* expert_ids,
                           const void* route_w, const void* const* packed_weights,
                           const void* const* scales, void* sink, const moe_w4a16_cfg* cfg);
int moe_w4a16_empty_launch(int32_t workgroups, int32_t threads, void* sink, void* stream);
int moe_w4a16_read_burst(const void* src, size_t bytes, int32_t loads_per_lane, void* sink,
                         void* stream);
int moe_w4a16_grid_barrier(int32_t workgroups, int32_t barriers, void* counter, void* stream);

/* Measurement helper: one wave that spins for `microseconds` (at most
 * 1,000,000) on the 100 MHz real-time counter, so that a host can enqueue
 * work behind it and the GPU then runs that work back to back. */
int moe_w4a16_delay(uint32_t microseconds, void* stream);

/* Kernel kinds reported by moe_w4a16_timing_end. */
#define MOE_KERNEL_DECODE_GATE_UP 1  /* decode: gate/up GEMV + SiLU*up, all k slots */
#define MOE_KERNEL_DECODE_DOWN 2     /* decode: down GEMV + combine (+ residual) */
#define MOE_KERNEL_RESOLVE 3         /* routing slots -> expert addresses */
#define MOE_KERNEL_BATCHED_GATE_UP 4 /* batched: grouped gate/up GEMM + SiLU*up */
#define MOE_KERNEL_BATCHED_DOWN 5    /* batched: grouped down GEMM */
#define MOE_KERNEL_COMBINE 6         /* slot-order combine (+ residual) */
#define MOE_KERNEL_SORT 7            /* moe_w4a16_sort_pairs */
#define MOE_KERNEL_DEQUANT 8         /* moe_w4a16_dequant */
#define MOE_KERNEL_STREAM_READ 9     /* moe_w4a16_stream_read */
#define MOE_KERNEL_ZERO 10           /* workspace fill */
#define MOE_KERNEL_DELAY 11          /* moe_w4a16_delay */
#define MOE_KERNEL_ROUTER 12         /* router projection, sigmoid, bias, top-k, coefficients */
#define MOE_KERNEL_PRENORM 13        /* batched: weightless RMS pre-norm of the layer input
                                        (under W4A4 also its MXFP4 rows) */
#define MOE_KERNEL_QUANT_X 14        /* batched W4A4 without pre-norm: x as MXFP4 rows */
#define MOE_KERNEL_FLOOR_GATE_UP 15  /* moe_w4a16_decode_floor: decode gate/up's loads only */
#define MOE_KERNEL_FLOOR_DOWN 16     /* moe_w4a16_decode_floor: decode down's loads only */
#define MOE_KERNEL_EMPTY 17          /* moe_w4a16_empty_launch */
#define MOE_KERNEL_READ_BURST 18     /* moe_w4a16_read_burst */
#define MOE_KERNEL_GRID_BARRIER 19   /* moe_w4a16_grid_barrier */

/*
 * Kernel timing (measurement only).  After moe_w4a16_timing_begin(capacity)
 * the calling thread's next `capacity` kernel launches of this library carry
 * a start and a stop HIP event that the kernel dispatch itself records
 * (hipExtLaunchKernel), so each pair spans exactly that kernel's execution
 * (launches into a stream under graph capture carry none).  The library
 * creates the events; moe_w4a16_timing_end waits for them, writes the
 * duration in milliseconds and the MOE_KERNEL_* kind of each timed launch,
 * in launch order, to the host arrays ms[] and kinds[] (room for `capacity`
 * entries), destroys the events and returns the number of launches written,
 * or a negative error (MOE_ERR_INVALID_ARG if more launches happened than
 * the capacity, or if timing was not begun on this thread).
 */
int moe_w4a16_timing_begin(int32_t capacity);
int moe_w4a16_timing_end(float* ms, int32_t* kinds, int32_t capacity);

/*
 * Hybrid (partially resident) layers ("LFM2.5-24B-A2B -- Packed MXFP4
 * Inference", "Hybrid mode" and "Bounded pinned RAM expert cache"), for when
 * HBM cannot hold every expert.  A handle owns a pinned RAM cache of expert
 * triplets with LRU eviction under a byte limit, a pinned table and id
 * buffer, and a small device table; the caller owns the device staging
 * buffer.  A triplet is one contiguous expert: gate, up and down nibbles
 * (nibble_bytes = 3 * inter * hidden / 2), then their scales, exactly as the
 * kernels read a resident expert.
 *
 * moe_w4a16_hybrid_create: triplet_bytes and nibble_bytes positive multiples
 *   of 256; cache_bytes / triplet_bytes >= staging_slots triplets of pinned
 *   memory (the cache's capacity); device_staging: device, 256-byte aligned,
 *   staging_slots * triplet_bytes bytes, owned by the caller and not touched
 *   by anything else while the handle is used; max_experts (<= 1024) and
 *   max_pairs bound E and T * k of later calls.  Allocates with
 *   hipHostMalloc/hipMalloc; *out receives the handle.
 *
 * moe_w4a16_hybrid_forward: one layer, as moe_w4a16_forward (same x, ids,
 *   route_w, out and cfg, whose stream is used), where expert e is either
 *   resident -- resident_w[e] and resident_s[e] (host arrays of device
 *   pointers) give its nibbles and scales -- or CPU-backed: both are NULL and
 *   host_src[e] is the host address of its triplet in the checkpoint
 *   (pageable memory that stays valid and unchanged; it is also the cache
 *   key).  The call (1) copies the ids to the host and synchronises the
 *   stream, (2) takes the distinct CPU-backed experts of the ids in order of
 *   first appearance (token-major, slot order; at most staging_slots of
 *   them), (3) for each, finds its triplet in the pinned cache or copies it
 *   there from host_src (a miss, evicting the least recently used), and
 *   enqueues one H2D copy into staging slot r, (4) enqueues the layer's
 *   composed pointer tables, and (5) runs the grouped layer.  Only routed CPU
 *   experts move.  The host work makes this call uncapturable; consecutive
 *   calls on one handle must use one stream.  Errors: MOE_ERR_INVALID_ARG for
 *   bad tables, ids out of range (checked on the host), too many routed CPU
 *   experts or a call larger than the handle's bounds; those of
 *   moe_w4a16_forward otherwise.
 *
 * moe_w4a16_hybrid_stats: stats4 = {calls, cache hits, cache misses, bytes
 *   copied to the GPU}.  moe_w4a16_hybrid_last_requests: the last call's
 *   routed CPU experts in request order and whether each hit the cache (room
 *   for `capacity` entries; *count receives the number).
 */
typedef struct moe_w4a16_hybrid moe_w4a16_hybrid;
int moe_w4a16_hybrid_create(int64_t triplet_bytes, int64_t nibble_bytes, int64_t cache_bytes,
                            int32_t staging_slots, void* device_staging, int32_t max_experts,
                            int32_t max_pairs, moe_w4a16_hybrid** out);
int moe_w4a16_hybrid_destroy(moe_w4a16_hybrid* handle);
int moe_w4a16_hybrid_forward(moe_w4a16_hybrid* handle, const void* x, const int32_t* expert_ids,
                             const void* route_w, const void* const* resident_w,
                             const void* const* resident_s, const void* const* host_src, void* out,
                             const moe_w4a16_cfg* cfg);
int moe_w4a16_hybrid_stats(const moe_w4a16_hybrid* handle, int64_t* stats4);
int moe_w4a16_hybrid_last_requests(const moe_w4a16_hybrid* handle, int32_t* experts,
                                   uint8_t* hits, int32_t capacity, int32_t* count);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
