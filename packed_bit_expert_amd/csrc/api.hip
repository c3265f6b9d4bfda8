// C ABI of the W4A16 MoE library: argument checks, workspace layout, path
// selection.  Every check reads host values only (cfg fields and pointer
// values) and runs before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// The calling thread's last failure, for the library's other C entry points.
int moe::report(int code, const char* msg) {
  if (code == MOE_OK) return ok();
  return fail(code, "%s", msg);
}

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// Kernel timing state of the calling thread (moe_w4a16_timing_*).
struct Timing {
  std::vector<hipEvent_t> ev;  // two per launch
  std::vector<int32_t> kind;
  int n = 0;          // launches recorded
  bool on = false;
  bool overflow = false;
};
thread_local Timing g_timing;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// Workspace regions (offsets from the base, each 256-byte aligned).
constexpr int kStackGroup = 64;  // layers whose routing slots are resolved in one pass

struct Layout {
  size_t hbuf, hq, ybuf, ping, scratch, ubuf, xq, logits, slots, total;
};

Layout layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K) {
  Layout L;
  size_t off = kCtrlBytes;
  L.hbuf = off;
  off += align256((size_t)(T * K * I) * 2);
  L.hq = off;  // batched W4A4: h as MXFP4 rows (codes, scales, 16-byte padded)
  off += align256((size_t)(T * K) * ((I / 2 + I / 32 + 15) & ~(int64_t)15));
  L.ybuf = off;
  off += align256((size_t)(T * K * H) * 2);
  L.ping = off;
  off += align256((size_t)(T * H) * 2);
  L.scratch = off;  // serial mode: the per-slot launches' unused combine output
  off += align256((size_t)(T * H) * 2);
  L.ubuf = off;  // batched: the pre-normed layer input
  off += align256((size_t)(T * H) * 2);
  L.xq = off;  // batched W4A4: the pre-normed layer input as MXFP4 rows
  off += align256((size_t)T * ((H / 2 + H / 32 + 15) & ~(int64_t)15));
  L.logits = off;  // router logits, FP64 [T][E]
  off += align256((size_t)(T * E) * 8);
  L.slots = off;
  off += align256((size_t)(T * K) * kStackGroup * sizeof(SlotRef));
  L.total = off;
  return L;
}

int check_shape(const moe_w4a16_cfg* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->abi_version != MOE_W4A16_ABI_VERSION)
    return fail(MOE_ERR_ABI_MISMATCH, "cfg->abi_version %d, library %d", c->abi_version,
                MOE_W4A16_ABI_VERSION);
  if (c->num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens %d < 0", c->num_tokens);
  if (c->num_experts < 1 || c->num_experts > 1024)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "num_experts %d outside 1..1024", c->num_experts);
  if (c->top_k < 1 || c->top_k > 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "top_k %d outside 1..8", c->top_k);
  if (c->scale_fmt != MOE_SCALE_E8M0_G32 && c->scale_fmt != MOE_SCALE_E4M3_G16)
    return fail(MOE_ERR_INVALID_ARG, "scale_fmt %d unknown", c->scale_fmt);
  if (!moe_w4a16_shape_supported(c->hidden, c->inter))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "hidden %d / inter %d not supported", c->hidden,
                c->inter);
  const uint32_t known = MOE_FLAG_PRENORM | MOE_FLAG_FORCE_DECODE | MOE_FLAG_FORCE_BATCHED |
                         MOE_FLAG_CHECK_IDS | MOE_FLAG_SERIAL | MOE_FLAG_W4A4;
  if (c->flags & ~known) return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", c->flags);
  if ((c->flags & MOE_FLAG_FORCE_DECODE) && (c->flags & MOE_FLAG_FORCE_BATCHED))
    return fail(MOE_ERR_INVALID_ARG, "FORCE_DECODE and FORCE_BATCHED together");
  if ((c->flags & MOE_FLAG_SERIAL) &&
      (c->num_tokens > 1 || (c->flags & MOE_FLAG_FORCE_BATCHED) ||
       !decode_supported(c->hidden, c->inter)))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_SERIAL needs T <= 1 on the decode path");
  if ((c->flags & MOE_FLAG_W4A4) && (c->flags & (MOE_FLAG_FORCE_DECODE | MOE_FLAG_SERIAL)))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_W4A4 runs the batched kernels only");
  if ((c->flags & MOE_FLAG_W4A4) && c->scale_fmt != MOE_SCALE_E8M0_G32)
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_W4A4 needs E8M0 block scales");
  if ((c->flags & MOE_FLAG_FORCE_DECODE) && !decode_supported(c->hidden, c->inter))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "no decode kernel for hidden %d / inter %d",
                c->hidden, c->inter);
  if (c->scale_fmt == MOE_SCALE_E4M3_G16 && !c->tensor_scales)
    return fail(MOE_ERR_INVALID_ARG, "E4M3 scales need tensor_scales");
  if (c->scale_fmt == MOE_SCALE_E8M0_G32 && c->tensor_scales)
    return fail(MOE_ERR_INVALID_ARG, "tensor_scales must be NULL for E8M0 scales");
  if ((c->flags & MOE_FLAG_PRENORM) && !(c->prenorm_eps >= 0.f))
    return fail(MOE_ERR_INVALID_ARG, "prenorm_eps must be >= 0");
  return MOE_OK;
}

bool use_decode(const moe_w4a16_cfg* c) {
  if (c->flags & (MOE_FLAG_FORCE_BATCHED | MOE_FLAG_W4A4)) return false;
  if (c->flags & MOE_FLAG_FORCE_DECODE) return true;
  return c->num_tokens == 1 && decode_supported(c->hidden, c->inter);
}

struct Call {
  const void* x;
  const int32_t* ids;
  const void* rw;
  const void* const* wtab;
  const void* const* stab;
  const float* tsc;
  const void* residual;
  void* out;
  const moe_w4a16_dump* dump;
  bool x_normed = false;  // batched stack: the workspace's u already holds prenorm(x)
  bool norm_out = false;  // batched stack: the combine also writes prenorm(out) there
};

int check_call(const moe_w4a16_cfg* c, const Call& k) {
  int rc = check_shape(c);
  if (rc) return rc;
  const size_t T = (size_t)c->num_tokens;
  if (T == 0) return MOE_OK;
  if (!k.x || !k.ids || !k.rw || !k.wtab || !k.stab || !k.out)
    return fail(MOE_ERR_INVALID_ARG, "x, expert_ids, route_w, tables and out must be non-NULL");
  if (!c->workspace) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(k.x, 16) || !aligned(k.out, 16) || (k.residual && !aligned(k.residual, 16)))
    return fail(MOE_ERR_MISALIGNED, "x, out and residual must be 16-byte aligned");
  if (!aligned(k.ids, 4) || !aligned(k.rw, 2) || !aligned(k.wtab, 8) || !aligned(k.stab, 8))
    return fail(MOE_ERR_MISALIGNED, "ids, route_w or a pointer table is misaligned");
  if (k.tsc && !aligned(k.tsc, 4)) return fail(MOE_ERR_MISALIGNED, "tensor_scales misaligned");
  if (!aligned(c->workspace, 256)) return fail(MOE_ERR_MISALIGNED, "workspace not 256-byte aligned");
  const size_t act = T * (size_t)c->hidden * 2;
  if (overlap(k.x, act, k.out, act)) return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
  if (k.residual && overlap(k.residual, act, k.out, act) && k.residual != k.out)
    return fail(MOE_ERR_INVALID_ARG, "out partially overlaps residual");
  const size_t need = moe_w4a16_workspace_bytes(c);
  if (c->workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", c->workspace_bytes,
                need);
  if (k.dump) {
    const void* d[5] = {k.dump->u, k.dump->g, k.dump->v, k.dump->h, k.dump->y};
    for (int i = 0; i < 5; ++i)
      if (d[i] && !aligned(d[i], 2)) return fail(MOE_ERR_MISALIGNED, "dump buffer misaligned");
  }
  return MOE_OK;
}

// Serial expert execution (T = 1): slot j as a one-slot decode layer whose
// down launch writes y_j (its own one-slot combine goes to scratch), then the
// slot-order combine of all y_j with the residual.
int run_serial(const moe_w4a16_cfg* c, const DecodeArgs& a, uint16_t* ybuf, uint16_t* scratch,
               hipStream_t s) {
  const int K = a.K, H = a.H, I = a.I;
  uint16_t* y = a.dy ? a.dy : ybuf;
  for (int j = 0; j < K; ++j) {
    DecodeArgs b = a;
    b.ids = a.ids + j;
    b.rw = a.rw + j;
    b.K = 1;
    b.hbuf = a.hbuf + (size_t)j * I;
    b.slots = a.slots + j;
    b.pre = a.pre ? a.pre + j : nullptr;
    b.residual = nullptr;
    b.out = scratch;
    b.du = j == 0 ? a.du : nullptr;
    b.dg = a.dg ? a.dg + (size_t)j * I : nullptr;
    b.dv = a.dv ? a.dv + (size_t)j * I : nullptr;
    b.dh = a.dh ? a.dh + (size_t)j * I : nullptr;
    b.dy = y + (size_t)j * H;
    const hipError_t e = launch_decode(b, c->scale_fmt, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch (serial slot)");
  }
  const hipError_t e = launch_combine(y, a.rw, a.residual, a.out, 1, K, H, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int run_layer(const moe_w4a16_cfg* c, const Call& k, const SlotRef* pre = nullptr) {
  const int T = c->num_tokens;
  if (T == 0) return ok();
  hipStream_t s = (hipStream_t)c->stream;
  const Layout L = layout(T, c->hidden, c->inter, c->num_experts, c->top_k);
  uint8_t* ws = (uint8_t*)c->workspace;
  int* err = &((Ctrl*)ws)->err;
  const moe_w4a16_dump* d = k.dump;
  hipError_t e;
  if (use_decode(c)) {
    DecodeArgs a;
    a.x = (const uint16_t*)k.x;
    a.ids = k.ids;
    a.rw = (const uint16_t*)k.rw;
    a.wtab = (const uint8_t* const*)k.wtab;
    a.stab = (const uint8_t* const*)k.stab;
    a.tsc = k.tsc;
    a.residual = (const uint16_t*)k.residual;
    a.out = (uint16_t*)k.out;
    a.hbuf = (uint16_t*)(ws + L.hbuf);
    a.slots = (SlotRef*)(ws + L.slots);
    a.pre = pre;
    a.du = d ? (uint16_t*)d->u : nullptr;
    a.dg = d ? (uint16_t*)d->g : nullptr;
    a.dv = d ? (uint16_t*)d->v : nullptr;
    a.dh = d ? (uint16_t*)d->h : nullptr;
    a.dy = d ? (uint16_t*)d->y : nullptr;
    a.err = err;
    a.T = T;
    a.H = c->hidden;
    a.I = c->inter;
    a.K = c->top_k;
    a.E = c->num_experts;
    a.flags = c->flags;
    a.eps = c->prenorm_eps;
    if (c->flags & MOE_FLAG_SERIAL) return run_serial(c, a, (uint16_t*)(ws + L.ybuf),
                                                      (uint16_t*)(ws + L.scratch), s);
    e = launch_decode(a, c->scale_fmt, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
  }
  BatchedArgs a;
  a.x = (const uint16_t*)k.x;
  a.ids = k.ids;
  a.rw = (const uint16_t*)k.rw;
  a.wtab = (const uint8_t* const*)k.wtab;
  a.stab = (const uint8_t* const*)k.stab;
  a.tsc = k.tsc;
  a.residual = (const uint16_t*)k.residual;
  a.out = (uint16_t*)k.out;
  a.hbuf = (uint16_t*)(ws + L.hbuf);
  a.ybuf = (uint16_t*)(ws + L.ybuf);
  a.du = d ? (uint16_t*)d->u : nullptr;
  a.dg = d ? (uint16_t*)d->g : nullptr;
  a.dv = d ? (uint16_t*)d->v : nullptr;
  a.dh = d ? (uint16_t*)d->h : nullptr;
  a.dy = d ? (uint16_t*)d->y : nullptr;
  a.err = err;
  a.ubuf = (uint16_t*)(ws + L.ubuf);
  a.hq = ws + L.hq;
  a.xqbuf = ws + L.xq;
  a.xq = nullptr;
  a.unext = k.norm_out ? a.ubuf : nullptr;
  a.x_normed = k.x_normed;
  a.T = T;
  a.H = c->hidden;
  a.I = c->inter;
  a.K = c->top_k;
  a.E = c->num_experts;
  a.flags = c->flags;
  a.eps = c->prenorm_eps;
  if (c->flags & MOE_FLAG_CHECK_IDS) {
    // pairs that a device check drops must still combine as y = 0
    e = launch_zero(a.ybuf, (size_t)T * c->top_k * c->hidden * 2, s);
    if (e != hipSuccess) return hip_fail(e, "workspace clear");
    if (d && d->y) {
      e = launch_zero(d->y, (size_t)T * c->top_k * c->hidden * 2, s);
      if (e != hipSuccess) return hip_fail(e, "dump clear");
    }
  }
  e = launch_batched(a, c->scale_fmt, s);
  if (e != hipSuccess) return hip_fail(e, "batched launch");
  return ok();
}

}  // namespace

extern "C" {

int moe_w4a16_abi_version(void) { return MOE_W4A16_ABI_VERSION; }

const char* moe_w4a16_last_error(void) { return g_err; }

int moe_w4a16_shape_supported(int32_t hidden, int32_t inter) {
  return batched_supported(hidden, inter) ? 1 : 0;
}

size_t moe_w4a16_workspace_bytes(const moe_w4a16_cfg* cfg) {
  if (check_shape(cfg) != MOE_OK) return 0;
  return layout(cfg->num_tokens, cfg->hidden, cfg->inter, cfg->num_experts, cfg->top_k).total;
}

int moe_w4a16_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  hipError_t e = launch_zero(workspace, bytes, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "workspace init");
}

int moe_w4a16_forward_debug(const void* x, const int32_t* expert_ids, const void* route_w,
                            const void* const* packed_weights, const void* const* scales,
                            void* out, const moe_w4a16_cfg* cfg, const moe_w4a16_dump* dump) {
  Call k{x, expert_ids, route_w, packed_weights, scales, cfg ? cfg->tensor_scales : nullptr,
         cfg ? cfg->residual : nullptr, out, dump};
  int rc = check_call(cfg, k);
  if (rc) return rc;
  return run_layer(cfg, k);
}

int moe_w4a16_forward(const void* x, const int32_t* expert_ids, const void* route_w,
                      const void* const* packed_weights, const void* const* scales, void* out,
                      const moe_w4a16_cfg* cfg) {
  return moe_w4a16_forward_debug(x, expert_ids, route_w, packed_weights, scales, out, cfg,
                                 nullptr);
}

int moe_w4a16_stack_forward(int32_t num_layers, const void* x, const int32_t* expert_ids,
                            const void* route_w, const void* const* packed_weights,
                            const void* const* scales, const float* tensor_scales, void* out,
                            const moe_w4a16_cfg* cfg) {
  if (num_layers < 1) return fail(MOE_ERR_INVALID_ARG, "num_layers %d < 1", num_layers);
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  moe_w4a16_cfg lc = *cfg;
  lc.flags |= MOE_FLAG_PRENORM;
  lc.tensor_scales = tensor_scales;
  lc.residual = x;
  Call k{x, expert_ids, route_w, packed_weights, scales, tensor_scales, x, out, nullptr};
  int rc = check_call(&lc, k);
  if (rc) return rc;
  const int64_t T = lc.num_tokens, K = lc.top_k, E = lc.num_experts;
  if (T == 0) return ok();
  const Layout L = layout(T, lc.hidden, lc.inter, E, K);
  void* ping = (uint8_t*)lc.workspace + L.ping;
  SlotRef* slots = (SlotRef*)((uint8_t*)lc.workspace + L.slots);
  int* err = &((Ctrl*)lc.workspace)->err;
  const bool decode = use_decode(&lc);
  const void* src = x;
  for (int l = 0; l < num_layers; ++l) {
    const int g = l % kStackGroup;
    if (decode && g == 0) {
      // the routing slots of the next (up to) 64 layers, resolved in one pass
      const int nl = num_layers - l < kStackGroup ? num_layers - l : kStackGroup;
      hipError_t e = launch_resolve(
          expert_ids + (size_t)l * T * K, (const uint8_t* const*)(packed_weights + (size_t)l * E),
          (const uint8_t* const*)(scales + (size_t)l * E),
          tensor_scales ? tensor_scales + (size_t)l * E * 2 : nullptr, (int)(nl * T * K),
          (int)(T * K), (int)E, lc.flags, err, slots, (hipStream_t)lc.stream);
      if (e != hipSuccess) return hip_fail(e, "slot resolve launch");
    }
    void* dst = ((num_layers - 1 - l) % 2 == 0) ? out : ping;
    lc.residual = src;
    lc.tensor_scales = tensor_scales ? tensor_scales + (size_t)l * E * 2 : nullptr;
    Call kl{src, expert_ids + (size_t)l * T * K, (const uint16_t*)route_w + (size_t)l * T * K,
            packed_weights + (size_t)l * E, scales + (size_t)l * E, lc.tensor_scales, src, dst,
            nullptr};
    // batched: each layer's combine leaves the next layer's pre-normed input
    kl.x_normed = !decode && l > 0;
    kl.norm_out = !decode && l + 1 < num_layers;
    rc = run_layer(&lc, kl, decode ? slots + (size_t)g * T * K : nullptr);
    if (rc) return rc;
    src = dst;
  }
  return ok();
}

int moe_w4a16_decode_floor(int32_t num_layers, const void* x, const int32_t* expert_ids,
                           const void* route_w, const void* const* packed_weights,
                           const void* const* scales, void* sink, const moe_w4a16_cfg* cfg) {
  if (num_layers < 1) return fail(MOE_ERR_INVALID_ARG, "num_layers %d < 1", num_layers);
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  moe_w4a16_cfg lc = *cfg;
  lc.flags = (lc.flags & ~(uint32_t)MOE_FLAG_PRENORM) | MOE_FLAG_PRENORM;
  lc.tensor_scales = nullptr;
  lc.residual = x;
  Call k{x, expert_ids, route_w, packed_weights, scales, nullptr, x, sink, nullptr};
  int rc = check_call(&lc, k);
  if (rc) return rc;
  if (lc.num_tokens != 1 || lc.scale_fmt != MOE_SCALE_E8M0_G32 ||
      !decode_floor_supported(lc.hidden, lc.inter, lc.top_k) || (lc.flags & ~(uint32_t)MOE_FLAG_PRENORM))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "the decode floor mirrors T = 1, hidden 2048, inter 1536, top-4, E8M0, no flags");
  const int64_t T = 1, K = lc.top_k, E = lc.num_experts;
  const Layout L = layout(T, lc.hidden, lc.inter, E, K);
  uint8_t* ws = (uint8_t*)lc.workspace;
  SlotRef* slots = (SlotRef*)(ws + L.slots);
  int* err = &((Ctrl*)ws)->err;
  hipStream_t s = (hipStream_t)lc.stream;
  const void* src = x;
  for (int l = 0; l < num_layers; ++l) {
    const int g = l % kStackGroup;
    if (g == 0) {
      const int nl = num_layers - l < kStackGroup ? num_layers - l : kStackGroup;
      hipError_t e = launch_resolve(
          expert_ids + (size_t)l * T * K, (const uint8_t* const*)(packed_weights + (size_t)l * E),
          (const uint8_t* const*)(scales + (size_t)l * E), nullptr, (int)(nl * T * K), (int)(T * K),
          (int)E, lc.flags, err, slots, s);
      if (e != hipSuccess) return hip_fail(e, "slot resolve launch");
    }
    // as in the stack, each layer reads what the previous layer's down
    // kernel has just written: its output goes to one of two workspace
    // buffers in turn (the last layer's to sink), and the next layer reads it
    void* dst = l + 1 == num_layers ? sink : (void*)(ws + (l % 2 == 0 ? L.ping : L.scratch));
    hipError_t e = launch_decode_floor(slots + (size_t)g * T * K, (const uint16_t*)src,
                                       (uint16_t*)(ws + L.hbuf),
                                       (const uint16_t*)route_w + (size_t)l * T * K,
                                       (const uint16_t*)src, (uint16_t*)dst, s);
    if (e != hipSuccess) return hip_fail(e, "decode floor launch");
    src = dst;
  }
  return ok();
}

int moe_w4a16_empty_launch(int32_t workgroups, int32_t threads, void* sink, void* stream) {
  if (workgroups < 1 || threads < 1 || threads > 1024 || !sink)
    return fail(MOE_ERR_INVALID_ARG, "workgroups >= 1, threads 1..1024 and a sink are required");
  const hipError_t e = launch_empty(workgroups, threads, (uint32_t*)sink, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "empty launch");
}

int moe_w4a16_grid_barrier(int32_t workgroups, int32_t barriers, void* counter, void* stream) {
  if (workgroups < 1 || barriers < 0 || barriers > 100000 || !counter || !aligned(counter, 4))
    return fail(MOE_ERR_INVALID_ARG, "workgroups >= 1, barriers 0..100000, an aligned counter");
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device attributes");
  if (workgroups > ncu)
    return fail(MOE_ERR_INVALID_ARG, "workgroups %d above the %d CUs: not all resident at once",
                workgroups, ncu);
  e = launch_grid_barrier(workgroups, barriers, (uint32_t*)counter, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "grid barrier launch");
}

int moe_w4a16_read_burst(const void* src, size_t bytes, int32_t loads_per_lane, void* sink,
                         void* stream) {
  if (!src || !sink) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(MOE_ERR_INVALID_ARG, "loads_per_lane must be 1, 2, 4 or 8");
  if (bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
    return fail(MOE_ERR_MISALIGNED, "src needs 16-byte alignment and a multiple of 16 bytes");
  const hipError_t e = launch_read_burst(src, bytes, loads_per_lane, (uint32_t*)sink,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "read burst launch");
}

int moe_w4a16_dequant(const void* nibbles, const void* scales, int32_t rows, int32_t cols,
                      int32_t scale_fmt, void* out, void* stream) {
  if (!nibbles || !scales || !out) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (rows < 0 || cols <= 0 || cols % 32)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows %d / cols %d (cols must be a multiple of 32)",
                rows, cols);
  if (scale_fmt != MOE_SCALE_E8M0_G32 && scale_fmt != MOE_SCALE_E4M3_G16)
    return fail(MOE_ERR_INVALID_ARG, "scale_fmt %d unknown", scale_fmt);
  if (!aligned(nibbles, 16) || !aligned(out, 16) || !aligned(scales, 2))
    return fail(MOE_ERR_MISALIGNED, "nibbles and out need 16-byte alignment");
  hipError_t e = launch_dequant((const uint8_t*)nibbles, (const uint8_t*)scales, rows, cols,
                                scale_fmt, (uint16_t*)out, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "dequant launch");
}

int moe_w4a16_combine(const void* y, const void* route_w, const void* residual, void* out,
                      int32_t num_tokens, int32_t top_k, int32_t hidden, void* stream) {
  if (num_tokens < 0 || top_k < 1 || top_k > 8 || hidden <= 0 || hidden % 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T %d, k %d, H %d (H must be a multiple of 8)",
                num_tokens, top_k, hidden);
  if (num_tokens == 0) return ok();
  if (!y || !route_w || !out) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(y, 16) || !aligned(out, 16) || (residual && !aligned(residual, 16)) ||
      !aligned(route_w, 2))
    return fail(MOE_ERR_MISALIGNED, "y, out and residual need 16-byte alignment");
  hipError_t e = launch_combine((const uint16_t*)y, (const uint16_t*)route_w,
                                (const uint16_t*)residual, (uint16_t*)out, num_tokens, top_k,
                                hidden, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "combine launch");
}

int moe_w4a16_sort_pairs(const int32_t* expert_ids, int32_t num_tokens, int32_t top_k,
                         int32_t num_experts, int32_t* counts, int32_t* offsets, int32_t* perm,
                         void* stream) {
  if (num_tokens < 0 || top_k < 1 || top_k > 8 || num_experts < 1 || num_experts > 1024)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T %d, k %d, E %d", num_tokens, top_k, num_experts);
  if (!expert_ids || !counts || !offsets || (num_tokens > 0 && !perm))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(expert_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(perm, 4))
    return fail(MOE_ERR_MISALIGNED, "int32 buffers need 4-byte alignment");
  // the hook writes counts, offsets and perm only (no active-expert list)
  hipError_t e = launch_sort(expert_ids, num_tokens * top_k, num_experts, counts, offsets, perm,
                             nullptr, nullptr, nullptr, 0, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "sort launch");
}

int moe_w4a16_device_status(void* workspace, int32_t* host_code, void* stream) {
  if (!workspace || !host_code) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  int v = 0;
  hipError_t e = hipMemcpyAsync(&v, &((Ctrl*)workspace)->err, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "device status read");
  if (v) {
    const int zero = 0;
    e = hipMemcpyAsync(&((Ctrl*)workspace)->err, &zero, sizeof(int), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "device status clear");
  }
  *host_code = v;
  if (v) return fail(MOE_ERR_DEVICE_CHECK, "device check failed: code %d", v);
  return ok();
}

int moe_w4a16_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
    return fail(MOE_ERR_MISALIGNED, "src needs 16-byte alignment and a multiple of 16 bytes");
  hipError_t e = launch_stream_read(src, bytes, (uint32_t*)sink, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "stream read launch");
}

}  // extern "C"

namespace {

int check_route(const moe_w4a16_cfg* c, const void* x, const void* router_w,
                const float* expert_bias, const int32_t* ids, const void* rw) {
  int rc = check_shape(c);
  if (rc) return rc;
  if (!router_supported(c->hidden, c->num_experts, c->top_k))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "router needs hidden 512, 1024, 1536 or 2048, num_experts <= 256, top_k <= num_experts");
  if (c->num_tokens == 0) return MOE_OK;
  if (!x || !router_w || !ids || !rw) return fail(MOE_ERR_INVALID_ARG, "NULL router argument");
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(ids, 4) || !aligned(rw, 2) ||
      (expert_bias && !aligned(expert_bias, 4)))
    return fail(MOE_ERR_MISALIGNED, "router arguments misaligned (x, router_w: 16 bytes)");
  if (!c->workspace) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(c->workspace, 256)) return fail(MOE_ERR_MISALIGNED, "workspace not 256-byte aligned");
  const size_t need = moe_w4a16_workspace_bytes(c);
  if (c->workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", c->workspace_bytes,
                need);
  return MOE_OK;
}

// With k (the layer the ids are for) on the decode path, the router also
// resolves the slots it selects into the workspace's slot table, which is
// returned through pre for the layer's kernels.
int run_route(const moe_w4a16_cfg* c, const void* x, const void* router_w, const float* bias,
              int32_t* ids, void* rw, const Call* k = nullptr, const SlotRef** pre = nullptr) {
  const int T = c->num_tokens;
  if (pre) *pre = nullptr;
  if (T == 0) return ok();
  const Layout L = layout(T, c->hidden, c->inter, c->num_experts, c->top_k);
  uint8_t* ws = (uint8_t*)c->workspace;
  RouteResolve res;
  if (k && pre && use_decode(c) && !(c->flags & MOE_FLAG_SERIAL)) {
    res.wtab = (const uint8_t* const*)k->wtab;
    res.stab = (const uint8_t* const*)k->stab;
    res.tsc = k->tsc;
    res.flags = c->flags;
    res.err = &((Ctrl*)ws)->err;
    res.slots = (SlotRef*)(ws + L.slots);
  }
  const hipError_t e = launch_route(
      (const uint16_t*)x, (const uint16_t*)router_w, bias, T, c->hidden, c->num_experts, c->top_k,
      (c->flags & MOE_FLAG_PRENORM) != 0, c->prenorm_eps, (double*)(ws + L.logits),
      (uint32_t*)(ws + kRouterCountOff), ids, (uint16_t*)rw, res, (hipStream_t)c->stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  if (res.slots) *pre = res.slots;
  return ok();
}

}  // namespace

extern "C" int moe_w4a16_route(const void* x, const void* router_w, const float* expert_bias,
                               int32_t* expert_ids, void* route_w, const moe_w4a16_cfg* cfg) {
  const int rc = check_route(cfg, x, router_w, expert_bias, expert_ids, route_w);
  if (rc) return rc;
  return run_route(cfg, x, router_w, expert_bias, expert_ids, route_w);
}

extern "C" int moe_w4a16_forward_routed(const void* x, const void* router_w,
                                        const float* expert_bias,
                                        const void* const* packed_weights,
                                        const void* const* scales, void* out, int32_t* expert_ids,
                                        void* route_w, const moe_w4a16_cfg* cfg) {
  int rc = check_route(cfg, x, router_w, expert_bias, expert_ids, route_w);
  if (rc) return rc;
  Call k{x, expert_ids, route_w, packed_weights, scales, cfg->tensor_scales, cfg->residual, out,
         nullptr};
  rc = check_call(cfg, k);
  if (rc) return rc;
  const SlotRef* pre = nullptr;
  rc = run_route(cfg, x, router_w, expert_bias, expert_ids, route_w, &k, &pre);
  if (rc) return rc;
  return run_layer(cfg, k, pre);
}

extern "C" int moe_w4a16_stack_forward_routed(int32_t num_layers, const void* x,
                                              const void* router_w, const float* expert_bias,
                                              const void* const* packed_weights,
                                              const void* const* scales,
                                              const float* tensor_scales, void* out,
                                              int32_t* expert_ids, void* route_w,
                                              const moe_w4a16_cfg* cfg) {
  if (num_layers < 1) return fail(MOE_ERR_INVALID_ARG, "num_layers %d < 1", num_layers);
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  moe_w4a16_cfg lc = *cfg;
  lc.flags |= MOE_FLAG_PRENORM;
  lc.tensor_scales = tensor_scales;
  lc.residual = x;
  int rc = check_route(&lc, x, router_w, expert_bias, expert_ids, route_w);
  if (rc) return rc;
  Call k{x, expert_ids, route_w, packed_weights, scales, tensor_scales, x, out, nullptr};
  rc = check_call(&lc, k);
  if (rc) return rc;
  const int64_t T = lc.num_tokens, K = lc.top_k, E = lc.num_experts, H = lc.hidden;
  if (T == 0) return ok();
  const Layout L = layout(T, lc.hidden, lc.inter, E, K);
  void* ping = (uint8_t*)lc.workspace + L.ping;
  const void* src = x;
  for (int l = 0; l < num_layers; ++l) {
    void* dst = ((num_layers - 1 - l) % 2 == 0) ? out : ping;
    int32_t* ids_l = expert_ids + (size_t)l * T * K;
    void* rw_l = (uint16_t*)route_w + (size_t)l * T * K;
    lc.residual = src;
    lc.tensor_scales = tensor_scales ? tensor_scales + (size_t)l * E * 2 : nullptr;
    Call kl{src, ids_l, rw_l, packed_weights + (size_t)l * E, scales + (size_t)l * E,
            lc.tensor_scales, src, dst, nullptr};
    const SlotRef* pre = nullptr;
    rc = run_route(&lc, src, (const uint16_t*)router_w + (size_t)l * E * H,
                   expert_bias ? expert_bias + (size_t)l * E : nullptr, ids_l, rw_l, &kl, &pre);
    if (rc) return rc;
    const bool batched = !use_decode(&lc);
    kl.x_normed = batched && l > 0;
    kl.norm_out = batched && l + 1 < num_layers;
    rc = run_layer(&lc, kl, pre);
    if (rc) return rc;
    src = dst;
  }
  return ok();
}

namespace moe {

LaunchEvents timing_begin(int kind, hipStream_t s) {
  Timing& t = g_timing;
  LaunchEvents ev;
  if (!t.on || capturing(s)) return ev;
  if (t.n >= (int)t.kind.size()) {
    t.overflow = true;
    return ev;
  }
  t.kind[t.n] = kind;
  ev.start = t.ev[2 * t.n];
  ev.stop = t.ev[2 * t.n + 1];
  return ev;
}

void timing_end(const LaunchEvents& ev) {
  if (ev.start) ++g_timing.n;
}

}  // namespace moe

namespace {

void timing_release() {
  Timing& t = g_timing;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t = Timing();
}

}  // namespace

extern "C" int moe_w4a16_timing_begin(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "timing capacity %d outside 1..2^20", capacity);
  timing_release();
  Timing& t = g_timing;
  t.ev.resize(2 * (size_t)capacity, nullptr);
  for (auto& e : t.ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      timing_release();
      return hip_fail(r, "hipEventCreate");
    }
  }
  t.kind.assign(capacity, 0);
  t.on = true;
  return ok();
}

extern "C" int moe_w4a16_timing_end(float* ms, int32_t* kinds, int32_t capacity) {
  Timing& t = g_timing;
  if (!t.on) return fail(MOE_ERR_INVALID_ARG, "kernel timing was not begun on this thread");
  if (t.overflow) {
    timing_release();
    return fail(MOE_ERR_INVALID_ARG, "more launches than the timing capacity");
  }
  if (!ms || !kinds || capacity < t.n) {
    const int n = t.n;
    timing_release();
    return fail(MOE_ERR_INVALID_ARG, "output arrays missing or shorter than %d launches", n);
  }
  for (int i = 0; i < t.n; ++i) {
    hipError_t r = hipEventSynchronize(t.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms[i], t.ev[2 * i], t.ev[2 * i + 1]);
    if (r != hipSuccess) {
      timing_release();
      return hip_fail(r, "kernel timing events");
    }
    kinds[i] = t.kind[i];
  }
  const int n = t.n;
  timing_release();
  ok();
  return n;
}

extern "C" int moe_w4a16_delay(uint32_t microseconds, void* stream) {
  if (microseconds > 1000000u)
    return fail(MOE_ERR_INVALID_ARG, "delay %u us above 1,000,000", microseconds);
  const hipError_t e = launch_delay(microseconds, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "delay launch");
  return ok();
}

// ---------------------------------------------------------------------------
// moe_w4a16_forward_noalloc: moe_w4a16_forward without a caller workspace,
// for callers that cannot allocate device memory.  The workspace regions
// (h, y, the pre-normed input, the routing slots, ...) live in one
// file-scope device array per GPU; nothing is allocated or freed.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// The array's device address on each GPU (the name is only a host-side
// stand-in), looked up once per device with that device current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_INVALID_ARG, "device %d beyond the %d the no-alloc entry point serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(MOE_ERR_HIP, "scratch array address unusable");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_w4a16_forward_noalloc(const void* x, const int32_t* expert_ids,
                                         const void* route_w, const void* const* packed_weights,
                                         const void* const* scales, void* out,
                                         const moe_w4a16_cfg* cfg) {
  int rc = check_shape(cfg);
  if (rc) return rc;
  if (cfg->flags & MOE_FLAG_CHECK_IDS)
    return fail(MOE_ERR_INVALID_ARG,
                "MOE_FLAG_CHECK_IDS is not available without a caller workspace (the error word "
                "would have no reader)");
  const size_t need = moe_w4a16_workspace_bytes(cfg);
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of workspace; the no-alloc entry point has %zu "
                "(fewer tokens per call, or moe_w4a16_forward with a workspace)",
                need, kNoAllocScratchBytes);
  if (cfg->num_tokens == 0) return ok();
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  moe_w4a16_cfg lc = *cfg;
  lc.workspace = ws;
  lc.workspace_bytes = kNoAllocScratchBytes;
  Call k{x, expert_ids, route_w, packed_weights, scales, lc.tensor_scales, lc.residual, out,
         nullptr};
  rc = check_call(&lc, k);
  if (rc) return rc;
  return run_layer(&lc, k);
}
