// Hybrid (partially resident) MoE layers: the pinned RAM expert cache, the
// per-call H2D transfers of routed CPU-backed experts and the composed
// pointer tables.  Host code only; the layer itself runs through
// moe_w4a16_forward on the same kernels as a fully resident layer.
//
// "LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Hybrid mode" and "Bounded
// pinned RAM expert cache": a partially resident layer obtains its selected
// expert ids on the CPU; resident experts are read in place; each selected
// CPU-backed expert comes from a packed RAM cache of contiguous triplets (LRU
// under a memory limit) or, on a miss, from the checkpoint, and reaches the
// GPU with one H2D copy into a persistent staging buffer; then the grouped
// layer runs.  Only routed CPU experts are transferred, and the CPU steps stay
// outside graph capture.
#include <string.h>

#include <algorithm>
#include <list>
#include <thread>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "kernels.h"

struct moe_w4a16_hybrid {
  int64_t triplet = 0, nib = 0;
  int capacity = 0;          // pinned cache triplets
  int staging_slots = 0;
  int max_experts = 0, max_pairs = 0;
  uint8_t* pinned = nullptr; // [capacity][triplet], hipHostMalloc
  uint8_t* staging = nullptr;  // device [staging_slots][triplet], caller's
  void** tab_host = nullptr;   // pinned [2][max_experts]: composed tables
  void** tab_dev = nullptr;    // device [2][max_experts]
  int32_t* ids_host = nullptr; // pinned [max_pairs]
  // LRU: most recently used at the front; key = the expert's checkpoint address
  std::list<std::pair<const void*, int>> order;
  std::unordered_map<const void*, std::list<std::pair<const void*, int>>::iterator> where;
  int64_t calls = 0, hits = 0, misses = 0, h2d_bytes = 0;
  std::vector<int32_t> last_experts;
  std::vector<uint8_t> last_hits;
};

namespace {

int herr(hipError_t e, const char* what) {
  char b[256];
  snprintf(b, sizeof b, "%s: %s", what, hipGetErrorString(e));
  return moe::report(MOE_ERR_HIP, b);
}

void release(moe_w4a16_hybrid* h) {
  if (!h) return;
  if (h->pinned) (void)hipHostFree(h->pinned);
  if (h->tab_host) (void)hipHostFree(h->tab_host);
  if (h->ids_host) (void)hipHostFree(h->ids_host);
  if (h->tab_dev) (void)hipFree(h->tab_dev);
  delete h;
}

// The pinned slot of `key` under LRU: its slot on a hit; on a miss a free
// slot or the least recently used entry's, which the caller fills from the
// checkpoint.
int cache_slot(moe_w4a16_hybrid* h, const void* key, bool* hit) {
  auto it = h->where.find(key);
  if (it != h->where.end()) {
    h->order.splice(h->order.begin(), h->order, it->second);
    *hit = true;
    return it->second->second;
  }
  *hit = false;
  int slot;
  if ((int)h->order.size() < h->capacity) {
    slot = (int)h->order.size();
  } else {
    slot = h->order.back().second;
    h->where.erase(h->order.back().first);
    h->order.pop_back();
  }
  h->order.emplace_front(key, slot);
  h->where[key] = h->order.begin();
  return slot;
}

// n copies of `bytes` each (dst[i] <- src[i]), split over up to four host
// threads in contiguous pieces of the concatenated copies.
void parallel_copy(const std::vector<uint8_t*>& dst, const std::vector<const uint8_t*>& src,
                   size_t bytes) {
  const size_t total = dst.size() * bytes;
  if (total == 0) return;
  const int nt = total >= (4u << 20) ? 4 : 1;
  auto work = [&](int t) {
    size_t lo = total * t / nt, hi = total * (t + 1) / nt;
    while (lo < hi) {
      const size_t i = lo / bytes, off = lo % bytes, n = std::min(hi - lo, bytes - off);
      memcpy(dst[i] + off, src[i] + off, n);
      lo += n;
    }
  };
  std::vector<std::thread> pool;
  int spawned = 1;
  try {
    for (; spawned < nt; ++spawned) pool.emplace_back(work, spawned);
  } catch (...) {  // no thread to be had: the calling thread copies the rest
  }
  for (int t = spawned; t < nt; ++t) work(t);
  work(0);
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int moe_w4a16_hybrid_create(int64_t triplet_bytes, int64_t nibble_bytes, int64_t cache_bytes,
                            int32_t staging_slots, void* device_staging, int32_t max_experts,
                            int32_t max_pairs, moe_w4a16_hybrid** out) {
  if (!out) return moe::report(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (triplet_bytes <= 0 || nibble_bytes <= 0 || nibble_bytes >= triplet_bytes ||
      triplet_bytes % 256 || nibble_bytes % 256)
    return moe::report(MOE_ERR_INVALID_ARG,
                       "triplet and nibble bytes must be positive multiples of 256, nibbles first");
  if (staging_slots < 1 || max_experts < 1 || max_experts > 1024 || max_pairs < 1)
    return moe::report(MOE_ERR_INVALID_ARG, "staging_slots, max_experts and max_pairs must be >= 1");
  if (!device_staging || ((uintptr_t)device_staging & 255))
    return moe::report(device_staging ? MOE_ERR_MISALIGNED : MOE_ERR_INVALID_ARG,
                       "device_staging must be a 256-byte aligned device buffer");
  if (cache_bytes / triplet_bytes < staging_slots)
    return moe::report(MOE_ERR_INVALID_ARG,
                       "the pinned cache must hold at least staging_slots triplets");
  auto* h = new moe_w4a16_hybrid;
  h->triplet = triplet_bytes;
  h->nib = nibble_bytes;
  h->capacity = (int)(cache_bytes / triplet_bytes);
  h->staging_slots = staging_slots;
  h->staging = (uint8_t*)device_staging;
  h->max_experts = max_experts;
  h->max_pairs = max_pairs;
  hipError_t e = hipHostMalloc((void**)&h->pinned, (size_t)h->capacity * triplet_bytes, hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc((void**)&h->tab_host, 2 * sizeof(void*) * max_experts, hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc((void**)&h->ids_host, sizeof(int32_t) * max_pairs, hipHostMallocDefault);
  if (e == hipSuccess) e = hipMalloc((void**)&h->tab_dev, 2 * sizeof(void*) * max_experts);
  if (e != hipSuccess) {
    release(h);
    return herr(e, "hybrid cache allocation");
  }
  *out = h;
  return moe::report(MOE_OK, "");
}

int moe_w4a16_hybrid_destroy(moe_w4a16_hybrid* h) {
  release(h);
  return moe::report(MOE_OK, "");
}

int moe_w4a16_hybrid_forward(moe_w4a16_hybrid* h, const void* x, const int32_t* expert_ids,
                             const void* route_w, const void* const* resident_w,
                             const void* const* resident_s, const void* const* host_src, void* out,
                             const moe_w4a16_cfg* cfg) {
  if (!h || !cfg || !resident_w || !resident_s || !host_src)
    return moe::report(MOE_ERR_INVALID_ARG, "handle, cfg and the three host tables are required");
  const int T = cfg->num_tokens, K = cfg->top_k, E = cfg->num_experts;
  if (T < 0 || K < 1 || E < 1) return moe::report(MOE_ERR_INVALID_ARG, "bad num_tokens/top_k/num_experts");
  if (T == 0) return moe::report(MOE_OK, "");
  if (E > h->max_experts || (int64_t)T * K > h->max_pairs)
    return moe::report(MOE_ERR_INVALID_ARG, "call larger than the handle's max_experts / max_pairs");
  if (cfg->scale_fmt != MOE_SCALE_E8M0_G32 && cfg->scale_fmt != MOE_SCALE_E4M3_G16)
    return moe::report(MOE_ERR_INVALID_ARG, "scale_fmt unknown");
  if ((int64_t)cfg->inter * cfg->hidden * 3 / 2 != h->nib)
    return moe::report(MOE_ERR_INVALID_ARG, "nibble bytes do not match hidden / inter");
  {
    // the scales follow the nibbles in a triplet: one byte per 32 (E8M0) or
    // 16 (E4M3) values of the three matrices
    const int64_t grp = cfg->scale_fmt == MOE_SCALE_E4M3_G16 ? 16 : 32;
    if (h->triplet < h->nib + (int64_t)3 * cfg->inter * cfg->hidden / grp)
      return moe::report(MOE_ERR_INVALID_ARG,
                         "triplet_bytes too small for the nibbles and scales of this scale_fmt");
  }
  for (int e = 0; e < E; ++e)
    if (!resident_w[e] != !resident_s[e] || (!resident_w[e] && !host_src[e]))
      return moe::report(MOE_ERR_INVALID_ARG,
                         "every expert needs both resident tables or a checkpoint address");
  hipStream_t s = (hipStream_t)cfg->stream;
  // 1. the selected ids, on the CPU (this synchronises the stream, so every
  // earlier H2D copy out of the pinned cache and every kernel that read the
  // staging buffer has finished)
  hipError_t e = hipMemcpyAsync(h->ids_host, expert_ids, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return herr(e, "id copy");
  // 2. the routed CPU-backed experts, in order of first appearance
  std::vector<int> slot_of(E, -1);
  h->last_experts.clear();
  h->last_hits.clear();
  for (int p = 0; p < T * K; ++p) {
    const int ex = h->ids_host[p];
    if (ex < 0 || ex >= E) return moe::report(MOE_ERR_INVALID_ARG, "expert id out of range");
    if (resident_w[ex] || slot_of[ex] >= 0) continue;
    const int st = (int)h->last_experts.size();
    if (st >= h->staging_slots)
      return moe::report(MOE_ERR_INVALID_ARG, "more routed CPU experts than staging slots");
    slot_of[ex] = st;
    h->last_experts.push_back(ex);
  }
  // 3. the cache decides hits and slots in request order; the hits' H2D
  // copies start at once, then the misses' slots are filled from the
  // checkpoint (on several host threads, while the hits' copies run) and
  // copied too.  No entry used in this call can be evicted by it (the cache
  // holds at least staging_slots triplets), and the id copy above waited for
  // every earlier copy out of the cache.
  const size_t nreq = h->last_experts.size();
  std::vector<int> cslot(nreq);
  std::vector<uint8_t*> fill_dst;
  std::vector<const uint8_t*> fill_src;
  for (size_t r = 0; r < nreq; ++r) {
    const int ex = h->last_experts[r];
    bool hit = false;
    cslot[r] = cache_slot(h, host_src[ex], &hit);
    h->last_hits.push_back(hit ? 1 : 0);
    (hit ? h->hits : h->misses)++;
    if (!hit) {
      fill_dst.push_back(h->pinned + (size_t)cslot[r] * h->triplet);
      fill_src.push_back((const uint8_t*)host_src[ex]);
    }
  }
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) parallel_copy(fill_dst, fill_src, (size_t)h->triplet);
    for (size_t r = 0; r < nreq; ++r) {
      if (h->last_hits[r] != (pass == 0 ? 1 : 0)) continue;
      e = hipMemcpyAsync(h->staging + r * h->triplet, h->pinned + (size_t)cslot[r] * h->triplet,
                         (size_t)h->triplet, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return herr(e, "expert H2D copy");
      h->h2d_bytes += h->triplet;
    }
  }
  // 4. the layer's pointer tables: resident experts in place, routed CPU
  // experts in their staging slots, other CPU experts (never read) at slot 0
  for (int ex = 0; ex < E; ++ex) {
    const uint8_t* b = h->staging + (size_t)(slot_of[ex] >= 0 ? slot_of[ex] : 0) * h->triplet;
    h->tab_host[ex] = resident_w[ex] ? (void*)resident_w[ex] : (void*)b;
    h->tab_host[E + ex] = resident_s[ex] ? (void*)resident_s[ex] : (void*)(b + h->nib);
  }
  e = hipMemcpyAsync(h->tab_dev, h->tab_host, 2 * sizeof(void*) * E, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return herr(e, "table copy");
  h->calls++;
  // 5. the grouped layer
  return moe_w4a16_forward(x, expert_ids, route_w, (const void* const*)h->tab_dev,
                           (const void* const*)(h->tab_dev + E), out, cfg);
}

int moe_w4a16_hybrid_stats(const moe_w4a16_hybrid* h, int64_t* stats4) {
  if (!h || !stats4) return moe::report(MOE_ERR_INVALID_ARG, "handle and stats are required");
  stats4[0] = h->calls;
  stats4[1] = h->hits;
  stats4[2] = h->misses;
  stats4[3] = h->h2d_bytes;
  return moe::report(MOE_OK, "");
}

int moe_w4a16_hybrid_last_requests(const moe_w4a16_hybrid* h, int32_t* experts, uint8_t* hits,
                                   int32_t capacity, int32_t* count) {
  if (!h || !count) return moe::report(MOE_ERR_INVALID_ARG, "handle and count are required");
  const int n = (int)h->last_experts.size();
  *count = n;
  if (n > capacity || (n > 0 && (!experts || !hits)))
    return moe::report(MOE_ERR_INVALID_ARG, "output arrays too small");
  for (int i = 0; i < n; ++i) {
    experts[i] = h->last_experts[i];
    hits[i] = h->last_hits[i];
  }
  return moe::report(MOE_OK, "");
}

}  // extern "C"
