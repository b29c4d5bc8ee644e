// Idle-group offload: whole groups in pinned host memory, device slots,
// group-granular swap-in and prefetch (C ABI in include/moe.h).
#include <algorithm>
#include <memory>
#include <vector>

#include "api_internal.h"

using namespace cefn;
using namespace cefn_api;

// ------------------------------------------------------ group offload ----
// Whole groups' weights live in pinned host memory; `slots` device slots
// hold the groups in use.  One entry per weight array: the handle's pointer
// field is repointed at the slot cache, so the GEMMs address group g's
// weights at slot gslot[g] with the array's usual per-group stride.
struct OffloadArray {
  void** field;     // handle member that the kernels read
  char* host;       // pinned: every group, group-major
  char* cache;      // device: slots x group_bytes
  size_t group_bytes;
};

struct OffloadState {
  int slots = 0;
  std::vector<OffloadArray> arrays;
  std::vector<int> slot_of;        // [G] slot holding the group, or -1
  std::vector<int> group_in;       // [slots] group in the slot, or -1
  std::vector<long> last_use;      // [slots] use stamp (least recently used is evicted)
  std::vector<double> heat;        // [G] moving average of the group's share of rows
  long stamp = 0;
  hipStream_t copy = nullptr;      // host-to-device copies (default priority)
  std::vector<hipEvent_t> slot_free;   // compute stream: last pass that read the slot is done
  std::vector<hipEvent_t> slot_ready;  // copy stream: the slot's copies are done
  int* pass_dev = nullptr;         // device [G][2][G]: per pass gslot then gcounts
  int* pass_host = nullptr;        // pinned staging of the same
  int* gcounts_host = nullptr;     // pinned [G]
  moe_offload_stats_t st{};
};

namespace cefn_api {

void delete_offload(moe_handle* h) {
  OffloadState* o = h->off;
  if (!o) return;
  if (o->copy) (void)hipStreamSynchronize(o->copy);
  for (auto& a : o->arrays) (void)hipHostFree(a.host);
  if (o->pass_host) (void)hipHostFree(o->pass_host);
  if (o->gcounts_host) (void)hipHostFree(o->gcounts_host);
  for (hipEvent_t e : o->slot_free) (void)hipEventDestroy(e);
  for (hipEvent_t e : o->slot_ready) (void)hipEventDestroy(e);
  if (o->copy) (void)hipStreamDestroy(o->copy);
  delete o;
  h->off = nullptr;
}

}  // namespace cefn_api

// ---- idle-group offload ----------------------------------------------------
namespace {

int enqueue_group_copy(moe_handle* h, int g, int slot) {
  OffloadState* o = h->off;
  if (hipStreamWaitEvent(o->copy, o->slot_free[slot], 0) != hipSuccess) return fail(MOE_ERR_HIP, "copy wait");
  for (const auto& a : o->arrays)
    if (hipMemcpyAsync(a.cache + (size_t)slot * a.group_bytes, a.host + (size_t)g * a.group_bytes, a.group_bytes,
                       hipMemcpyHostToDevice, o->copy) != hipSuccess)
      return fail(MOE_ERR_HIP, "group copy");
  if (hipEventRecord(o->slot_ready[slot], o->copy) != hipSuccess) return fail(MOE_ERR_HIP, "copy event");
  if (o->group_in[slot] >= 0) o->slot_of[o->group_in[slot]] = -1;
  o->group_in[slot] = g;
  o->slot_of[g] = slot;
  for (const auto& a : o->arrays) o->st.bytes_h2d += (int64_t)a.group_bytes;
  return MOE_OK;
}

// Slot to load a group into: an empty one, else the least recently used
// whose group is not in `keep`.
int pick_slot(const OffloadState* o, const std::vector<char>& keep) {
  int best = -1;
  for (int s = 0; s < o->slots; ++s) {
    const int g = o->group_in[s];
    if (g < 0) return s;
    if (keep[g]) continue;
    if (best < 0 || o->last_use[s] < o->last_use[best]) best = s;
  }
  return best;
}

}  // namespace

extern "C" {

int moe_offload_enable(moe_handle* h, int32_t slots) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  const moe_config& c = h->cfg;
  if (h->off) return fail(MOE_ERR_INVALID_ARG, "offload already enabled");
  if (slots < 1 || slots > c.G) return fail(MOE_ERR_INVALID_ARG, "slots=%d outside [1, G=%d]", slots, c.G);
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_ERR_HIP, "synchronise");
  delete_bwd(h);  // the backward layouts are not kept for an offloaded handle
  std::unique_ptr<OffloadState> o(new OffloadState());
  o->slots = slots;
  const size_t es = elem_bytes(h->mma);
  const bool int4 = c.resid == MOE_RESID_INT4_G32;
  const size_t K = c.K, Pin = h->P_in, f = c.f, d = c.d;
  auto add = [&](void** field, size_t gb) {
    if (*field && gb) o->arrays.push_back(OffloadArray{field, nullptr, nullptr, gb});
  };
  add(&h->W1, h->w1_gs * es);
  add(&h->W2, h->w2_gs * es);
  if (c.r > 0) {
    add(&h->At, int4 ? h->at_gs * 4 : h->at_gs * es);
    if (int4) add(reinterpret_cast<void**>(&h->At_s), h->at_sgs * 2);
    add(&h->B1, K * (int4 ? Pin * f * 8 : Pin * f * 16 * es));
    if (int4) add(reinterpret_cast<void**>(&h->B1_s), K * Pin * (f / 32) * RPAD * 2);
    add(&h->Ad, K * (f / 32) * 2 * 64 * (int4 ? 4 : 8 * es));
    if (int4) add(reinterpret_cast<void**>(&h->Ad_s), K * (f / 32) * RPAD * 2);
    add(&h->Bd, int4 ? h->bd_gs * 4 : h->bd_gs * es);
    if (int4) add(reinterpret_cast<void**>(&h->Bd_s), K * (d / 32) * RPAD * 2);
  }
  h->off = o.get();  // so delete_offload can clean up a partial set-up
  o.release();
  OffloadState* off = h->off;
  auto undo = [&](int code, const char* what) {
    delete_offload(h);
    return fail(code, "%s", what);
  };
  for (auto& a : off->arrays) {
    const size_t total = a.group_bytes * c.G;
    void* host = nullptr;
    if (hipHostMalloc(&host, total, hipHostMallocDefault) != hipSuccess) return undo(MOE_ERR_OOM, "pinned host memory");
    a.host = static_cast<char*>(host);
    if (hipMemcpy(a.host, *a.field, total, hipMemcpyDeviceToHost) != hipSuccess) return undo(MOE_ERR_HIP, "copy out");
  }
  // device slot caches replace the full arrays
  for (auto& a : off->arrays) {
    char* cache = nullptr;
    if (dalloc(h, &cache, a.group_bytes * slots)) return undo(MOE_ERR_OOM, "slot cache");
    void* old = *a.field;
    auto it = std::find(h->allocs.begin(), h->allocs.end(), old);
    if (it != h->allocs.end()) {
      h->allocs.erase(it);
      (void)hipFree(old);
    }
    a.cache = cache;
    *a.field = cache;
  }
  const int G = c.G;
  off->slot_of.assign(G, -1);
  off->group_in.assign(slots, -1);
  off->last_use.assign(slots, 0);
  off->heat.assign(G, 0.0);
  if (dalloc(h, &off->pass_dev, (size_t)G * 2 * G)) return undo(MOE_ERR_OOM, "pass tables");
  void* ph = nullptr;
  if (hipHostMalloc(&ph, sizeof(int) * (size_t)G * 2 * G, hipHostMallocDefault) != hipSuccess)
    return undo(MOE_ERR_OOM, "pinned staging");
  off->pass_host = static_cast<int*>(ph);
  if (hipHostMalloc(&ph, sizeof(int) * (size_t)G, hipHostMallocDefault) != hipSuccess)
    return undo(MOE_ERR_OOM, "pinned counts");
  off->gcounts_host = static_cast<int*>(ph);
  if (hipStreamCreateWithFlags(&off->copy, hipStreamNonBlocking) != hipSuccess) return undo(MOE_ERR_HIP, "copy stream");
  off->slot_free.assign(slots, nullptr);
  off->slot_ready.assign(slots, nullptr);
  for (int s2 = 0; s2 < slots; ++s2)
    if (hipEventCreateWithFlags(&off->slot_free[s2], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&off->slot_ready[s2], hipEventDisableTiming) != hipSuccess)
      return undo(MOE_ERR_HIP, "events");
  // warm start: the first groups, in order
  for (int g = 0; g < slots; ++g)
    if (enqueue_group_copy(h, g, g)) return undo(MOE_ERR_HIP, "initial copies");
  off->st.bytes_h2d = 0;
  if (hipStreamSynchronize(off->copy) != hipSuccess) return undo(MOE_ERR_HIP, "initial copies");
  return MOE_OK;
}

int moe_offload_stats(const moe_handle* h, moe_offload_stats_t* out) {
  if (!h || !out) return fail(MOE_ERR_INVALID_ARG, "null handle or stats");
  if (!h->off) return fail(MOE_ERR_INVALID_ARG, "offload not enabled");
  *out = h->off->st;
  return MOE_OK;
}

int moe_forward_offload(moe_handle* h, const void* X, int32_t T, void* Y, const moe_route_out* routing,
                        void* stream) {
  if (!h) return fail(MOE_ERR_INVALID_ARG, "null handle");
  OffloadState* o = h->off;
  if (!o) return fail(MOE_ERR_INVALID_ARG, "offload not enabled (moe_offload_enable)");
  const moe_config& c = h->cfg;
  if (T < 0 || T > c.T_max) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, T_max=%d]", T, c.T_max);
  if (T == 0) return routing ? moe_route(h, X, 0, routing, stream) : MOE_OK;
  if (!X || !Y) return fail(MOE_ERR_INVALID_ARG, "null X or Y");
  if (X == Y) return fail(MOE_ERR_INVALID_ARG, "X and Y may not alias");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = c.G;
  ++o->st.calls;
  FwdState fs{};
  TRY(fwd_prelude(h, h->ws, X, T, routing, st, fs));
  // which groups this batch touches
  if (hipMemcpyAsync(o->gcounts_host, fs.live.gcounts, sizeof(int) * G, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(MOE_ERR_HIP, "group counts to host");
  const int* gc = o->gcounts_host;
  std::vector<int> need;
  for (int g = 0; g < G; ++g)
    if (gc[g] > 0 && o->slot_of[g] >= 0) need.push_back(g);  // resident first
  for (int g = 0; g < G; ++g)
    if (gc[g] > 0 && o->slot_of[g] < 0) need.push_back(g);
  const int n = (int)need.size();
  const int per = n <= o->slots ? n : std::max(1, o->slots / 2);
  int pass = 0;
  for (int b = 0; b < n; b += per, ++pass) {
    const int e = std::min(n, b + per);
    std::vector<char> keep(G, 0);
    for (int q = b; q < e; ++q) keep[need[q]] = 1;
    for (int q = b; q < e; ++q) {
      const int g = need[q];
      if (o->slot_of[g] >= 0) {
        ++o->st.group_hits;
        continue;
      }
      const int slot = pick_slot(o, keep);
      if (slot < 0) return fail(MOE_ERR_HIP, "no free slot");
      TRY(enqueue_group_copy(h, g, slot));
      ++o->st.group_loads;
    }
    int* tab = o->pass_host + (size_t)pass * 2 * G;
    for (int g = 0; g < G; ++g) {
      tab[g] = keep[g] ? o->slot_of[g] : 0;
      tab[G + g] = keep[g] ? gc[g] : 0;
    }
    int* dtab = o->pass_dev + (size_t)pass * 2 * G;
    if (hipMemcpyAsync(dtab, tab, sizeof(int) * 2 * G, hipMemcpyHostToDevice, st) != hipSuccess)
      return fail(MOE_ERR_HIP, "pass table copy");
    for (int q = b; q < e; ++q)
      if (hipStreamWaitEvent(st, o->slot_ready[o->slot_of[need[q]]], 0) != hipSuccess)
        return fail(MOE_ERR_HIP, "wait for group copy");
    TRY(fwd_gemms(h, h->ws, X, T, Y, st, fs, dtab + G, dtab));
    for (int q = b; q < e; ++q) {
      const int slot = o->slot_of[need[q]];
      o->last_use[slot] = ++o->stamp;
      if (hipEventRecord(o->slot_free[slot], st) != hipSuccess) return fail(MOE_ERR_HIP, "slot event");
    }
  }
  o->st.passes += pass;
  TRY(fwd_combine(h, h->ws, T, Y, st, fs));
  // prefetch: groups used most in recent batches, into slots of groups used less
  double rows = 0;
  for (int g = 0; g < G; ++g) rows += gc[g];
  for (int g = 0; g < G; ++g) o->heat[g] = 0.5 * o->heat[g] + 0.5 * (rows > 0 ? gc[g] / rows : 0.0);
  std::vector<int> cand;
  for (int g = 0; g < G; ++g)
    if (o->slot_of[g] < 0 && o->heat[g] > 0) cand.push_back(g);
  std::stable_sort(cand.begin(), cand.end(), [&](int a, int b2) { return o->heat[a] > o->heat[b2]; });
  int budget = std::max(1, o->slots / 2);
  for (int g : cand) {
    if (budget-- <= 0) break;
    int victim = -1;
    for (int s2 = 0; s2 < o->slots; ++s2) {
      const int r = o->group_in[s2];
      if (r < 0) {
        victim = s2;
        break;
      }
      if (o->heat[r] < o->heat[g] && (victim < 0 || o->heat[r] < o->heat[o->group_in[victim]])) victim = s2;
    }
    if (victim < 0) break;
    TRY(enqueue_group_copy(h, g, victim));
    ++o->st.prefetched;
  }
  return MOE_OK;
}

}  // extern "C"
