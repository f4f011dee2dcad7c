// expert_slot_cache: expert-granular residency over a fixed HBM slot pool.
//
// The pages' design, restated: every expert's weights live in pinned host
// memory ("NovaLLM: Running Massive MoE Models Fully In-Memory", section 3,
// Optimization #2); only experts the router selected are brought into VRAM,
// loaded right before they run, with the loads overlapping compute (same page,
// Optimization #1); the cache intercepts the router's expert list, checks
// residency and evicts least-recently-used bundles; a step that needs more
// experts than there are slots runs in waves, each wave's copies finishing
// before its experts compute ("Running 35B MoE
// Models on 8GB GPUs", section "Technical Insight"); transfers are asynchronous
// host-to-HBM copies issued only for non-resident experts ("The Billion-Token
// Bottleneck", section "Predictive Prefetching").
//
// Prefetch: a background reader fetches the next layer ahead of its compute
// ("NovaLLM", section 3, Optimization #1); predicted experts that are not
// resident are copied asynchronously before the model reaches their layer,
// highest expected demand first ("The Billion-Token Bottleneck", sections
// "Predictive Prefetching" and "The Orchestration Layer").
//
// Two halves:
//  planner   pure host code: per step, the touched set (from the expert
//            histogram), the access order (resident ascending, then
//            non-resident ascending), waves of <= n_slots, LRU with the lowest
//            free slot first; prefetch inserts predicted experts between steps
//            without evicting an expert of the step last planned. Runs without
//            a device (dry_run) for tests.
//  executor  a side stream for host->HBM bundle copies; per-slot "last read"
//            events recorded on the compute stream (a copy into a slot waits for
//            the last kernel that read it); per-wave "copies done" events that
//            the compute stream waits on before the wave's miss experts run;
//            per-slot "filled" events of prefetch copies, which the compute
//            stream waits on before a wave's hits run when one of them is still
//            in flight.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"

using namespace moeffn;

struct expert_slot_cache {
  moe_cache_cfg cfg{};
  std::vector<const void*> bundles;
  // planner
  std::vector<int32_t> slot_of, owner;
  std::vector<int64_t> last;
  int64_t clock = 0;
  int64_t step_clock = 0;                // clock before the last planned step's first access
  int32_t n_layers = 1;                  // > 1: entries are layer-major groups run in cyclic order
  int32_t step_layer = 0;                // layer of the last planned step's entries
  int64_t wave_clock = 0;                // clock before the current wave's first access
  double freq_decay = 0.0;               // > 0: victims by decayed routing frequency before recency
  std::vector<double> freq;              // per entry: sum over planned steps of decay^age * counts
  std::vector<char> prefetched;          // per expert: brought in by prefetch, not yet used by a step
  std::vector<std::vector<moe_cache_entry>> waves;
  bool planned = false;
  moe_cache_stats st{};
  // executor
  int device = -1;
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> last_read;     // per slot
  std::vector<char> last_read_valid;
  std::vector<hipEvent_t> copy_begin, copy_done;  // per wave
  std::vector<hipEvent_t> wait_begin, wait_end;   // per wave: the compute stream around its wait for the copies
  std::vector<char> wave_copied;         // copies issued for the wave this step
  std::vector<char> timing_pending;      // copy span events to be added to copy_ms
  std::vector<char> wait_pending;        // wait span events to be added to wait_ms
  int64_t copies_issued = 0;             // bundle copies attempted since create
  int64_t fail_copy_at = 0;              // > 0: copy number fail_copy_at fails (MOEFFN_FAIL_COPY_AT, tests)
  std::vector<hipEvent_t> fill_done;     // per slot: end of its last prefetch copy
  std::vector<char> fill_pending;        // per slot: the compute stream has not waited for it
  hipEvent_t compute_mark = nullptr;     // blocking mode: all compute enqueued before a wave
  int32_t* counts_pinned = nullptr;
  int32_t* tables_pinned = nullptr;      // [max_waves][2][E]
  int max_waves = 0;
};

namespace {

void plan_reset(expert_slot_cache* c) {
  const int E = c->cfg.n_experts, S = c->cfg.n_slots;
  c->slot_of.assign(E, -1);
  c->owner.assign(S, -1);
  c->last.assign(E, 0);
  c->prefetched.assign(E, 0);
  c->freq.assign(E, 0.0);
  c->clock = 0;
  c->step_clock = 0;
  c->step_layer = 0;
  c->wave_clock = 0;
  c->waves.clear();
  c->planned = false;
  c->st = moe_cache_stats{};
}

// Victim order: with a layer order, the entry whose layer runs furthest after
// the current one first (distance (layer - current - 1) mod L, largest first);
// then, with a frequency decay, the smallest decayed routing frequency; then
// the least recently used. Plain LRU when neither is set. `ok` filters
// candidates.
template <class Ok>
int pick_victim(const expert_slot_cache* c, Ok ok) {
  const int L = c->n_layers, per = c->cfg.n_experts / L;
  int victim = -1, vdist = -1;
  for (int s = 0; s < c->cfg.n_slots; ++s) {
    const int v = c->owner[s];
    if (v < 0 || !ok(v)) continue;
    const int dist = L > 1 ? ((v / per - c->step_layer - 1) % L + L) % L : 0;
    bool better = victim < 0 || dist > vdist;
    if (!better && dist == vdist) {
      const double fv = c->freq_decay > 0 ? c->freq[v] : 0.0, fw = c->freq_decay > 0 ? c->freq[victim] : 0.0;
      better = fv < fw || (fv == fw && c->last[v] < c->last[victim]);
    }
    if (better) {
      victim = v;
      vdist = dist;
    }
  }
  return victim;
}

moe_cache_entry access(expert_slot_cache* c, int e) {
  moe_cache_entry r{e, -1, 0, -1};
  c->clock += 1;
  if (c->slot_of[e] >= 0) {
    c->last[e] = c->clock;
    c->st.hits += 1;
    if (c->prefetched[e]) {
      c->st.prefetch_used += 1;
      c->prefetched[e] = 0;
    }
    r.slot = c->slot_of[e];
    r.hit = 1;
    return r;
  }
  c->st.misses += 1;
  int slot = -1;
  for (int s = 0; s < c->cfg.n_slots; ++s)
    if (c->owner[s] < 0) { slot = s; break; }
  if (slot < 0) {
    // never an entry of the wave being formed (plain LRU cannot pick one: they are the newest)
    const int victim = pick_victim(c, [&](int v) { return c->last[v] <= c->wave_clock; });
    slot = c->slot_of[victim];
    c->slot_of[victim] = -1;
    c->prefetched[victim] = 0;
    c->st.evictions += 1;
    r.evicted = victim;
  }
  c->owner[slot] = e;
  c->slot_of[e] = slot;
  c->last[e] = c->clock;
  r.slot = slot;
  return r;
}

// One predicted expert. Resident: its recency is refreshed (no copy; slot < 0
// in the result). Otherwise it takes the lowest free slot, else the slot of the
// least recently used expert last used before the last planned step began:
// experts of that step may still be read by its kernels, and experts named by
// a prefetch since then are the prediction itself. With no such victim nothing
// changes and r.expert is -1.
moe_cache_entry prefetch_one(expert_slot_cache* c, int e) {
  moe_cache_entry r{e, -1, 0, -1};
  if (c->slot_of[e] >= 0) {
    c->clock += 1;
    c->last[e] = c->clock;
    return r;
  }
  int slot = -1;
  for (int s = 0; s < c->cfg.n_slots; ++s)
    if (c->owner[s] < 0) { slot = s; break; }
  if (slot < 0) {
    const int victim = pick_victim(c, [&](int v) { return c->last[v] <= c->step_clock; });
    if (victim < 0) {
      r.expert = -1;
      return r;
    }
    slot = c->slot_of[victim];
    c->slot_of[victim] = -1;
    c->prefetched[victim] = 0;
    c->st.evictions += 1;
    r.evicted = victim;
  }
  c->clock += 1;
  c->owner[slot] = e;
  c->slot_of[e] = slot;
  c->last[e] = c->clock;
  c->prefetched[e] = 1;
  c->st.prefetches += 1;
  r.slot = slot;
  return r;
}

moe_status plan_step(expert_slot_cache* c, const int32_t* counts) {
  const int E = c->cfg.n_experts, S = c->cfg.n_slots;
  if (c->n_layers > 1) {
    const int per = E / c->n_layers;
    int layer = -1;
    for (int e = 0; e < E; ++e) {
      if (counts[e] <= 0) continue;
      MOE_REQUIRE(layer < 0 || e / per == layer, MOE_EINVAL,
                  "expert_slot_cache: a step touches entries of layers %d and %d", layer, e / per);
      layer = e / per;
    }
    if (layer >= 0) c->step_layer = layer;
  }
  if (c->freq_decay > 0)
    for (int e = 0; e < E; ++e) c->freq[e] = c->freq_decay * c->freq[e] + (double)std::max(counts[e], 0);
  c->step_clock = c->clock;
  std::vector<int> order;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0 && c->slot_of[e] >= 0) order.push_back(e);
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0 && c->slot_of[e] < 0) order.push_back(e);
  c->waves.clear();
  for (size_t w0 = 0; w0 < order.size(); w0 += S) {
    c->wave_clock = c->clock;
    std::vector<moe_cache_entry> wave;
    for (size_t i = w0; i < std::min(order.size(), w0 + S); ++i) wave.push_back(access(c, order[i]));
    c->waves.push_back(std::move(wave));
  }
  c->st.waves += (int64_t)c->waves.size();
  c->st.steps += 1;
  c->planned = true;
  return MOE_OK;
}

// Adds finished copy spans and compute-stream wait spans to the stats (events of earlier
// steps; a span whose events have not completed yet stays pending unless `wait`).
void collect_timing(expert_slot_cache* c, bool wait) {
  for (int w = 0; w < c->max_waves; ++w) {
    float ms = 0.f;
    if (c->timing_pending[w]) {
      if (wait) (void)hipEventSynchronize(c->copy_done[w]);
      if (hipEventElapsedTime(&ms, c->copy_begin[w], c->copy_done[w]) == hipSuccess) {
        c->st.copy_ms += ms;
        c->timing_pending[w] = 0;
      }
    }
    if (c->wait_pending[w]) {
      if (wait) (void)hipEventSynchronize(c->wait_end[w]);
      if (hipEventElapsedTime(&ms, c->wait_begin[w], c->wait_end[w]) == hipSuccess) {
        c->st.wait_ms += ms;
        c->wait_pending[w] = 0;
      }
    }
  }
  (void)hipGetLastError();   // a not-ready query is not an error of a later call
}

// A bundle copy failed: the slot it was meant for holds no valid bundle, and neither do the
// slots of the step's misses whose copies were not issued yet (this wave's entries from
// `from` on, and every miss of the later waves). They all leave the planner's residency, so
// a later step misses on them again; the step itself ends here (planned = false).
void drop_unfilled(expert_slot_cache* c, int w, size_t from) {
  for (int v = w; v < (int)c->waves.size(); ++v) {
    const auto& wave = c->waves[v];
    for (size_t i = (v == w ? from : 0); i < wave.size(); ++i) {
      const moe_cache_entry& en = wave[i];
      if (en.hit || c->slot_of[en.expert] != en.slot) continue;
      c->slot_of[en.expert] = -1;
      c->owner[en.slot] = -1;
      c->prefetched[en.expert] = 0;
    }
  }
  c->planned = false;
}

// hipMemcpyAsync of one bundle, or the injected failure of the tests (MOEFFN_FAIL_COPY_AT).
hipError_t copy_bundle(expert_slot_cache* c, void* dst, const void* src) {
  c->copies_issued += 1;
  if (c->fail_copy_at > 0 && c->copies_issued == c->fail_copy_at) return hipErrorInvalidValue;
  return hipMemcpyAsync(dst, src, (size_t)c->cfg.bundle_bytes, hipMemcpyHostToDevice, c->side);
}

void destroy_device(expert_slot_cache* c) {
  if (c->cfg.dry_run) return;
  for (auto& e : c->last_read) if (e) (void)hipEventDestroy(e);
  for (auto& e : c->copy_begin) if (e) (void)hipEventDestroy(e);
  for (auto& e : c->copy_done) if (e) (void)hipEventDestroy(e);
  for (auto& e : c->wait_begin) if (e) (void)hipEventDestroy(e);
  for (auto& e : c->wait_end) if (e) (void)hipEventDestroy(e);
  for (auto& e : c->fill_done) if (e) (void)hipEventDestroy(e);
  if (c->compute_mark) (void)hipEventDestroy(c->compute_mark);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->counts_pinned) (void)hipHostFree(c->counts_pinned);
  if (c->tables_pinned) (void)hipHostFree(c->tables_pinned);
}

}  // namespace

extern "C" moe_status expert_slot_cache_create(const moe_cache_cfg* cfg, expert_slot_cache** out) {
  clear_error();
  MOE_REQUIRE(cfg && out, MOE_EINVAL, "expert_slot_cache_create: NULL argument");
  *out = nullptr;
  const moe_cache_cfg k = *cfg;
  MOE_REQUIRE(k.n_experts >= 1 && k.n_experts <= 1024, MOE_EINVAL, "expert_slot_cache_create: n_experts=%d outside [1, 1024]", k.n_experts);
  MOE_REQUIRE(k.n_slots >= 1, MOE_ECAPACITY, "expert_slot_cache_create: n_slots=%d < 1 (the pool must hold one expert)", k.n_slots);
  MOE_REQUIRE(k.bundle_bytes > 0, MOE_EINVAL, "expert_slot_cache_create: bundle_bytes must be > 0");
  MOE_REQUIRE(k.slot_stride >= k.bundle_bytes && k.slot_stride % 256 == 0, MOE_ECAPACITY,
              "expert_slot_cache_create: slot_stride %lld must be >= bundle_bytes %lld and a multiple of 256",
              (long long)k.slot_stride, (long long)k.bundle_bytes);
  if (!k.dry_run) {
    MOE_REQUIRE(k.bundles_host && k.pool, MOE_EINVAL, "expert_slot_cache_create: bundles_host and pool are required");
    MOE_REQUIRE(aligned(k.pool, 256), MOE_EINVAL, "expert_slot_cache_create: pool must be 256-byte aligned");
    for (int e = 0; e < k.n_experts; ++e) {
      MOE_REQUIRE(k.bundles_host[e] != nullptr, MOE_EINVAL, "expert_slot_cache_create: bundle %d is NULL", e);
      hipPointerAttribute_t attr;
      std::memset(&attr, 0, sizeof(attr));
      const hipError_t err = hipPointerGetAttributes(&attr, k.bundles_host[e]);
      if (err != hipSuccess) (void)hipGetLastError();
      MOE_REQUIRE(err == hipSuccess && attr.type == hipMemoryTypeHost, MOE_EINVAL,
                  "expert_slot_cache_create: bundle %d is not in pinned host memory", e);
    }
  }
  expert_slot_cache* c = new (std::nothrow) expert_slot_cache();
  MOE_REQUIRE(c != nullptr, MOE_ENOMEM, "expert_slot_cache_create: out of host memory");
  c->cfg = k;
  if (!k.dry_run) c->bundles.assign(k.bundles_host, k.bundles_host + k.n_experts);
  plan_reset(c);
  c->max_waves = (k.n_experts + k.n_slots - 1) / k.n_slots;
  if (!k.dry_run) {
    auto fail = [&](const char* what, hipError_t e) {
      set_error("expert_slot_cache_create: %s: %s", what, hipGetErrorString(e));
      destroy_device(c);
      delete c;
      return MOE_EHIP;
    };
    hipError_t e;
    if ((e = hipGetDevice(&c->device)) != hipSuccess) return fail("hipGetDevice", e);
    if ((e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess) return fail("hipStreamCreate", e);
    c->last_read.assign(k.n_slots, nullptr);
    c->last_read_valid.assign(k.n_slots, 0);
    for (auto& ev : c->last_read)
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return fail("hipEventCreate", e);
    c->fill_done.assign(k.n_slots, nullptr);
    c->fill_pending.assign(k.n_slots, 0);
    for (auto& ev : c->fill_done)
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return fail("hipEventCreate", e);
    if ((e = hipEventCreateWithFlags(&c->compute_mark, hipEventDisableTiming)) != hipSuccess)
      return fail("hipEventCreate", e);
    c->copy_begin.assign(c->max_waves, nullptr);
    c->copy_done.assign(c->max_waves, nullptr);
    c->wait_begin.assign(c->max_waves, nullptr);
    c->wait_end.assign(c->max_waves, nullptr);
    c->wave_copied.assign(c->max_waves, 0);
    c->timing_pending.assign(c->max_waves, 0);
    c->wait_pending.assign(c->max_waves, 0);
    for (int w = 0; w < c->max_waves; ++w) {
      if ((e = hipEventCreate(&c->copy_begin[w])) != hipSuccess) return fail("hipEventCreate", e);
      if ((e = hipEventCreate(&c->copy_done[w])) != hipSuccess) return fail("hipEventCreate", e);
      if ((e = hipEventCreate(&c->wait_begin[w])) != hipSuccess) return fail("hipEventCreate", e);
      if ((e = hipEventCreate(&c->wait_end[w])) != hipSuccess) return fail("hipEventCreate", e);
    }
    if (const char* f = std::getenv("MOEFFN_FAIL_COPY_AT")) c->fail_copy_at = std::atoll(f);
    if ((e = hipHostMalloc((void**)&c->counts_pinned, sizeof(int32_t) * k.n_experts, hipHostMallocDefault)) != hipSuccess)
      return fail("hipHostMalloc", e);
    if ((e = hipHostMalloc((void**)&c->tables_pinned, sizeof(int32_t) * k.n_experts * 2 * c->max_waves,
                           hipHostMallocDefault)) != hipSuccess)
      return fail("hipHostMalloc", e);
  }
  *out = c;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_destroy(expert_slot_cache* c) {
  clear_error();
  if (!c) return MOE_OK;
  if (!c->cfg.dry_run && c->side) (void)hipStreamSynchronize(c->side);
  destroy_device(c);
  delete c;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_reset(expert_slot_cache* c) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_reset: NULL cache");
  if (!c->cfg.dry_run) {
    MOE_HIP(hipStreamSynchronize(c->side));
    std::fill(c->last_read_valid.begin(), c->last_read_valid.end(), 0);
    std::fill(c->timing_pending.begin(), c->timing_pending.end(), 0);
    std::fill(c->wait_pending.begin(), c->wait_pending.end(), 0);
    std::fill(c->fill_pending.begin(), c->fill_pending.end(), 0);
  }
  plan_reset(c);
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_plan_host(expert_slot_cache* c, const int32_t* counts_host, int32_t* n_waves_out) {
  clear_error();
  MOE_REQUIRE(c && counts_host, MOE_EINVAL, "expert_slot_cache_plan_host: NULL argument");
  if (moe_status st = plan_step(c, counts_host)) return st;
  if (n_waves_out) *n_waves_out = (int32_t)c->waves.size();
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_acquire(expert_slot_cache* c, const int32_t* counts, void* stream,
                                                int32_t* n_waves_out) {
  clear_error();
  MOE_REQUIRE(c && counts, MOE_EINVAL, "expert_slot_cache_acquire: NULL argument");
  MOE_REQUIRE(!c->cfg.dry_run, MOE_ESTATE, "expert_slot_cache_acquire: cache was created as a dry run");
  hipStream_t s = as_stream(stream);
  const int E = c->cfg.n_experts;
  MOE_HIP(hipMemcpyAsync(c->counts_pinned, counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s));
  MOE_HIP(hipStreamSynchronize(s));  // the router's expert list reaches the host here
  c->st.d2h_bytes += (int64_t)sizeof(int32_t) * E;
  collect_timing(c, false);
  std::fill(c->wave_copied.begin(), c->wave_copied.end(), 0);
  if (moe_status st = plan_step(c, c->counts_pinned)) return st;
  if (n_waves_out) *n_waves_out = (int32_t)c->waves.size();
  return MOE_OK;
}

namespace {

moe_status issue_copies(expert_slot_cache* c, int w, hipStream_t compute) {
  if (c->wave_copied[w]) return MOE_OK;
  c->wave_copied[w] = 1;
  if (c->cfg.blocking) {
    // block, transfer, then execute: no copy starts before all compute enqueued so far
    MOE_HIP(hipEventRecord(c->compute_mark, compute));
    MOE_HIP(hipStreamWaitEvent(c->side, c->compute_mark, 0));
  }
  bool any = false;
  const auto& wave = c->waves[w];
  for (size_t i = 0; i < wave.size(); ++i) {
    const moe_cache_entry& en = wave[i];
    if (en.hit) continue;
    if (!any) {
      MOE_HIP(hipEventRecord(c->copy_begin[w], c->side));
      any = true;
    }
    if (c->last_read_valid[en.slot]) MOE_HIP(hipStreamWaitEvent(c->side, c->last_read[en.slot], 0));
    c->fill_pending[en.slot] = 0;  // the wave's copy_done covers the slot from now on
    char* dst = static_cast<char*>(c->cfg.pool) + (int64_t)en.slot * c->cfg.slot_stride;
    const hipError_t err = copy_bundle(c, dst, c->bundles[en.expert]);
    if (err != hipSuccess) {
      (void)hipGetLastError();
      const int expert = en.expert, slot = en.slot;
      drop_unfilled(c, w, i);
      c->timing_pending[w] = 0;
      set_error("expert_slot_cache: copy of expert %d into slot %d failed: %s", expert, slot,
                hipGetErrorString(err));
      return MOE_EHIP;
    }
    c->st.h2d_bytes += c->cfg.bundle_bytes;
  }
  MOE_HIP(hipEventRecord(c->copy_done[w], c->side));
  if (any) c->timing_pending[w] = 1;
  return MOE_OK;
}

}  // namespace

extern "C" moe_status expert_slot_cache_wave(expert_slot_cache* c, int32_t wave, int32_t part, void* stream,
                                             int32_t* slot_of_expert, int32_t* n_in_part) {
  clear_error();
  MOE_REQUIRE(c && slot_of_expert, MOE_EINVAL, "expert_slot_cache_wave: NULL argument");
  MOE_REQUIRE(!c->cfg.dry_run, MOE_ESTATE, "expert_slot_cache_wave: cache was created as a dry run");
  MOE_REQUIRE(c->planned, MOE_ESTATE, "expert_slot_cache_wave: call expert_slot_cache_acquire first");
  MOE_REQUIRE(wave >= 0 && wave < (int)c->waves.size(), MOE_EINVAL, "expert_slot_cache_wave: wave %d out of range", wave);
  MOE_REQUIRE(part == 0 || part == 1, MOE_EINVAL, "expert_slot_cache_wave: part must be 0 or 1");
  hipStream_t s = as_stream(stream);
  const int E = c->cfg.n_experts;
  if (moe_status st = issue_copies(c, wave, s)) return st;
  int32_t* table = c->tables_pinned + ((size_t)wave * 2 + part) * E;
  std::fill(table, table + E, -1);
  int n = 0;
  const bool blocking = c->cfg.blocking != 0;
  if (blocking ? part == 0 : part == 1) {
    // the compute stream's wait for the wave's copies, timed by events on that stream (the
    // previous step's span is complete: acquire synchronised the stream before planning)
    if (c->wait_pending[wave]) collect_timing(c, true);
    MOE_HIP(hipEventRecord(c->wait_begin[wave], s));
    MOE_HIP(hipStreamWaitEvent(s, c->copy_done[wave], 0));
    MOE_HIP(hipEventRecord(c->wait_end[wave], s));
    c->wait_pending[wave] = 1;
  }
  for (const auto& en : c->waves[wave]) {
    const bool take = blocking ? (part == 0) : (part == 0 ? en.hit != 0 : en.hit == 0);
    if (take) {
      table[en.expert] = en.slot;
      ++n;
      if (en.hit && c->fill_pending[en.slot]) {
        // a prefetched bundle: its copy may still be in flight
        MOE_HIP(hipStreamWaitEvent(s, c->fill_done[en.slot], 0));
        c->fill_pending[en.slot] = 0;
      }
    }
  }
  MOE_HIP(hipMemcpyAsync(slot_of_expert, table, sizeof(int32_t) * E, hipMemcpyHostToDevice, s));
  if (n_in_part) *n_in_part = n;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_release(expert_slot_cache* c, int32_t wave, void* stream) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_release: NULL cache");
  MOE_REQUIRE(!c->cfg.dry_run, MOE_ESTATE, "expert_slot_cache_release: cache was created as a dry run");
  MOE_REQUIRE(c->planned && wave >= 0 && wave < (int)c->waves.size(), MOE_ESTATE,
              "expert_slot_cache_release: wave %d was not planned", wave);
  hipStream_t s = as_stream(stream);
  for (const auto& en : c->waves[wave]) {
    MOE_HIP(hipEventRecord(c->last_read[en.slot], s));
    c->last_read_valid[en.slot] = 1;
  }
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_set_layers(expert_slot_cache* c, int32_t n_layers) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_set_layers: NULL cache");
  MOE_REQUIRE(n_layers >= 1 && c->cfg.n_experts % n_layers == 0, MOE_EINVAL,
              "expert_slot_cache_set_layers: n_layers=%d must divide n_experts=%d", n_layers, c->cfg.n_experts);
  c->n_layers = n_layers;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_set_frequency(expert_slot_cache* c, double decay) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_set_frequency: NULL cache");
  MOE_REQUIRE(decay >= 0.0 && decay <= 1.0, MOE_EINVAL, "expert_slot_cache_set_frequency: decay %g outside [0, 1]",
              decay);
  c->freq_decay = decay;
  std::fill(c->freq.begin(), c->freq.end(), 0.0);
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_prefetch(expert_slot_cache* c, const int32_t* experts_host, int32_t n,
                                                 int32_t* n_copies_out) {
  clear_error();
  MOE_REQUIRE(c && (experts_host || n == 0), MOE_EINVAL, "expert_slot_cache_prefetch: NULL argument");
  MOE_REQUIRE(n >= 0, MOE_EINVAL, "expert_slot_cache_prefetch: n=%d < 0", n);
  MOE_REQUIRE(!c->cfg.blocking, MOE_ESTATE,
              "expert_slot_cache_prefetch: a blocking cache transfers only what a step needs");
  for (int i = 0; i < n; ++i)
    MOE_REQUIRE(experts_host[i] >= 0 && experts_host[i] < c->cfg.n_experts, MOE_EINVAL,
                "expert_slot_cache_prefetch: expert %d outside [0, %d)", experts_host[i], c->cfg.n_experts);
  int copies = 0;
  for (int i = 0; i < n; ++i) {
    const moe_cache_entry en = prefetch_one(c, experts_host[i]);
    if (en.expert < 0) break;  // every slot holds an expert of the last planned step
    if (en.slot < 0) continue;  // already resident
    ++copies;
    if (c->cfg.dry_run) continue;
    if (c->last_read_valid[en.slot]) MOE_HIP(hipStreamWaitEvent(c->side, c->last_read[en.slot], 0));
    char* dst = static_cast<char*>(c->cfg.pool) + (int64_t)en.slot * c->cfg.slot_stride;
    const hipError_t err = copy_bundle(c, dst, c->bundles[en.expert]);
    if (err != hipSuccess) {
      (void)hipGetLastError();
      c->slot_of[en.expert] = -1;
      c->owner[en.slot] = -1;
      c->prefetched[en.expert] = 0;
      set_error("expert_slot_cache_prefetch: copy of expert %d into slot %d failed: %s", en.expert, en.slot,
                hipGetErrorString(err));
      return MOE_EHIP;
    }
    MOE_HIP(hipEventRecord(c->fill_done[en.slot], c->side));
    c->fill_pending[en.slot] = 1;
    c->st.h2d_bytes += c->cfg.bundle_bytes;
  }
  if (n_copies_out) *n_copies_out = copies;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_wave_plan(const expert_slot_cache* c, int32_t wave, moe_cache_entry* entries,
                                                  int32_t capacity, int32_t* n_entries) {
  clear_error();
  MOE_REQUIRE(c && n_entries, MOE_EINVAL, "expert_slot_cache_wave_plan: NULL argument");
  MOE_REQUIRE(c->planned && wave >= 0 && wave < (int)c->waves.size(), MOE_ESTATE,
              "expert_slot_cache_wave_plan: wave %d was not planned", wave);
  const auto& w = c->waves[wave];
  *n_entries = (int32_t)w.size();
  MOE_REQUIRE(entries == nullptr || capacity >= (int32_t)w.size(), MOE_ECAPACITY,
              "expert_slot_cache_wave_plan: capacity %d < %zu", capacity, w.size());
  if (entries) std::copy(w.begin(), w.end(), entries);
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_stats(const expert_slot_cache* c, moe_cache_stats* out) {
  clear_error();
  MOE_REQUIRE(c && out, MOE_EINVAL, "expert_slot_cache_stats: NULL argument");
  if (!c->cfg.dry_run) collect_timing(const_cast<expert_slot_cache*>(c), true);
  *out = c->st;
  return MOE_OK;
}
