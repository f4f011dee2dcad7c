// expert_slot_cache_dev: the expert slot pool with its plan made on the device.
//
// The pages intercept the router's expert list on the host before the experts
// run ("Running 35B MoE Models on 8GB GPUs", section "Technical Insight"), a
// synchronisation they also name as a cost, next to the launch overhead that
// graph capture removes ("NovaLLM", section 3). Here the same residency step
// runs without the host: one workgroup reads the expert histogram, checks
// residency and plans the LRU accesses of the step (the rules of the host
// planner: resident experts first, then the others, each in ascending id; the
// lowest free slot, else the least recently used expert), then a copy kernel on
// a side stream pulls the missed bundles from pinned host memory over PCIe
// while the step's hits compute. Nothing waits on the host, so a whole decode
// step (routing, plan, copies, expert FFN, combine) can be one captured graph.
//
// A step that touches more experts than there are slots runs in waves, as on
// the host: the plan writes one miss table per wave, and wave w's copies start
// only after the caller's kernels of wave w-1 (they may reuse its slots).
#include <climits>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"

using namespace moeffn;

namespace {

constexpr int kPlanThreads = 1024;   // one thread per expert and per slot
constexpr int kCopyThreads = 256;
constexpr int kCopyBlocksPerBundle = 16;

enum Ctl { kClock = 0, kSteps, kHits, kMisses, kEvictions, kWaves, kStepHits, kCopies, kMixed, kCtlN };

struct DevState {
  int32_t* slot_of;   // [E]
  int32_t* owner;     // [S]
  int64_t* last;      // [E] recency stamps
  int64_t* ctl;       // [kCtlN]
  int2* copies;       // [E] (expert, slot) of the last step's misses, in miss order (up to E of them)
  double* freq;       // [E] decayed routed rows (used when decay > 0)
  double* decay;      // [1] frequency decay, read by every plan (graphs see changes); 0 = LRU
  int64_t* layers;    // [1] layer order: entries are this many layer-major groups (1 = none)
};

// Rank of this thread's flag among the block's set flags (ascending thread
// index) and, in *total, how many are set. Every thread of the block calls it.
__device__ int block_rank(bool flag, int* wave_cnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wave_cnt[wave] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const int c = wave_cnt[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// Smallest 64-bit key over the block (every thread calls it; t >= S passes LLONG_MAX).
__device__ long long block_min(long long v, long long* wave_min) {
  for (int off = 32; off > 0; off >>= 1) {
    const long long o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) wave_min[threadIdx.x >> 6] = v;
  __syncthreads();
  long long m = wave_min[0];
  for (int w = 1; w < kPlanThreads / 64; ++w) m = wave_min[w] < m ? wave_min[w] : m;
  __syncthreads();
  return m;
}

// Plans one step as the sequential LRU does: accesses in the order resident
// touched experts (ascending id), then the others (ascending id), in waves of
// at most S. A hit restamps its expert; a miss takes the lowest free slot, else
// the slot whose expert has the oldest stamp (an expert used earlier in this
// step can go in a later wave; one of the current wave cannot, it is newer).
// Resident experts are all hits and all fall in wave 0 (there are at most S).
// Outputs: hit_table[E] (wave 0's hits), miss_tables[w][E] for w < max_waves,
// the copy list in miss order, and per-step counts in ctl.
__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(const int32_t* __restrict__ counts, DevState st,
                                                                  int E, int S, int max_waves,
                                                                  int32_t* __restrict__ hit_table,
                                                                  int32_t* __restrict__ miss_tables) {
  __shared__ int wave_cnt[kPlanThreads / 64];
  __shared__ long long wave_min[kPlanThreads / 64];
  __shared__ int miss_list[kPlanThreads];     // missed experts, ascending
  __shared__ int slot_owner[kPlanThreads];
  __shared__ long long slot_stamp[kPlanThreads];
  __shared__ double slot_freq[kPlanThreads];
  const int t = threadIdx.x;
  const double decay = *st.decay;
  const int L = (int)*st.layers, per = E / L;
  bool touched = false, resident = false;
  int my_slot = -1;
  if (t < E && decay > 0.0) {
    // separately rounded multiply and add: the same doubles as the host planner's
    st.freq[t] = __dadd_rn(__dmul_rn(decay, st.freq[t]), (double)max(counts[t], 0));
  }
  if (t < E) {
    touched = counts[t] > 0;
    my_slot = st.slot_of[t];
    if (my_slot >= S) my_slot = -1;  // slots are < S in a consistent table; never index with another
    resident = my_slot >= 0;
  }
  int n_hit = 0, n_miss = 0;
  const int hit_rank = block_rank(touched && resident, wave_cnt, &n_hit);
  const int miss_rank = block_rank(touched && !resident, wave_cnt, &n_miss);
  const long long clock = st.ctl[kClock];
  int layer = 0;  // the step's layer (layer order only): that of its lowest touched entry
  if (L > 1) {
    const long long lo = block_min(touched ? (long long)t : LLONG_MAX, wave_min);
    const long long hi = -block_min(touched ? -(long long)t : LLONG_MAX, wave_min);
    if (lo != LLONG_MAX) {
      layer = (int)(lo / per);
      if (hi / per != layer && t == 0) st.ctl[kMixed] += 1;  // reported by stats
    }
  }
  if (t < S) {
    int o = st.owner[t];
    if (o >= E) o = -1;
    slot_owner[t] = o;
    slot_stamp[t] = o >= 0 ? (long long)st.last[o] : 0;
    slot_freq[t] = o >= 0 && decay > 0.0 ? st.freq[o] : 0.0;
  }
  if (touched && !resident) miss_list[miss_rank] = t;
  __syncthreads();
  if (touched && resident) slot_stamp[my_slot] = clock + 1 + hit_rank;  // the hits, in access order
  __syncthreads();
  // misses one at a time: the lowest free slot; else, outside the current wave, the smallest
  // routing frequency (when decay > 0; frequencies are >= 0, so their bit patterns order like
  // the values), then the oldest stamp
  for (int j = 0; j < n_miss; ++j) {
    const long long wave_start = clock + 1 + (long long)((n_hit + j) / S) * S;
    const bool occupied = t < S && slot_owner[t] >= 0;
    const bool cand = occupied && slot_stamp[t] < wave_start;
    long long key = t < S && !occupied ? (long long)t : LLONG_MAX;
    long long m = block_min(key, wave_min);
    if (m == LLONG_MAX) {  // block-uniform: no free slot
      bool keep_d = cand;
      if (L > 1) {  // the layer whose next step is furthest away: (layer - current - 1) mod L largest
        const int dist = cand ? ((slot_owner[t] / per - layer - 1) % L + L) % L : 0;
        const long long dkey = cand ? (long long)(L - 1 - dist) : LLONG_MAX;
        const long long md = block_min(dkey, wave_min);
        keep_d = cand && dkey == md;
      }
      const long long fbits = keep_d ? (long long)__double_as_longlong(slot_freq[t]) : LLONG_MAX;
      const long long mf = decay > 0.0 ? block_min(fbits, wave_min) : 0;
      const bool keep = keep_d && (decay > 0.0 ? fbits == mf : true);
      key = keep ? slot_stamp[t] : LLONG_MAX;
      m = block_min(key, wave_min);
      if (!keep) key = LLONG_MIN;  // never equal to m
    }
    if (t < S && key == m) {  // slot indices and stamps are distinct: one thread matches
      const int e = miss_list[j];
      const int wave = (n_hit + j) / S;
      if (wave < max_waves) miss_tables[(size_t)wave * E + e] = t;
      st.copies[j] = make_int2(e, t);
      if (slot_owner[t] >= 0) atomicAdd(reinterpret_cast<unsigned long long*>(st.ctl + kEvictions), 1ull);
      slot_owner[t] = e;
      slot_stamp[t] = clock + 1 + n_hit + j;
      slot_freq[t] = decay > 0.0 ? st.freq[e] : 0.0;
    }
    __syncthreads();
  }
  // tables: -1 for every expert a table does not name
  if (t < E) {
    hit_table[t] = touched && resident ? my_slot : -1;
    for (int w = 0; w < max_waves; ++w) {
      const bool mine = touched && !resident && (n_hit + miss_rank) / S == w;
      if (!mine) miss_tables[(size_t)w * E + t] = -1;
    }
    if (my_slot >= 0 && slot_owner[my_slot] != t) st.slot_of[t] = -1;  // evicted this step
  }
  __syncthreads();
  if (t < S) {
    const int o = slot_owner[t];
    st.owner[t] = o;
    if (o >= 0) {
      st.slot_of[o] = t;
      st.last[o] = slot_stamp[t];
    }
  }
  if (t == 0) {
    st.ctl[kClock] = clock + n_hit + n_miss;
    st.ctl[kSteps] += 1;
    st.ctl[kHits] += n_hit;
    st.ctl[kMisses] += n_miss;
    st.ctl[kWaves] += (n_hit + n_miss + S - 1) / S;
    st.ctl[kStepHits] = n_hit;
    st.ctl[kCopies] = n_miss;
  }
}

// Copies wave `wave`'s missed bundles host -> slot: misses j with access
// position n_hit + j in [wave*S, (wave+1)*S). blockIdx.y = copy within the wave
// (blocks past the wave's copies exit at once); the x blocks of one bundle
// stride over its 16-byte words, four loads in flight per thread.
__global__ __launch_bounds__(kCopyThreads) void cache_copy_kernel(const int64_t* __restrict__ ctl,
                                                                 const int2* __restrict__ copies,
                                                                 const uint4* const* __restrict__ src,
                                                                 uint8_t* __restrict__ pool, int64_t stride,
                                                                 int64_t n16, int n_experts, int n_slots, int wave) {
  const int n_hit = (int)ctl[kStepHits], n_miss = (int)ctl[kCopies];
  const int j0 = max(0, wave * n_slots - n_hit), j1 = min(n_miss, (wave + 1) * n_slots - n_hit);
  const int c = j0 + (int)blockIdx.y;
  if (c >= j1) return;
  const int2 cp = copies[c];
  if (cp.x < 0 || cp.x >= n_experts || cp.y < 0 || cp.y >= n_slots) return;
  const uint4* __restrict__ from = src[cp.x];
  uint4* __restrict__ to = reinterpret_cast<uint4*>(pool + (int64_t)cp.y * stride);
  const int64_t step = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n16; i += 4 * step) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * step < n16) v[u] = from[i + u * step];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * step < n16) to[i + u * step] = v[u];
  }
}

}  // namespace

struct expert_slot_cache_dev {
  moe_cache_cfg cfg{};
  int device = -1;
  hipStream_t side = nullptr;
  int max_waves = 1;
  double decay = 0.0;
  int n_layers = 1;
  std::vector<hipEvent_t> fork, join;  // per wave
  void* block = nullptr;  // device: state, copy list and source pointers
  DevState st{};
  const uint4** src = nullptr;
  bool stepped = false;
};

namespace {

size_t state_bytes(int E, int S) {
  return align_up(sizeof(int32_t) * E, 256) + align_up(sizeof(int32_t) * S, 256) +
         align_up(sizeof(int64_t) * E, 256) + align_up(sizeof(int64_t) * kCtlN, 256) +
         align_up(sizeof(int2) * E, 256) + align_up(sizeof(void*) * E, 256) + align_up(sizeof(double) * E, 256) +
         256;
}

// Empty pool, zero counters (synchronous; not for use under capture).
moe_status init_state(expert_slot_cache_dev* c) {
  const int E = c->cfg.n_experts, S = c->cfg.n_slots;
  std::vector<int32_t> neg(std::max(E, S), -1);
  std::vector<int64_t> zero(std::max(E, (int)kCtlN), 0);
  MOE_HIP(hipMemcpy(c->st.slot_of, neg.data(), sizeof(int32_t) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(c->st.owner, neg.data(), sizeof(int32_t) * S, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(c->st.last, zero.data(), sizeof(int64_t) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(c->st.ctl, zero.data(), sizeof(int64_t) * kCtlN, hipMemcpyHostToDevice));
  std::vector<double> fzero(E, 0.0);
  MOE_HIP(hipMemcpy(c->st.freq, fzero.data(), sizeof(double) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(c->st.decay, &c->decay, sizeof(double), hipMemcpyHostToDevice));
  const int64_t layers = c->n_layers;
  MOE_HIP(hipMemcpy(c->st.layers, &layers, sizeof(int64_t), hipMemcpyHostToDevice));
  c->stepped = false;
  return MOE_OK;
}

void destroy_dev(expert_slot_cache_dev* c) {
  if (c->side) (void)hipStreamSynchronize(c->side);
  for (auto& ev : c->fork) if (ev) (void)hipEventDestroy(ev);
  for (auto& ev : c->join) if (ev) (void)hipEventDestroy(ev);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->block) (void)hipFree(c->block);
}

}  // namespace

extern "C" moe_status expert_slot_cache_dev_create(const moe_cache_cfg* cfg, expert_slot_cache_dev** out) {
  clear_error();
  MOE_REQUIRE(cfg && out, MOE_EINVAL, "expert_slot_cache_dev_create: NULL argument");
  *out = nullptr;
  const moe_cache_cfg k = *cfg;
  MOE_REQUIRE(!k.blocking && !k.dry_run, MOE_EINVAL,
              "expert_slot_cache_dev_create: blocking and dry_run are host-planner modes");
  MOE_REQUIRE(k.n_experts >= 1 && k.n_experts <= kPlanThreads, MOE_EINVAL,
              "expert_slot_cache_dev_create: n_experts=%d outside [1, %d]", k.n_experts, kPlanThreads);
  MOE_REQUIRE(k.n_slots >= 1 && k.n_slots <= kPlanThreads, MOE_ECAPACITY,
              "expert_slot_cache_dev_create: n_slots=%d outside [1, %d]", k.n_slots, kPlanThreads);
  MOE_REQUIRE(k.bundle_bytes > 0 && k.bundle_bytes % 16 == 0, MOE_EINVAL,
              "expert_slot_cache_dev_create: bundle_bytes %lld must be a positive multiple of 16",
              (long long)k.bundle_bytes);
  MOE_REQUIRE(k.slot_stride >= k.bundle_bytes && k.slot_stride % 256 == 0, MOE_ECAPACITY,
              "expert_slot_cache_dev_create: slot_stride %lld must be >= bundle_bytes %lld and a multiple of 256",
              (long long)k.slot_stride, (long long)k.bundle_bytes);
  MOE_REQUIRE(k.bundles_host && k.pool, MOE_EINVAL, "expert_slot_cache_dev_create: bundles_host and pool are required");
  MOE_REQUIRE(aligned(k.pool, 256), MOE_EINVAL, "expert_slot_cache_dev_create: pool must be 256-byte aligned");
  std::vector<const void*> src(k.n_experts);
  for (int e = 0; e < k.n_experts; ++e) {
    const void* h = k.bundles_host[e];
    MOE_REQUIRE(h != nullptr && aligned(h, 16), MOE_EINVAL,
                "expert_slot_cache_dev_create: bundle %d is NULL or not 16-byte aligned", e);
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t err = hipPointerGetAttributes(&attr, h);
    if (err != hipSuccess) (void)hipGetLastError();
    MOE_REQUIRE(err == hipSuccess && attr.type == hipMemoryTypeHost, MOE_EINVAL,
                "expert_slot_cache_dev_create: bundle %d is not in pinned host memory", e);
    void* dptr = nullptr;
    err = hipHostGetDevicePointer(&dptr, const_cast<void*>(h), 0);
    if (err != hipSuccess) (void)hipGetLastError();
    MOE_REQUIRE(err == hipSuccess && dptr != nullptr, MOE_EINVAL,
                "expert_slot_cache_dev_create: bundle %d has no device mapping", e);
    src[e] = dptr;
  }
  auto* c = new (std::nothrow) expert_slot_cache_dev();
  MOE_REQUIRE(c != nullptr, MOE_ENOMEM, "expert_slot_cache_dev_create: out of host memory");
  c->cfg = k;
  auto fail = [&](const char* what, hipError_t e) {
    set_error("expert_slot_cache_dev_create: %s: %s", what, hipGetErrorString(e));
    destroy_dev(c);
    delete c;
    return MOE_EHIP;
  };
  hipError_t e;
  const int E = k.n_experts, S = k.n_slots;
  if ((e = hipGetDevice(&c->device)) != hipSuccess) return fail("hipGetDevice", e);
  if ((e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess) return fail("hipStreamCreate", e);
  c->max_waves = (E + S - 1) / S;
  c->fork.assign(c->max_waves, nullptr);
  c->join.assign(c->max_waves, nullptr);
  for (int w = 0; w < c->max_waves; ++w) {
    if ((e = hipEventCreateWithFlags(&c->fork[w], hipEventDisableTiming)) != hipSuccess) return fail("hipEventCreate", e);
    if ((e = hipEventCreateWithFlags(&c->join[w], hipEventDisableTiming)) != hipSuccess) return fail("hipEventCreate", e);
  }
  if ((e = hipMalloc(&c->block, state_bytes(E, S))) != hipSuccess) return fail("hipMalloc", e);
  char* p = static_cast<char*>(c->block);
  c->st.slot_of = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t) * E, 256);
  c->st.owner = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t) * S, 256);
  c->st.last = reinterpret_cast<int64_t*>(p);
  p += align_up(sizeof(int64_t) * E, 256);
  c->st.ctl = reinterpret_cast<int64_t*>(p);
  p += align_up(sizeof(int64_t) * kCtlN, 256);
  c->st.copies = reinterpret_cast<int2*>(p);
  p += align_up(sizeof(int2) * E, 256);
  c->src = reinterpret_cast<const uint4**>(p);
  p += align_up(sizeof(void*) * E, 256);
  c->st.freq = reinterpret_cast<double*>(p);
  p += align_up(sizeof(double) * E, 256);
  c->st.decay = reinterpret_cast<double*>(p);
  c->st.layers = reinterpret_cast<int64_t*>(p + 8);
  if ((e = hipMemcpy(c->src, src.data(), sizeof(void*) * E, hipMemcpyHostToDevice)) != hipSuccess)
    return fail("hipMemcpy", e);
  if (moe_status s = init_state(c)) {
    destroy_dev(c);
    delete c;
    return s;
  }
  *out = c;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_destroy(expert_slot_cache_dev* c) {
  clear_error();
  if (!c) return MOE_OK;
  destroy_dev(c);
  delete c;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_reset(expert_slot_cache_dev* c) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_dev_reset: NULL cache");
  MOE_HIP(hipDeviceSynchronize());
  return init_state(c);
}

extern "C" moe_status expert_slot_cache_dev_set_frequency(expert_slot_cache_dev* c, double decay) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_dev_set_frequency: NULL cache");
  MOE_REQUIRE(decay >= 0.0 && decay <= 1.0, MOE_EINVAL,
              "expert_slot_cache_dev_set_frequency: decay %g outside [0, 1]", decay);
  MOE_HIP(hipDeviceSynchronize());
  std::vector<double> fzero(c->cfg.n_experts, 0.0);
  MOE_HIP(hipMemcpy(c->st.freq, fzero.data(), sizeof(double) * c->cfg.n_experts, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(c->st.decay, &decay, sizeof(double), hipMemcpyHostToDevice));
  c->decay = decay;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_set_layers(expert_slot_cache_dev* c, int32_t n_layers) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_dev_set_layers: NULL cache");
  MOE_REQUIRE(n_layers >= 1 && c->cfg.n_experts % n_layers == 0, MOE_EINVAL,
              "expert_slot_cache_dev_set_layers: n_layers=%d must divide n_experts=%d", n_layers, c->cfg.n_experts);
  MOE_HIP(hipDeviceSynchronize());
  const int64_t layers = n_layers;
  MOE_HIP(hipMemcpy(c->st.layers, &layers, sizeof(int64_t), hipMemcpyHostToDevice));
  c->n_layers = n_layers;
  return MOE_OK;
}

extern "C" int32_t expert_slot_cache_dev_max_waves(const expert_slot_cache_dev* c) {
  return c ? c->max_waves : 0;
}

extern "C" moe_status expert_slot_cache_dev_step(expert_slot_cache_dev* c, const int32_t* counts, void* stream,
                                                 int32_t* hit_table, int32_t* miss_tables) {
  clear_error();
  MOE_REQUIRE(c && counts && hit_table && miss_tables, MOE_EINVAL, "expert_slot_cache_dev_step: NULL argument");
  MOE_REQUIRE(aligned(counts, 4) && aligned(hit_table, 4) && aligned(miss_tables, 4), MOE_EINVAL,
              "expert_slot_cache_dev_step: misaligned table");
  if (moe_status s = check_launch("expert_slot_cache_dev_step (earlier work)")) return s;
  hipLaunchKernelGGL(cache_plan_kernel, dim3(1), dim3(kPlanThreads), 0, as_stream(stream), counts, c->st,
                     c->cfg.n_experts, c->cfg.n_slots, c->max_waves, hit_table, miss_tables);
  if (moe_status r = check_launch("cache_plan_kernel")) return r;
  c->stepped = true;
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_copy(expert_slot_cache_dev* c, int32_t wave, void* stream) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_dev_copy: NULL cache");
  MOE_REQUIRE(c->stepped, MOE_ESTATE, "expert_slot_cache_dev_copy: no step was planned");
  MOE_REQUIRE(wave >= 0 && wave < c->max_waves, MOE_EINVAL, "expert_slot_cache_dev_copy: wave %d outside [0, %d)",
              wave, c->max_waves);
  const int E = c->cfg.n_experts, S = c->cfg.n_slots;
  MOE_HIP(hipEventRecord(c->fork[wave], as_stream(stream)));
  MOE_HIP(hipStreamWaitEvent(c->side, c->fork[wave], 0));
  hipLaunchKernelGGL(cache_copy_kernel, dim3(kCopyBlocksPerBundle, S), dim3(kCopyThreads), 0, c->side,
                     c->st.ctl, c->st.copies, c->src, static_cast<uint8_t*>(c->cfg.pool), (int64_t)c->cfg.slot_stride,
                     (int64_t)(c->cfg.bundle_bytes / 16), E, S, (int)wave);
  if (moe_status r = check_launch("cache_copy_kernel")) return r;
  MOE_HIP(hipEventRecord(c->join[wave], c->side));
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_join(expert_slot_cache_dev* c, int32_t wave, void* stream) {
  clear_error();
  MOE_REQUIRE(c, MOE_EINVAL, "expert_slot_cache_dev_join: NULL cache");
  MOE_REQUIRE(c->stepped, MOE_ESTATE, "expert_slot_cache_dev_join: no step was planned");
  MOE_REQUIRE(wave >= 0 && wave < c->max_waves, MOE_EINVAL, "expert_slot_cache_dev_join: wave %d outside [0, %d)",
              wave, c->max_waves);
  MOE_HIP(hipStreamWaitEvent(as_stream(stream), c->join[wave], 0));
  return MOE_OK;
}

extern "C" moe_status expert_slot_cache_dev_stats(expert_slot_cache_dev* c, moe_cache_stats* out) {
  clear_error();
  MOE_REQUIRE(c && out, MOE_EINVAL, "expert_slot_cache_dev_stats: NULL argument");
  MOE_HIP(hipDeviceSynchronize());
  int64_t ctl[kCtlN];
  MOE_HIP(hipMemcpy(ctl, c->st.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  *out = moe_cache_stats{};
  out->steps = ctl[kSteps];
  out->hits = ctl[kHits];
  out->misses = ctl[kMisses];
  out->evictions = ctl[kEvictions];
  out->waves = ctl[kWaves];
  out->h2d_bytes = ctl[kMisses] * c->cfg.bundle_bytes;
  MOE_REQUIRE(ctl[kMixed] == 0, MOE_ESTATE,
              "expert_slot_cache_dev_stats: %lld steps touched entries of several layers under the layer order",
              (long long)ctl[kMixed]);
  return MOE_OK;
}
