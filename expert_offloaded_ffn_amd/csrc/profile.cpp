// Optional per-kernel timing for measurement tools: hipEvents recorded on the
// launch stream around the library's heavy kernels, summed on read.
#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moeffn {
namespace {

struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  hipEvent_t open[MOE_PROF_KINDS] = {};
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> done;
  moe_profile acc{};
};

Prof& prof() {
  static Prof p;
  return p;
}

thread_local int t_label = 0;   // moe_profile_label of the calling thread

hipEvent_t take(Prof& p) {
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence at the record, whose cache write-back and invalidate
  // would otherwise sit between the timed launch and its events
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_mark(hipStream_t s, int kind, bool end) {
  Prof& p = prof();
  if (!p.on) return;
  kind += t_label * MOE_PROF_LABELED;
  std::lock_guard<std::mutex> lock(p.mu);
  hipEvent_t e = take(p);
  if (!e) return;
  (void)hipEventRecord(e, s);
  if (!end) {
    if (p.open[kind]) p.pool.push_back(p.open[kind]);
    p.open[kind] = e;
  } else if (p.open[kind]) {
    p.done.push_back({kind, {p.open[kind], e}});
    p.open[kind] = nullptr;
  } else {
    p.pool.push_back(e);
  }
}

}  // namespace moeffn

using namespace moeffn;

extern "C" moe_status moe_profile_enable(int32_t on) {
  clear_error();
  Prof& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  for (auto& d : p.done) {
    p.pool.push_back(d.second.first);
    p.pool.push_back(d.second.second);
  }
  p.done.clear();
  p.acc = moe_profile{};
  p.on = on != 0;
  return MOE_OK;
}

extern "C" moe_status moe_profile_label(int32_t label) {
  clear_error();
  MOE_REQUIRE(label == 0 || label == 1, MOE_EINVAL, "moe_profile_label: label %d is not 0 or 1", label);
  t_label = label;
  return MOE_OK;
}

extern "C" moe_status moe_profile_read(moe_profile* out) {
  clear_error();
  MOE_REQUIRE(out != nullptr, MOE_EINVAL, "moe_profile_read: out is NULL");
  Prof& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  for (auto& d : p.done) {
    MOE_HIP(hipEventSynchronize(d.second.second));
    float ms = 0.f;
    MOE_HIP(hipEventElapsedTime(&ms, d.second.first, d.second.second));
    p.acc.ms[d.first] += ms;
    p.acc.launches[d.first] += 1;
    p.pool.push_back(d.second.first);
    p.pool.push_back(d.second.second);
  }
  p.done.clear();
  *out = p.acc;
  return MOE_OK;
}
