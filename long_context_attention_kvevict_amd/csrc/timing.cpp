// Event-based stage timing (see timing.h).  Process-wide, not thread-safe:
// meant for a benchmark driving one stream.
#include "timing.h"

#include <vector>

#include "../../include/kvevict.h"

namespace kve {

namespace {

struct Rec {
  int stage;
  hipEvent_t begin, end;
};

struct Timing {
  uint32_t mask = 0;   // stages being timed
  std::vector<hipEvent_t> pool;   // reusable events
  size_t next = 0;
  std::vector<Rec> recs;
  hipEvent_t open[ST_COUNT] = {};
};

Timing g;
constexpr size_t kPool = 4096;

hipEvent_t take_event() {
  if (g.next >= g.pool.size()) return nullptr;
  return g.pool[g.next++];
}

}  // namespace

void stage_begin(int stage, hipStream_t st) {
  if (!((g.mask >> stage) & 1u)) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, st) == hipSuccess) g.open[stage] = e;
  else g.open[stage] = nullptr;
}

void stage_end(int stage, hipStream_t st) {
  if (!((g.mask >> stage) & 1u)) return;
  hipEvent_t b = g.open[stage];
  hipEvent_t e = take_event();
  if (!b || !e) return;
  if (hipEventRecord(e, st) == hipSuccess) g.recs.push_back({stage, b, e});
  g.open[stage] = nullptr;
}

}  // namespace kve

extern "C" {

int32_t kvevict_timing_enable(int32_t stage_mask) {
  using namespace kve;
  if (stage_mask && g.pool.empty()) {
    g.pool.reserve(kPool);
    for (size_t i = 0; i < kPool; ++i) {
      // Timing only: no system-scope fence (cache write-back and invalidate)
      // when an event is recorded, which would slow the kernel after it.
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return KVE_EHIP;
      g.pool.push_back(e);
    }
  }
  g.mask = static_cast<uint32_t>(stage_mask) & ((1u << ST_COUNT) - 1u);
  g.next = 0;
  g.recs.clear();
  return KVE_OK;
}

int32_t kvevict_timing_summary(double* avg_ms, int32_t* counts, int32_t n_stages) {
  using namespace kve;
  if (!avg_ms || !counts) return KVE_EINVAL;
  for (int i = 0; i < n_stages; ++i) { avg_ms[i] = 0.0; counts[i] = 0; }
  for (const Rec& r : g.recs) {
    if (hipEventSynchronize(r.end) != hipSuccess) return KVE_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess) return KVE_EHIP;
    if (r.stage < n_stages) { avg_ms[r.stage] += ms; counts[r.stage] += 1; }
  }
  for (int i = 0; i < n_stages; ++i)
    if (counts[i]) avg_ms[i] /= counts[i];
  g.next = 0;
  g.recs.clear();
  return KVE_OK;
}

}  // extern "C"
