// Optional per-stage timing of the library's launches with HIP events.
//
// While a profiling window is open (gbla_profile_begin .. gbla_profile_end),
// every selected stage of the forward / backward entry points records one event
// before and one after its kernel(s) on the caller's stream, so the elapsed time between the
// two is that stage's device time on that stream. gbla_profile_end waits for
// the recorded events and returns per-stage totals. The window is process-wide
// state meant for benchmarking. An entry point called while no window is open
// reads one atomic flag and takes no lock, so unprofiled calls share no state;
// a stage whose window was closed or reopened while it ran records nothing.
#include <atomic>
#include <mutex>
#include <vector>

#include "gbla.h"
#include "internal.h"

namespace gbla {

namespace {
const char* kStageNames[kNumStages] = {
    "pack_proj", "conv_fwd", "proj_fwd", "state_partial", "combine_state", "readout",
    "pack_wt", "conv_recompute", "proj_recompute", "bwd_dstate", "combine_dstate", "bwd_token",
    "dbg_reduce", "gemm_dx", "conv_bwd", "gemm_dw", "dw_reduce", "dconv_reduce",
    "lion_log_decay", "lion_proj", "lion_chunk_state", "lion_scan", "lion_readout",
    "lion_bwd_state", "lion_bwd_scan", "lion_bwd_token", "lion_da", "lion_db_reduce", "finalize",
};

struct Profiler {
  std::mutex mu;
  std::atomic<bool> open{false};  // mirrors `active`, read without the lock
  uint64_t generation = 0;        // incremented by every begin and end
  bool active = false;
  uint64_t mask = ~0ull;  // stages that record events
  int capacity = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // 2 per record
  std::vector<int> stage;
};
Profiler& prof() {
  static Profiler p;
  return p;
}
}  // namespace

StageScope::StageScope(int stage_id, hipStream_t s) : rec_(-1), gen_(0), s_(s) {
  Profiler& p = prof();
  if (!p.open.load(std::memory_order_acquire)) return;  // no window: no lock, no shared state
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.active || p.used >= p.capacity || !((p.mask >> stage_id) & 1ull)) return;
  rec_ = p.used++;
  gen_ = p.generation;
  p.stage[rec_] = stage_id;
  (void)hipEventRecord(p.ev[2 * rec_], s_);
}

StageScope::~StageScope() {
  if (rec_ < 0) return;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  // the window this record belongs to may have been closed (events destroyed)
  // or replaced by a new one since the constructor ran
  if (!p.active || p.generation != gen_ || 2 * (size_t)rec_ + 1 >= p.ev.size()) return;
  (void)hipEventRecord(p.ev[2 * rec_ + 1], s_);
}

}  // namespace gbla

using namespace gbla;

extern "C" {

GBLA_API gbla_status gbla_profile_begin(int max_records) { return gbla_profile_begin_stages(max_records, ~0ull); }

GBLA_API gbla_status gbla_profile_begin_stages(int max_records, uint64_t stage_mask) {
  if (max_records < 1 || max_records > (1 << 20)) return GBLA_ERR_BAD_SHAPE;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  ++p.generation;
  p.mask = stage_mask;
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.assign(2 * (size_t)max_records, nullptr);
  p.stage.assign(max_records, -1);
  for (auto& e : p.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      p.active = false;
      p.open.store(false, std::memory_order_release);
      return GBLA_ERR_HIP;
    }
  p.capacity = max_records;
  p.used = 0;
  p.active = true;
  p.open.store(true, std::memory_order_release);
  return GBLA_OK;
}

GBLA_API gbla_status gbla_profile_end(double* ms_per_stage, int* launches_per_stage, int max_stages, int* n_stages) {
  if (!ms_per_stage || !launches_per_stage || !n_stages) return GBLA_ERR_NULL_ARG;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.active) return GBLA_ERR_BAD_SHAPE;
  const int ns = max_stages < kNumStages ? max_stages : kNumStages;
  for (int i = 0; i < ns; ++i) {
    ms_per_stage[i] = 0.0;
    launches_per_stage[i] = 0;
  }
  gbla_status st = GBLA_OK;
  for (int r = 0; r < p.used; ++r) {
    float ms = 0.f;
    if (hipEventSynchronize(p.ev[2 * r + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, p.ev[2 * r], p.ev[2 * r + 1]) != hipSuccess) {
      st = GBLA_ERR_HIP;
      continue;
    }
    const int sid = p.stage[r];
    if (sid >= 0 && sid < ns) {
      ms_per_stage[sid] += ms;
      launches_per_stage[sid] += 1;
    }
  }
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.stage.clear();
  ++p.generation;
  p.active = false;
  p.open.store(false, std::memory_order_release);
  p.capacity = p.used = 0;
  *n_stages = kNumStages;
  return st;
}

GBLA_API const char* gbla_profile_stage_name(int stage) {
  return stage >= 0 && stage < kNumStages ? kStageNames[stage] : "unknown";
}

}  // extern "C"
