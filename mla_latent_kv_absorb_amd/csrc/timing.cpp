// Optional per-kernel HIP event timing for benchmarks (see mla_timing_enable in mla_absorb.h).
// Single-kernel launches get events stamped by the dispatch itself (hipExtLaunchKernel); groups of
// launches are bracketed by events recorded on the stream.
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/mla_absorb.h"
#include "launch.h"

namespace {

struct Record {
  int id;
  hipEvent_t start, stop;
};

struct TimingState {
  uint32_t mask = 0;
  bool failed = false;
  std::vector<Record> records;
  std::vector<hipEvent_t> pool;
  hipEvent_t pending_start = nullptr;
  int pending_id = -1;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      failed = true;
      return nullptr;
    }
    return e;
  }
};

thread_local TimingState g_timing;

}  // namespace

namespace mla {

void timing_begin(int id, hipStream_t stream) {
  TimingState &t = g_timing;
  if (!(t.mask & (1u << id))) return;
  hipEvent_t e = t.take();
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    t.failed = true;
    t.pool.push_back(e);
    return;
  }
  t.pending_start = e;
  t.pending_id = id;
}

void timing_end(int id, hipStream_t stream) {
  TimingState &t = g_timing;
  if (!(t.mask & (1u << id)) || t.pending_id != id || !t.pending_start) return;
  hipEvent_t e = t.take();
  hipEvent_t s = t.pending_start;
  t.pending_start = nullptr;
  t.pending_id = -1;
  if (!e) {
    t.pool.push_back(s);
    return;
  }
  if (hipEventRecord(e, stream) != hipSuccess) {
    t.failed = true;
    t.pool.push_back(s);
    t.pool.push_back(e);
    return;
  }
  t.records.push_back({id, s, e});
}

void timing_events(int id, hipEvent_t *start, hipEvent_t *stop) {
  TimingState &t = g_timing;
  *start = *stop = nullptr;
  if (!(t.mask & (1u << id))) return;
  hipEvent_t a = t.take();
  if (!a) return;
  hipEvent_t b = t.take();
  if (!b) {
    t.pool.push_back(a);
    return;
  }
  *start = a;
  *stop = b;
}

void timing_record(int id, hipEvent_t start, hipEvent_t stop, hipError_t launch_status) {
  TimingState &t = g_timing;
  if (!start || !stop) return;
  if (launch_status != hipSuccess) {
    t.failed = true;
    t.pool.push_back(start);
    t.pool.push_back(stop);
    return;
  }
  t.records.push_back({id, start, stop});
}

}  // namespace mla

extern "C" {

int32_t mla_timing_enable(uint32_t kernel_mask) {
  g_timing.mask = kernel_mask & ((1u << MLA_NUM_KERNELS) - 1);
  return MLA_OK;
}

int32_t mla_timing_collect(int32_t launches[MLA_NUM_KERNELS], double ms[MLA_NUM_KERNELS]) {
  TimingState &t = g_timing;
  for (int i = 0; i < MLA_NUM_KERNELS; ++i) {
    if (launches) launches[i] = 0;
    if (ms) ms[i] = 0.0;
  }
  bool failed = t.failed;
  for (const Record &r : t.records) {
    float dt = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&dt, r.start, r.stop) != hipSuccess) {
      failed = true;
    } else {
      if (launches) launches[r.id] += 1;
      if (ms) ms[r.id] += dt;
    }
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.records.clear();
  t.failed = false;
  return failed ? MLA_ERR_HIP : MLA_OK;
}

const char *mla_kernel_name(int32_t id) {
  switch (id) {
    case MLA_KERNEL_ABSORB_Q: return "absorb_q";
    case MLA_KERNEL_ATTN: return "attn";
    case MLA_KERNEL_COMBINE: return "combine";
    case MLA_KERNEL_EXPAND_PREP: return "expand_prep";
    case MLA_KERNEL_EXPAND: return "expand";
    case MLA_KERNEL_PLAIN: return "plain";
    case MLA_KERNEL_NAIVE: return "naive";
    default: return "";
  }
}

}  // extern "C"
