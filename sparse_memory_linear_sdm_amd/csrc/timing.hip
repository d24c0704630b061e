// Kernel timing for calls made with SDM_FLAG_TIMING: a HIP event pair on the
// call's stream around every launch, kept in a process-wide record until read.
// Recording never changes what the kernels compute; if an event cannot be created
// or recorded the launch simply goes unrecorded.
#include <deque>
#include <mutex>
#include <vector>

#include "sdm_internal.h"

namespace sdm {
namespace {

struct Record {
  const char* name;
  hipEvent_t a, b;
};

constexpr size_t kMaxRecords = 65536;

std::mutex g_mu;
std::deque<Record> g_records;    // oldest first
std::vector<hipEvent_t> g_pool;  // events free for reuse
thread_local bool t_on = false;

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_pool.empty()) {
      hipEvent_t e = g_pool.back();
      g_pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void give_back(hipEvent_t e) {
  if (!e) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pool.push_back(e);
}

}  // namespace

void timing_enable(bool on) { t_on = on; }
bool timing_enabled() { return t_on; }

KernelTimer::KernelTimer(const char* name, hipStream_t s) : name_(name), s_(s) {
  if (!t_on) return;
  a_ = take_event();
  if (a_ && hipEventRecord(a_, s_) != hipSuccess) {
    give_back(a_);
    a_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!a_) return;
  hipEvent_t b = take_event();
  if (!b || hipEventRecord(b, s_) != hipSuccess) {
    give_back(a_);
    give_back(b);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back({name_, a_, b});
  while (g_records.size() > kMaxRecords) {
    g_pool.push_back(g_records.front().a);
    g_pool.push_back(g_records.front().b);
    g_records.pop_front();
  }
}

}  // namespace sdm

extern "C" SDM_API int32_t sdm_timing_read(sdm_kernel_time* out, int32_t max) {
  if (max <= 0) return 0;
  if (!out) return SDM_ERR_NULL;
  std::vector<sdm::Record> got;
  {
    std::lock_guard<std::mutex> lk(sdm::g_mu);
    while (!sdm::g_records.empty() && (int32_t)got.size() < max) {
      got.push_back(sdm::g_records.front());
      sdm::g_records.pop_front();
    }
  }
  int32_t status = 0;
  for (size_t i = 0; i < got.size(); ++i) {
    float ms = 0.0f;
    if (hipEventSynchronize(got[i].b) != hipSuccess ||
        hipEventElapsedTime(&ms, got[i].a, got[i].b) != hipSuccess)
      status = SDM_ERR_HIP;
    out[i].name = got[i].name;
    out[i].ms = ms;
    sdm::give_back(got[i].a);
    sdm::give_back(got[i].b);
  }
  return status != 0 ? status : (int32_t)got.size();
}
