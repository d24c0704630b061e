// Internal declarations shared by the HIP translation units of libsdm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm.h"

namespace sdm {

// Where the projection epilogue writes (see proj_gemm.hip).  Row m is the global
// token index b*T + t; the scores buffer may hold only rows [scores_row0, ...).
struct ProjDst {
  float* scores;          // [rows, H, 4n] fp32, indexed by (m - scores_row0)
  int64_t scores_row0;
  float* v;               // [M, H, d_v]
  float* gate;            // [M, H, d_v]  activated
  float* alpha;           // [M, H]
  float* beta;            // [M, H]
  const float* A;         // [H]
  const float* b_dt;      // [H]
  int H, n, d_v, P, gate_act;
};

// Projection Y = x[row0 : row0+rows] W_proj^T with the gate epilogue.
hipError_t launch_proj_gemm(const sdm_dims& d, const void* x, const void* w_proj, int64_t row0,
                            int64_t rows, const ProjDst& dst, hipStream_t s);

// Top-W / top-R selection for `rows` token rows whose half-scores start at
// `scores` ([rows, H, 4n]); results go to global rows out_row0 + r.
hipError_t launch_select(const sdm_dims& d, const float* scores, int64_t rows, int64_t out_row0,
                         int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                         hipStream_t s);

// Recurrent scan over all (b, h) walks.
struct ScanArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* gate;
  const float* alpha;
  const float* beta;
  const float* norm_w;  // nullable
  float* state;
  float* out;
  float* y_raw;         // nullable
  int64_t B, T;
  int32_t H, N, W, R, d_v;
  float eps;
};
hipError_t launch_scan(const sdm_dims& d, const ScanArgs& a, void* ws, size_t ws_bytes,
                       hipStream_t s);
size_t scan_workspace_bytes(const sdm_dims& d);

// Slot-owner stream schedule of the scan (scan_stream.hip).
// Instrumentation (SDM_FLAG_TIMING): the C entry points switch recording on for
// the calling thread; every launch site holds a KernelTimer around its launch.
void timing_enable(bool on);
bool timing_enabled();
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

struct StreamArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* gate;
  const float* alpha;
  const float* beta;
  const float* norm_w;
  float* state;
  float* out;
  float* y_raw;
  int* counts;     // [walks][rounds][GT]
  int* offsets;    // [walks][GT][rounds + 1]
  // owner-stream entry: {slot | token-in-round << 24, weight bits | read << 31}
  uint2* entries;  // [walks][walk_entries]
  float* y_part;   // [parts][B][Tc][H][d_v]
  float4* trash;   // one float4 per scan thread: sink of non-writing accesses' stores
  int* begins;    // two-phase: [walks][GT][rounds] start of each packed segment
  uint2* clean;   // two-phase: [B][Tc][H][R] clean reads {slot, weight bits}, grouped by part
  int* cstart;    // two-phase: [B][Tc][H][parts + 1] start of each part's clean reads
  int64_t B, T, t0, Tc, walk_entries;
  int32_t H, N, W, R, d_v;
  float eps;
  int32_t S, parts, GT, log2GT, log2GW, rounds;
};
struct StreamPlan {
  int SW, S, NT, parts, GT, log2GT, rounds;
  bool two_phase;  // clean reads summed in registers after each round's writes
  int64_t Tc;
};
StreamPlan plan_stream(const sdm_dims& d, int64_t N);
size_t stream_workspace_bytes(const sdm_dims& d, const StreamPlan& pl);
hipError_t launch_stream_scan(const ScanArgs& a, const StreamPlan& pl, void* ws, hipStream_t s);
bool scan_uses_stream(const sdm_dims& d);

}  // namespace sdm
