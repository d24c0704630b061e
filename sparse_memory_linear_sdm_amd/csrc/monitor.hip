// Slot-update histogram: the collapse monitor of the papers.ananclaw.com summary
// (engineering-risks section, risk 3): per head, how many tokens wrote each slot,
// so that updates piling onto a few slots become visible.
//
// One thread per write id, a global integer atomic per id (the counts of one head,
// N * 4 bytes, do not fit a workgroup's LDS at the workloads' N; integer adds
// commute, so the result is exact and independent of order).
#include "sdm_internal.h"

namespace sdm {
namespace {

__global__ __launch_bounds__(256) void slot_histogram_kernel(const int32_t* __restrict__ idx_w,
                                                             int64_t total, int32_t W, int32_t H,
                                                             int32_t N, int32_t* counts) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += stride) {
    const int32_t id = idx_w[e];
    const int32_t h = (int32_t)((e / W) % H);
    if (id >= 0 && id < N) atomicAdd(counts + (int64_t)h * N + id, 1);
  }
}

}  // namespace

hipError_t launch_slot_histogram(const sdm_dims& d, int64_t N, const int32_t* idx_w,
                                 int32_t* counts, hipStream_t s) {
  const int64_t total = d.B * d.T * d.H * (int64_t)d.W;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192));
  KernelTimer kt("slot_histogram", s);
  hipLaunchKernelGGL(slot_histogram_kernel, grid, dim3(256), 0, s, idx_w, total, d.W, d.H,
                     (int32_t)N, counts);
  return hipGetLastError();
}

}  // namespace sdm
