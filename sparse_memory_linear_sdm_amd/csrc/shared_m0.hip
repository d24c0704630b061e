// Shared learned initial state with copy on first touch.
//
// The learned initial state M0 is one parameter of the layer, the same for every
// sequence (ai-paper-analysis.pages.dev, section on the learned M0; m.163.com
// article on arXiv 2607.07386, section 三).  Instead of every sequence carrying a
// full copy of it, a sequence's store holds only the rows it has touched, and a
// bitmap of N bits per (b, h) says which: the effective row of slot i is
// store[i] if its bit is set, else M0[h][i].
//
// Before the scan, this pass visits every id the call will read or write.  Each
// visit sets the slot's bit with an atomic OR; the visit that finds the bit clear
// (exactly one per slot, however many tokens of the call name it) copies the M0
// row into the store.  The scan kernels then run unchanged on the store: every row
// they touch is current.  Rows never touched are never read or written, so a fresh
// sequence needs no initialised store at all.
#include "sdm_internal.h"

namespace sdm {
namespace {

// One wavefront per 64 accesses of the flattened [B*T*H][W + R] id lists.
__global__ __launch_bounds__(256) void materialize_kernel(const int32_t* __restrict__ idx_w,
                                                          const int32_t* __restrict__ idx_r,
                                                          int64_t total, int32_t T, int32_t H,
                                                          int32_t W, int32_t R, int32_t N,
                                                          uint32_t row_bytes, const char* m0,
                                                          char* store, uint32_t* touched) {
  const int lane = threadIdx.x & 63;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x);
  const int WR = W + R;
  const int64_t words = (N + 31) / 32;
  int32_t walk = 0, id = -1, h = 0;
  bool first = false;
  if (e < total) {
    const int64_t tok = e / WR;  // (b * T + t) * H + h
    const int k = (int)(e - tok * WR);
    id = k < W ? idx_w[tok * W + k] : idx_r[tok * R + (k - W)];
    h = (int32_t)(tok % H);
    walk = (int32_t)((tok / H / T) * H + h);  // b * H + h
    if (id >= 0 && id < N) {
      const uint32_t bit = 1u << (id & 31);
      const uint32_t old = atomicOr(touched + walk * words + (id >> 5), bit);
      first = (old & bit) == 0;
    }
  }
  // the wavefront copies each newly touched row together, 16 bytes per lane
  uint64_t todo = __ballot(first);
  const uint32_t chunks = row_bytes / 16;
  while (todo) {
    const int src = __ffsll((long long)todo) - 1;
    todo &= todo - 1;
    const int32_t sw = __shfl(walk, src);
    const int32_t si = __shfl(id, src);
    const int32_t sh = __shfl(h, src);
    const uint4* from = reinterpret_cast<const uint4*>(m0 + ((int64_t)sh * N + si) * row_bytes);
    uint4* to = reinterpret_cast<uint4*>(store + ((int64_t)sw * N + si) * row_bytes);
    for (uint32_t c = lane; c < chunks; c += 64) to[c] = from[c];
  }
}

}  // namespace

hipError_t launch_materialize(const sdm_dims& d, int64_t N, const int32_t* idx_w,
                              const int32_t* idx_r, const void* m0, void* store,
                              uint32_t* touched, hipStream_t s) {
  const int64_t total = d.B * d.T * d.H * (int64_t)(d.W + d.R);
  if (total == 0) return hipSuccess;
  const uint32_t row_bytes =
      (uint32_t)d.d_v * ((d.flags & SDM_FLAG_STATE_BF16) ? 2u : 4u);  // 32 .. 1024, 16 | it
  const dim3 grid((unsigned)((total + 255) / 256));
  KernelTimer kt("materialize_m0", s);
  hipLaunchKernelGGL(materialize_kernel, grid, dim3(256), 0, s, idx_w, idx_r, total, (int32_t)d.T,
                     d.H, d.W, d.R, (int32_t)N, row_bytes, static_cast<const char*>(m0),
                     static_cast<char*>(store), touched);
  return hipGetLastError();
}

}  // namespace sdm
