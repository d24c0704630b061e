// Shared learned initial state with copy on first touch.
//
// The learned initial state M0 is one parameter of the layer, the same for every
// sequence (ai-paper-analysis.pages.dev, section on the learned M0; m.163.com
// article on arXiv 2607.07386, section 三).  Instead of every sequence carrying a
// full copy of it, a sequence's store holds only the rows it has touched, and a
// bitmap of N bits per (b, h) says which: the effective row of slot i is
// store[i] if its bit is set, else M0[h][i].
//
// Before the scan, this pass visits every id the call will read or write.  A visit
// that finds the slot's bit clear sets it with an atomic OR; the one visit whose OR
// finds it clear (exactly one per slot, however many tokens of the call name it)
// copies the M0 row into the store.  The scan kernels then run unchanged on the
// store: every row they touch is current.  Rows never touched are never read or
// written, so a fresh sequence needs no initialised store at all.
#include "sdm_internal.h"

namespace sdm {
namespace {

// One wavefront per 64 accesses of the flattened [B*T*H][W + R] id lists.
__global__ __launch_bounds__(256) void materialize_kernel(const int32_t* __restrict__ idx_w,
                                                          const int32_t* __restrict__ idx_r,
                                                          int64_t total, int32_t T, int32_t H,
                                                          int32_t W, int32_t R, int32_t N,
                                                          uint32_t row_bytes,
                                                          const char* __restrict__ m0,
                                                          char* __restrict__ store,
                                                          uint32_t* __restrict__ touched) {
  __shared__ int4 rows[4][64];  // per wavefront: (walk, id, head) of each row it claimed
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
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
      uint32_t* word = touched + walk * words + (id >> 5);
      const uint32_t bit = 1u << (id & 31);
      // Within the pass bits only go from clear to set (the caller clears bitmaps in
      // earlier work, which a kernel boundary makes visible).  So a set bit seen by a
      // plain, cached load is final, and only a clear one -- possibly stale -- needs
      // the device-wide atomic that decides which visit copies.  Calls that continue
      // a sequence then cost one cached load per id instead of one atomic.
      if ((*word & bit) == 0) first = (atomicOr(word, bit) & bit) == 0;
    }
  }
  // the wavefront copies all rows it claimed together: rank the claiming lanes,
  // publish (walk, id, head) by rank, then stream 16-byte chunks, 4 per lane in flight
  const uint64_t todo = __ballot(first);
  const uint32_t nrows = (uint32_t)__popcll(todo);
  if (first) rows[wv][__popcll(todo & ((1ull << lane) - 1))] = make_int4(walk, id, h, 0);
  __syncthreads();
  const uint32_t chunks = row_bytes / 16;
  const uint32_t n = nrows * chunks;
  for (uint32_t j0 = 0; j0 < n; j0 += 256) {
    uint4 v[4];
    uint4* dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t j = j0 + u * 64 + lane;
      dst[u] = nullptr;
      v[u] = make_uint4(0, 0, 0, 0);
      if (j < n) {
        const int4 r = rows[wv][j / chunks];
        const uint32_t c = j % chunks;
        v[u] = reinterpret_cast<const uint4*>(m0 + ((int64_t)r.z * N + r.y) * row_bytes)[c];
        dst[u] = reinterpret_cast<uint4*>(store + ((int64_t)r.x * N + r.y) * row_bytes) + c;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u]) *dst[u] = v[u];
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
