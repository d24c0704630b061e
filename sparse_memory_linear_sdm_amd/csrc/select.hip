// Product-key slot selection of the SDM selection pass.
//
// For each (token, head) and each role (write with count W, read with count R):
// the two half-score vectors a, b in R^n define N = n*n slot scores a_i + b_j
// (outer sum; "Sparse Delta Memory" summary on paper.rainbus.top, method
// paragraph, step 1; ai-paper-analysis.pages.dev, section "步骤 1").  The best
// `count` slots are found without scoring all N:
//   1. rank each half by (value desc, index asc) and keep its best k = min(count, n)
//      -- any slot outside top-k(a) x top-k(b) is beaten by `count` slots that are
//      inside it, so the shortcut is exact (ties included);
//   2. of the k*k combinations keep only ranks (r1, r2) with (r1+1)(r2+1) <= count
//      -- every pair (r1' <= r1, r2' <= r2) beats (r1, r2), so the others cannot
//      make the cut (280 candidates instead of 4096 for count = 64);
//   3. score the candidates in fp64 (the sum of two fp32 values is exact there),
//      rank by (score desc, slot id asc), keep `count`;
//   4. return the ids ascending with softmax weights of their scores.
// One wavefront per problem; the ranking steps are bitonic sorts in LDS.
#include "sdm_internal.h"

namespace sdm {
namespace {

// fp32 -> uint32 whose unsigned order is the float order (-0 folded onto +0).
__device__ __forceinline__ uint32_t ord32(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // +-0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t ord64(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  if ((u << 1) == 0) u = 0;
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double unord64(uint64_t k) {
  uint64_t u = (k & 0x8000000000000000ull) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)u);
}

// Bitonic sort of np (power of two) entries so that better() entries come first.
// The block is a single wavefront, so __syncthreads() is a cheap wave barrier.
template <typename Better>
__device__ void bitonic_best_first(uint64_t* key, uint32_t* id, int np, Better better) {
  const int lane = threadIdx.x;
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = lane; p < (np >> 1); p += 64) {
        const int i = ((p / stride) * 2 * stride) + (p & (stride - 1));
        const int j = i + stride;
        const bool first_best = (i & size) == 0;
        const uint64_t ki = key[i], kj = key[j];
        const uint32_t ii = id ? id[i] : 0u, ij = id ? id[j] : 0u;
        const bool swap = first_best ? better(kj, ij, ki, ii) : better(ki, ii, kj, ij);
        if (swap) {
          key[i] = kj;
          key[j] = ki;
          if (id) {
            id[i] = ij;
            id[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

constexpr int KEYS_BYTES = 2 * SDM_MAX_HALF * 8;  // two halves of 64-bit keys (16 KB)

__global__ __launch_bounds__(64) void select_kernel(const float* __restrict__ scores, int64_t rows,
                                                    int H, int n, int W, int R,
                                                    int64_t out_row0, int32_t* __restrict__ idx_w,
                                                    float* __restrict__ wt_w,
                                                    int32_t* __restrict__ idx_r,
                                                    float* __restrict__ wt_r) {
  __shared__ __attribute__((aligned(16))) unsigned char keys_raw[KEYS_BYTES];
  __shared__ float topv[2][SDM_MAX_COUNT];
  __shared__ uint32_t topi[2][SDM_MAX_COUNT];
  __shared__ float red[64];

  const int lane = threadIdx.x;
  const int64_t prob = blockIdx.x;
  const int role = (int)(prob & 1);  // 0 = write, 1 = read
  const int64_t rh = prob >> 1;
  const int64_t r = rh / H;
  const int h = (int)(rh - r * H);
  if (r >= rows) return;
  const int count = role ? R : W;
  const int k = count < n ? count : n;
  const float* half = scores + (r * H + h) * (int64_t)(4 * n) + role * 2 * n;

  // ---- 1. best k of each half, ranked by (value desc, index asc) ----
  uint64_t* hk = reinterpret_cast<uint64_t*>(keys_raw);
  const int np = pow2_at_least(n);
  for (int s = 0; s < 2; ++s) {
    uint64_t* kk = hk + s * SDM_MAX_HALF;
    for (int i = lane; i < np; i += 64) {
      // low word: larger for smaller index, so equal values rank lower index first
      kk[i] = (i < n) ? (((uint64_t)ord32(half[s * n + i]) << 32) | (uint32_t)(0xffffffffu - i))
                      : 0ull;
    }
  }
  __syncthreads();
  auto key_only = [](uint64_t a, uint32_t, uint64_t b, uint32_t) { return a > b; };
  bitonic_best_first(hk, nullptr, np, key_only);
  bitonic_best_first(hk + SDM_MAX_HALF, nullptr, np, key_only);
  for (int s = 0; s < 2; ++s)
    for (int i = lane; i < k; i += 64) {
      const uint64_t key = hk[s * SDM_MAX_HALF + i];
      topv[s][i] = unord32((uint32_t)(key >> 32));
      topi[s][i] = 0xffffffffu - (uint32_t)(key & 0xffffffffu);
    }
  __syncthreads();

  // ---- 2. dominance-pruned candidates (r1+1)(r2+1) <= count ----
  uint64_t* ck = reinterpret_cast<uint64_t*>(keys_raw);
  int total = 0;
  for (int r1 = 0; r1 < k; ++r1) {
    const int c = min(k, count / (r1 + 1));
    total += c;
  }
  const int npc = pow2_at_least(total);
  uint32_t* cid = reinterpret_cast<uint32_t*>(keys_raw + npc * 8);
  for (int r1 = lane; r1 < k; r1 += 64) {
    int off = 0;
    for (int a = 0; a < r1; ++a) off += min(k, count / (a + 1));
    const int c = min(k, count / (r1 + 1));
    const double va = (double)topv[0][r1];
    const uint32_t ia = topi[0][r1] * (uint32_t)n;
    for (int r2 = 0; r2 < c; ++r2) {
      const double s = va + (double)topv[1][r2];  // exact in fp64
      ck[off + r2] = ord64(s);
      cid[off + r2] = ia + topi[1][r2];
    }
  }
  for (int i = total + lane; i < npc; i += 64) {
    ck[i] = 0ull;
    cid[i] = 0xffffffffu;
  }
  __syncthreads();

  // ---- 3. rank by (score desc, id asc), keep `count` ----
  auto score_then_id = [](uint64_t a, uint32_t ia, uint64_t b, uint32_t ib) {
    return a > b || (a == b && ia < ib);
  };
  bitonic_best_first(ck, cid, npc, score_then_id);
  const double smax = unord64(ck[0]);
  __syncthreads();

  // ---- 4. ids ascending, softmax weights ----
  const int npo = pow2_at_least(count);
  for (int i = count + lane; i < npo; i += 64) {
    ck[i] = 0ull;
    cid[i] = 0xffffffffu;
  }
  __syncthreads();
  auto id_asc = [](uint64_t, uint32_t ia, uint64_t, uint32_t ib) { return ia < ib; };
  bitonic_best_first(ck, cid, npo, id_asc);

  float wsum = 0.0f;
  float wloc[SDM_MAX_COUNT / 64];
#pragma unroll
  for (int q = 0; q < SDM_MAX_COUNT / 64; ++q) {
    const int i = lane + q * 64;
    wloc[q] = (i < count) ? expf((float)(unord64(ck[i]) - smax)) : 0.0f;
    wsum += wloc[q];
  }
  red[lane] = wsum;
  __syncthreads();
  float tot = 0.0f;
  for (int i = 0; i < 64; ++i) tot += red[i];
  const float inv = 1.0f / tot;
  const int64_t base = ((out_row0 + r) * H + h) * (int64_t)count;
  int32_t* oi = role ? idx_r : idx_w;
  float* ow = role ? wt_r : wt_w;
#pragma unroll
  for (int q = 0; q < SDM_MAX_COUNT / 64; ++q) {
    const int i = lane + q * 64;
    if (i < count) {
      oi[base + i] = (int32_t)cid[i];
      ow[base + i] = wloc[q] * inv;
    }
  }
}

}  // namespace

hipError_t launch_select(const sdm_dims& d, const float* scores, int64_t rows, int64_t out_row0,
                         int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                         hipStream_t s) {
  const int64_t probs = rows * d.H * 2;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)probs), dim3(64), 0, s, scores, rows, d.H, d.n,
                     d.W, d.R, out_row0, idx_w, wt_w, idx_r, wt_r);
  return hipGetLastError();
}

}  // namespace sdm
