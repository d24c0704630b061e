// Chunkwise-parallel schedule of the scan (SDM_FLAG_SCAN_CHUNK), both write rules.
//
// The form is the one the m.163.com article on arXiv 2607.07386 (section 八,
// training paragraph) and the paper.rainbus.top summary (the novelty paragraph:
// chunk-wise parallelism through the WY representation) describe: fixed-size
// chunks, parallel inside a chunk and serial across chunks, with the mutual
// influence of two tokens a sparse inner product of their ascending slot lists,
// found by a two-pointer merge.  For both rules every slot j written by token u
// evolves as M[j] <- a_{u,j} M[j] + k_{u,j} x_u, where
//   per-slot rule:  a_{u,j} = alpha_u (1 - beta_u k_{u,j}),  x_u = beta_u v_u
//   GDN rule:       a_{u,j} = alpha_u,
//                   x_u = beta_u (v_u - alpha_u sum_{j in W_u} k_{u,j} M_{u-1}[j]).
// With L_j(t) the sum of log a_{u,j} over the chunk's writers u <= t of slot j,
// G_j(s, t] = exp(L_j(t) - L_j(s)) and M0 the state at the chunk start:
//   y_t = sum_{j in R_t} q_{t,j} exp(L_j(t)) M0[j] + sum_{s <= t} A_{t,s} x_s,
//   A_{t,s} = sum over j in R_t and W_s of q_{t,j} k_{s,j} G_j(s, t]        (merge)
//   GDN:  x = Tm (v - r),  r_t = sum_{j in W_t} k_{t,j} exp(L_j(t)) M0[j],
//         Tm = (I + diag(beta) B)^-1 diag(beta),
//         B_{t,s} = sum over j in W_t and W_s of k_{t,j} k_{s,j} G_j(s, t]  (merge, s < t)
//   chunk end, per slot j written in the chunk (its last writer e):
//         M[j] = exp(L_j(e)) M0[j] + sum over j's writers s of G_j(s, e] k_{s,j} x_s.
// Every log a is floored at -80: a forget gate that is exactly 0 (or beta k = 1)
// decays by e^-80 instead of to 0, which keeps the differences of L finite.
// Token ids must be ascending within each list (the selection's output order).
//
// chunk_prep: one workgroup per (walk, chunk), all chunks at once: the links
//   between a slot's writers inside the chunk (binary search of the earlier tokens'
//   sorted lists, only for slots that a hashed bitmap shows may repeat), L at every
//   write and read entry, A and, for GDN, B and Tm (forward substitution).  The
//   pairwise sparse inner products are summed through those links rather than by
//   merging every pair of lists: the same sums, but a merge walks all 2W entries of
//   each of the C^2/2 pairs although, with N >> C W, almost no pair shares a slot.
// chunk_walk: one workgroup per (walk, 16-column slice of d_v), the walk's chunks in
//   order: x, the reads and the chunk-end rows (in training also the write log).  The
//   columns of the state evolve independently under both rules, so slices need no
//   communication.  y then goes through the norm/gate kernel.
// chunk_back (training, key-weighted rule): the reverse walk in the same chunks, from
//   chunk_prep's matrices and its chains of each slot's reads (see below).
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kChunk = 32;
constexpr float kLogFloor = -80.0f;
constexpr int32_t kNextBit = 1 << 16;  // link word: a later writer of the slot exists
// Backward read chains.  Read word: bits 0-12 the previous read of the same slot that
// saw the same row (entry + 1, 0 if none); kReadOnlyTail on the last read of a slot
// the chunk does not write; kReadNext (prep only) when a later read continues the
// chain; bits 16-28 (prep only) the slot's first writer + 1 for a read of the
// chunk-start row.  Write word: bits 0-12 the last read that saw the row this write
// left (+ 1); bits 16-28, on a slot's first writer, the last read before it (+ 1).
constexpr int32_t kPrevMask = 0x1fff;
constexpr int32_t kReadOnlyTail = 1 << 13;
constexpr int32_t kReadNext = 1 << 14;
constexpr int kSlice = 16;             // state columns per chunk_walk workgroup
constexpr int kBatch = 16;             // rows a lane group keeps in flight
constexpr int kWalkThreads = 512;      // chunk_walk: four lane groups per token
// chunk_prep marks each written slot in two hashed bitmaps (seen once, seen again),
// so that only entries whose slot may occur twice in the chunk search for it
constexpr int kFilterBits = 16;
constexpr int kFilterWords = (1 << kFilterBits) / 32;

__device__ __forceinline__ uint32_t slot_hash(int32_t j) {
  return ((uint32_t)j * 2654435761u) >> (32 - kFilterBits);
}

struct ChunkArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* alpha;
  const float* beta;
  float* Lw;       // [B, T, H, W] L at each write entry (through its own token)
  float* Lr;       // [B, T, H, R] L at each read entry
  int32_t* link;   // [B, T, H, W] low 16 bits: previous writer (s W + k) + 1, 0 if none
  float* Am;       // [walks][chunks][C][C] A_{t,s}, zero above the diagonal
  float* Tm;       // [walks][chunks][C][C] GDN only
  float* state;    // [B, H, N, d_v] fp32
  float* y;        // [B, T, H, d_v]
  float* log;      // training forward: [B, T, H, W, d_v] fp32 rows before each write, or null
  // backward only
  int32_t* rch;    // [B, T, H, R] read words
  int32_t* wrd;    // [B, T, H, W] write words
  float* dM;       // [B, H, N, d_v] IN dL/dM at the end, OUT at the start
  const float* dy; // [B, T, H, d_v] gradient of the read vectors
  float* g_v;      // [B, T, H, d_v] d_v
  float* pr;       // [S][B*T*H][R] per-slice shares of d_wt_r
  float2* pw;      // [S][B*T*H][W] per-slice shares of (<G, e>, <de, m>)
  float* pa;       // [S][B*T*H] per-slice shares of d_alpha
  int64_t B, T;
  int64_t rows;    // B T H
  int32_t H, N, W, R, d_v, chunks;
};

// Position of key in the ascending list ids[0..n), or -1.
__device__ __forceinline__ int find_sorted(const int32_t* ids, int n, int32_t key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return (lo < n && ids[lo] == key) ? lo : -1;
}

__device__ __forceinline__ float4 fma4(float s, float4 m, float4 acc) {
  acc.x = fmaf(s, m.x, acc.x);
  acc.y = fmaf(s, m.y, acc.y);
  acc.z = fmaf(s, m.z, acc.z);
  acc.w = fmaf(s, m.w, acc.w);
  return acc;
}
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// LDS words of chunk_prep: write lists (ids, k, L, links), read-side L and latest
// writers, A, B and Tm, beta, the two slot bitmaps.  The backward's read chains reuse
// the k, read-L and A/B/Tm words once those are stored (R <= 3 C).
size_t prep_lds_bytes(int W, int R) {
  return ((size_t)4 * kChunk * W + 2 * kChunk * R + 3 * kChunk * kChunk + kChunk +
          2 * kFilterWords) * 4;
}

template <bool GDN, bool BACK = false>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs a) {
  constexpr int C = kChunk;
  extern __shared__ int32_t lds[];
  const int W = a.W, R = a.R;
  int32_t* iw = lds;
  float* kw = reinterpret_cast<float*>(iw + C * W);
  float* lw = kw + C * W;
  int32_t* lk = reinterpret_cast<int32_t*>(lw + C * W);
  float* lr = reinterpret_cast<float*>(lk + C * W);
  int32_t* rl = reinterpret_cast<int32_t*>(lr + C * R);  // latest writer + 1, 0 if none
  float* Al = reinterpret_cast<float*>(rl + C * R);
  float* Bm = Al + C * C;
  float* Tl = Bm + C * C;
  float* be = Tl + C * C;
  uint32_t* seen1 = reinterpret_cast<uint32_t*>(be + C);
  uint32_t* seen2 = seen1 + kFilterWords;

  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x / a.chunks;
  const int c = (int)(blockIdx.x - w * a.chunks);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int64_t t0 = (int64_t)c * C;
  const int Cc = (int)(a.T - t0 < C ? a.T - t0 : C);
  auto tok = [&](int t) { return (b * a.T + t0 + t) * a.H + h; };

  // the chunk's write lists; the log decay of each write entry
#pragma unroll 4
  for (int e = tid; e < Cc * W; e += 256) {
    const int t = e / W, k = e - t * W;
    const int64_t gi = tok(t) * W + k;
    const float kk = a.wt_w[gi];
    iw[e] = a.idx_w[gi];
    kw[e] = kk;
    float la = logf(a.alpha[tok(t)]);
    if (!GDN) la += log1pf(-a.beta[tok(t)] * kk);
    lw[e] = fmaxf(la, kLogFloor);
    lk[e] = 0;
  }
  if (tid < Cc) be[tid] = a.beta[tok(tid)];
  for (int i = tid; i < 2 * kFilterWords; i += 256) seen1[i] = 0u;
  __syncthreads();
  for (int e = tid; e < Cc * W; e += 256) {
    const uint32_t hs = slot_hash(iw[e]);
    const uint32_t bit = 1u << (hs & 31);
    if (atomicOr(&seen1[hs >> 5], bit) & bit) atomicOr(&seen2[hs >> 5], bit);
  }
  __syncthreads();

  // links: the latest earlier token of the chunk writing the same slot (ORs commute,
  // so the words do not depend on the threads' order).  A slot whose hash was
  // written once has no other writer; for the others the whole wavefront searches
  // together, lane u in token u's list, and the highest lane that finds it wins.
  const int lane = tid & 63;
  for (int e0 = tid - lane; e0 < Cc * W; e0 += 256) {
    const int e = e0 + lane;
    int32_t j = 0;
    bool maybe = false;
    if (e < Cc * W) {
      j = iw[e];
      const uint32_t hs = slot_hash(j);
      maybe = (seen2[hs >> 5] >> (hs & 31)) & 1u;
    }
    uint64_t m = __ballot(maybe);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const int32_t jj = __shfl(j, l);
      const int te = (e0 + l) / W;
      const int pos = lane < te ? find_sorted(iw + lane * W, W, jj) : -1;
      const uint64_t hit = __ballot(pos >= 0);
      if (hit) {
        const int u = 63 - __builtin_clzll(hit);
        const int p = __shfl(pos, u);
        if (lane == 0) {
          atomicOr(&lk[e0 + l], u * W + p + 1);
          atomicOr(&lk[u * W + p], kNextBit);
        }
      }
    }
  }
  __syncthreads();

  // L at each write entry: its own log decay plus those of the earlier writers
  constexpr int kMaxPer = C * SDM_MAX_COUNT / 256;
  float run[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = tid + 256 * i;
    float s = 0.0f;
    if (e < Cc * W) {
      s = lw[e];
      int p = lk[e] & 0xffff;
      while (p) {
        s += lw[p - 1];
        p = lk[p - 1] & 0xffff;
      }
    }
    run[i] = s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = tid + 256 * i;
    if (e < Cc * W) lw[e] = run[i];
  }
  __syncthreads();

  // each read entry: the slot's latest writer at or before the token and its L (none
  // if the slot's hash was never written), searched by the whole wavefront as above
  for (int e0 = tid - lane; e0 < Cc * R; e0 += 256) {
    const int e = e0 + lane;
    int32_t j = 0;
    bool maybe = false;
    if (e < Cc * R) {
      const int t = e / R, k = e - t * R;
      j = a.idx_r[tok(t) * R + k];
      const uint32_t hs = slot_hash(j);
      maybe = (seen1[hs >> 5] >> (hs & 31)) & 1u;
    }
    float L = 0.0f;
    int lat = 0;
    uint64_t m = __ballot(maybe);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const int32_t jj = __shfl(j, l);
      const int te = (e0 + l) / R;
      const int pos = lane <= te ? find_sorted(iw + lane * W, W, jj) : -1;
      const uint64_t hit = __ballot(pos >= 0);
      if (hit) {
        const int u = 63 - __builtin_clzll(hit);
        const int p = __shfl(pos, u);
        if (lane == l) {
          L = lw[u * W + p];
          lat = u * W + p + 1;
        }
      }
    }
    if (e < Cc * R) {
      lr[e] = L;
      rl[e] = lat;
    }
  }
  __syncthreads();

  // The tokens' pairwise sparse inner products.  A pair shares a slot exactly when
  // the reading (or later writing) token's entry links to a writer of the other one,
  // so each sum runs over the links instead of merging the two full lists: row t of
  // A over t's read entries in order, each through its slot's writers s <= t (latest
  // first); row t of B over t's write entries, each through the earlier writers.
  if (tid < C) {
    const int t = tid;
    for (int s = 0; s < C; ++s) Al[t * C + s] = 0.0f;
    if (t < Cc) {
      for (int k = 0; k < R; ++k) {
        int p = rl[t * R + k];
        if (!p) continue;
        const float q = a.wt_r[tok(t) * R + k];
        const float L = lr[t * R + k];
        while (p) {
          const int s = (p - 1) / W;
          Al[t * C + s] += q * kw[p - 1] * expf(L - lw[p - 1]);
          p = lk[p - 1] & 0xffff;
        }
      }
    }
  } else if (GDN && tid >= 64 && tid < 64 + C) {
    const int t = tid - 64;
    for (int s = 0; s < C; ++s) Bm[t * C + s] = 0.0f;
    if (t < Cc) {
      for (int k = 0; k < W; ++k) {
        const int e = t * W + k;
        int p = lk[e] & 0xffff;
        if (!p) continue;
        const float kt = kw[e], L = lw[e];
        while (p) {
          const int s = (p - 1) / W;
          Bm[t * C + s] += kt * kw[p - 1] * expf(L - lw[p - 1]);
          p = lk[p - 1] & 0xffff;
        }
      }
    }
  }
  __syncthreads();
  float* Ag = a.Am + ((int64_t)w * a.chunks + c) * C * C;
  for (int pi = tid; pi < C * C; pi += 256) Ag[pi] = Al[pi];

  if (GDN) {
    // Tm = (I + diag(beta) B)^-1 diag(beta), row by row; lane m owns column m
    if (tid < C) {
      const int m = tid;
      for (int t = 0; t < C; ++t) {
        float acc = t == m ? 1.0f : 0.0f;
        for (int s = 0; s < t; ++s) acc = fmaf(-Bm[t * C + s], Tl[s * C + m], acc);
        Tl[t * C + m] = t < Cc ? be[t] * acc : 0.0f;
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    float* Tg = a.Tm + ((int64_t)w * a.chunks + c) * C * C;
    for (int pi = tid; pi < C * C; pi += 256) Tg[pi] = Tl[pi];
  }

  for (int e = tid; e < Cc * W; e += 256) {
    const int t = e / W, k = e - t * W;
    const int64_t gi = tok(t) * W + k;
    a.Lw[gi] = lw[e];
    a.link[gi] = lk[e];
  }
  for (int e = tid; e < Cc * R; e += 256) {
    const int t = e / R, k = e - t * R;
    a.Lr[tok(t) * R + k] = lr[e];
  }

  if constexpr (BACK) {
    // Chains of each slot's reads for the backward, in words freed above: read ids in
    // the read-L words, read words in A/B/Tm, write words in the k words.
    __syncthreads();
    int32_t* irl = reinterpret_cast<int32_t*>(lr);
    int32_t* rw = reinterpret_cast<int32_t*>(Al);
    int32_t* wrd = reinterpret_cast<int32_t*>(kw);
    for (int e = tid; e < Cc * R; e += 256) {
      const int t = e / R, k = e - t * R;
      irl[e] = a.idx_r[tok(t) * R + k];
    }
    __syncthreads();
    // A read of the chunk-start row of a slot the chunk writes later: that slot's first
    // writer, the earliest later token whose write list holds it (lowest lane wins).
    for (int e0 = tid - lane; e0 < Cc * R; e0 += 256) {
      const int e = e0 + lane;
      int32_t j = 0;
      bool maybe = false;
      if (e < Cc * R) {
        j = irl[e];
        const uint32_t hs = slot_hash(j);
        maybe = rl[e] == 0 && ((seen1[hs >> 5] >> (hs & 31)) & 1u);
        rw[e] = 0;
      }
      uint64_t m = __ballot(maybe);
      while (m) {
        const int l = __builtin_ctzll(m);
        m &= m - 1;
        const int32_t jj = __shfl(j, l);
        const int te = (e0 + l) / R;
        const int pos = (lane > te && lane < Cc) ? find_sorted(iw + lane * W, W, jj) : -1;
        const uint64_t hit = __ballot(pos >= 0);
        if (hit) {
          const int u = __builtin_ctzll(hit);
          const int p = __shfl(pos, u);
          if (lane == l) rw[e] = (u * W + p + 1) << 16;
        }
      }
    }
    for (int i = tid; i < Cc * W; i += 256) wrd[i] = 0;
    __syncthreads();
    for (int i = tid; i < 2 * kFilterWords; i += 256) seen1[i] = 0u;
    __syncthreads();
    for (int e = tid; e < Cc * R; e += 256) {
      const uint32_t hs = slot_hash(irl[e]);
      const uint32_t bit = 1u << (hs & 31);
      if (atomicOr(&seen1[hs >> 5], bit) & bit) atomicOr(&seen2[hs >> 5], bit);
    }
    __syncthreads();
    // the latest earlier read of the same slot; it continues the chain when it saw the
    // same row (the same latest writer, or both the chunk-start row)
    for (int e0 = tid - lane; e0 < Cc * R; e0 += 256) {
      const int e = e0 + lane;
      int32_t j = 0;
      bool maybe = false;
      if (e < Cc * R) {
        j = irl[e];
        const uint32_t hs = slot_hash(j);
        maybe = (seen2[hs >> 5] >> (hs & 31)) & 1u;
      }
      int prev = 0;
      uint64_t m = __ballot(maybe);
      while (m) {
        const int l = __builtin_ctzll(m);
        m &= m - 1;
        const int32_t jj = __shfl(j, l);
        const int te = (e0 + l) / R;
        const int pos = lane < te ? find_sorted(irl + lane * R, R, jj) : -1;
        const uint64_t hit = __ballot(pos >= 0);
        if (hit) {
          const int u = 63 - __builtin_clzll(hit);
          const int p = __shfl(pos, u);
          if (lane == l) prev = u * R + p + 1;
        }
      }
      if (prev && rl[prev - 1] == rl[e]) {
        atomicOr(&rw[e], prev);
        atomicOr(&rw[prev - 1], kReadNext);
      }
    }
    __syncthreads();
    // chain tails: the last read of a writer's row, the last read of the chunk-start
    // row before the slot's first writer, or the last read of a slot not written
    for (int e = tid; e < Cc * R; e += 256) {
      const int32_t wv = rw[e];
      if (wv & kReadNext) continue;
      if (rl[e])
        atomicOr(&wrd[rl[e] - 1], e + 1);
      else if (wv >> 16)
        atomicOr(&wrd[(wv >> 16) - 1], (e + 1) << 16);
      else
        atomicOr(&rw[e], kReadOnlyTail);
    }
    __syncthreads();
    for (int e = tid; e < Cc * R; e += 256) {
      const int t = e / R, k = e - t * R;
      a.rch[tok(t) * R + k] = rw[e] & (kPrevMask | kReadOnlyTail);
    }
    for (int e = tid; e < Cc * W; e += 256) {
      const int t = e / W, k = e - t * W;
      a.wrd[tok(t) * W + k] = wrd[e];
    }
  }

}

size_t walk_lds_bytes(int W, int R) {
  return ((size_t)4 * kChunk * W + 3 * kChunk * R + 2 * kChunk * kChunk) * 4 +
         (size_t)(2 * kChunk + kWalkThreads / (kSlice / 4)) * (kSlice / 4) * 16;
}

// Weighted sum of rows ids[e] (e = e0 + GPT i, i < cnt) of this lane's 4 columns,
// weight wt[e] exp(L[e]), kBatch rows in flight.
template <int GPT>
__device__ __forceinline__ float4 gather_sum(const float* Mb, int d_v, const int32_t* ids,
                                             const float* wt, const float* L, int e0, int cnt) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < cnt; i0 += kBatch) {
    float4 m[kBatch];
    float s[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool ok = i0 + u < cnt;
      const int e = ok ? e0 + GPT * (i0 + u) : e0;
      s[u] = ok ? wt[e] * expf(L[e]) : 0.0f;
      m[u] = *reinterpret_cast<const float4*>(Mb + (int64_t)ids[e] * d_v);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) acc = fma4(s[u], m[u], acc);
  }
  return acc;
}

// LOG (training forward): each slot's last writer also stores the row every writer of
// its chain replaced -- the chunk-start row for the first, else the fold above taken
// at the previous writer -- to the write log.
template <bool GDN, bool LOG>
__global__ __launch_bounds__(kWalkThreads) void chunk_walk_kernel(ChunkArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = kWalkThreads;
  constexpr int LPR = kSlice / 4;  // lanes per row slice (one float4 each)
  constexpr int G = NT / LPR;      // lane groups
  constexpr int GPT = G / C;       // lane groups per token
  static_assert(GPT * C == G, "whole lane groups per token");
  extern __shared__ int32_t lds[];
  const int W = a.W, R = a.R;
  int32_t* iw = lds;
  float* kw = reinterpret_cast<float*>(iw + C * W);
  float* lw = kw + C * W;
  int32_t* lk = reinterpret_cast<int32_t*>(lw + C * W);
  int32_t* ir = lk + C * W;
  float* qr = reinterpret_cast<float*>(ir + C * R);
  float* lr = qr + C * R;
  float* Am = lr + C * R;
  float* Tl = Am + C * C;
  float4* xs = reinterpret_cast<float4*>(Tl + C * C);  // [C][LPR] x_t
  float4* vr = xs + C * LPR;                            // [C][LPR] v_t - r_t (GDN)
  float4* part = vr + C * LPR;                          // [G][LPR]

  const int tid = threadIdx.x;
  const int li = tid % LPR, g = tid / LPR;
  const int tl = g / GPT, sub = g % GPT;  // the token and share of its lists this group takes
  const int64_t walks = a.B * a.H;
  const int64_t w = blockIdx.x % walks;
  const int slice = (int)(blockIdx.x / walks);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int d_v = a.d_v;
  float* const Mb = a.state + w * (int64_t)a.N * d_v + slice * kSlice + li * 4;
  const int col = slice * kSlice;

  for (int c = 0; c < a.chunks; ++c) {
    const int64_t t0 = (int64_t)c * C;
    const int Cc = (int)(a.T - t0 < C ? a.T - t0 : C);
    auto tok = [&](int t) { return (b * a.T + t0 + t) * a.H + h; };
    const int64_t cm = ((int64_t)w * a.chunks + c) * C * C;
    // stage the chunk's lists: every load of a round issued before its LDS stores
    constexpr int kRounds = C * SDM_MAX_COUNT / NT;
    {
      int32_t v0[kRounds], v3[kRounds];
      float v1[kRounds], v2[kRounds];
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * W) {
          const int t = e / W, k = e - t * W;
          const int64_t gi = tok(t) * W + k;
          v0[i] = a.idx_w[gi];
          v1[i] = a.wt_w[gi];
          v2[i] = a.Lw[gi];
          v3[i] = a.link[gi];
        }
      }
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * W) {
          iw[e] = v0[i];
          kw[e] = v1[i];
          lw[e] = v2[i];
          lk[e] = v3[i];
        }
      }
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * R) {
          const int t = e / R, k = e - t * R;
          const int64_t gi = tok(t) * R + k;
          v0[i] = a.idx_r[gi];
          v1[i] = a.wt_r[gi];
          v2[i] = a.Lr[gi];
        }
      }
#pragma unroll
      for (int i = 0; i < kRounds; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * R) {
          ir[e] = v0[i];
          qr[e] = v1[i];
          lr[e] = v2[i];
        }
      }
    }
    for (int pi = tid; pi < C * C; pi += NT) {
      Am[pi] = a.Am[cm + pi];
      if (GDN) Tl[pi] = a.Tm[cm + pi];
    }
    __syncthreads();

    // x_t for this slice
    if (GDN) {
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tl < Cc) r = gather_sum<GPT>(Mb, d_v, iw, kw, lw, tl * W + sub, (W - sub + GPT - 1) / GPT);
      part[g * LPR + li] = r;
      __syncthreads();
      if (tid < C * LPR) {
        const int t = tid / LPR, q = tid % LPR;
        float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < Cc) {
          const float4 vv = reinterpret_cast<const float4*>(a.v + tok(t) * d_v + col)[q];
          float4 rr = part[(GPT * t) * LPR + q];
#pragma unroll
          for (int u = 1; u < GPT; ++u) rr = add4(rr, part[(GPT * t + u) * LPR + q]);
          d = make_float4(vv.x - rr.x, vv.y - rr.y, vv.z - rr.z, vv.w - rr.w);
        }
        vr[t * LPR + q] = d;
      }
      __syncthreads();
      if (tid < C * LPR) {
        const int t = tid / LPR, q = tid % LPR;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s <= t; ++s) x = fma4(Tl[t * C + s], vr[s * LPR + q], x);
        xs[t * LPR + q] = x;
      }
    } else if (tid < C * LPR) {
      const int t = tid / LPR, q = tid % LPR;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < Cc) {
        const float be = a.beta[tok(t)];
        const float4 vv = reinterpret_cast<const float4*>(a.v + tok(t) * d_v + col)[q];
        x = make_float4(be * vv.x, be * vv.y, be * vv.z, be * vv.w);
      }
      xs[t * LPR + q] = x;
    }

    // reads: the chunk-start rows, then the chunk's own writes through A
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tl < Cc) acc = gather_sum<GPT>(Mb, d_v, ir, qr, lr, tl * R + sub, (R - sub + GPT - 1) / GPT);
    part[g * LPR + li] = acc;
    __syncthreads();  // every read of the chunk-start rows is done past this point
    if (tid < C * LPR) {
      const int t = tid / LPR, q = tid % LPR;
      if (t < Cc) {
        float4 y = part[(GPT * t) * LPR + q];
#pragma unroll
        for (int u = 1; u < GPT; ++u) y = add4(y, part[(GPT * t + u) * LPR + q]);
        for (int s = 0; s <= t; ++s) y = fma4(Am[t * C + s], xs[s * LPR + q], y);
        reinterpret_cast<float4*>(a.y + tok(t) * d_v + col)[q] = y;
      }
    }

    // chunk-end rows: the last writer of each slot folds its chain of writers
    for (int e0 = g; e0 < Cc * W; e0 += G * kBatch) {
      float4 m[kBatch];
      bool last[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + G * u;
        last[u] = e < Cc * W && !(lk[e] & kNextBit);
        m[u] = *reinterpret_cast<const float4*>(Mb + (int64_t)iw[last[u] ? e : e0] * d_v);
      }
      // the row after writer q of a chain: the chunk-start row and every writer of the
      // chain up to q, each decayed to q
      auto fold = [&](int q, float4 m0) {
        const float lq = lw[q];
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
        r = fma4(expf(lq), m0, r);
        int p = q + 1;
        while (p) {
          const int s = (p - 1) / W;
          r = fma4(expf(lq - lw[p - 1]) * kw[p - 1], xs[s * LPR + li], r);
          p = lk[p - 1] & 0xffff;
        }
        return r;
      };
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (!last[u]) continue;
        const int e = e0 + G * u;
        *reinterpret_cast<float4*>(Mb + (int64_t)iw[e] * d_v) = fold(e, m[u]);
        if constexpr (LOG) {
          for (int c = e;;) {  // the chain backwards: the row each writer replaced
            const int p = lk[c] & 0xffff;  // previous writer + 1, 0 for the first
            const float4 before = p ? fold(p - 1, m[u]) : m[u];
            const int s = c / W;
            const int64_t lr = tok(s) * W + (c - s * W);
            *reinterpret_cast<float4*>(a.log + lr * d_v + col + li * 4) = before;
            if (!p) break;
            c = p - 1;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---- backward (key-weighted rule) ---------------------------------------------
// The reverse walk in the same chunks, chunks in reverse order.  Within a chunk the
// only coupling between slots is de_u = beta_u sum_{j in W_u} k_{u,j} G_{u,j}, with
// G_{u,j} = dL/dM[j] just after token u's write.  Following slot j back from the
// chunk end, G_{u,j} = G_j(u, end] dM_end[j] + sum over reads (t >= u) of
// q_{t,j} G_j(u, t] dy_t - sum over later writers u' of k_{u',j} G_j(u, u'] de_{u'}, so
//   de = Tm^T h,  h_u = sum_{t >= u} A_{t,u} dy_t + sum_{j in W_u} k_{u,j} G_j(u, end] dM_end[j]
// (Tm, A from chunk_prep).  With de known, every slot the chunk touches is walked back
// on its own by one lane group: its reads (each saw the row its latest writer left)
// and writes in reverse, the G of each write, the restored row and the chunk-start
// gradient -- the same per-entry steps as the direct reverse walk.
//
// One workgroup of 512 threads per (walk, 16-column slice).  Lane group (token u,
// share s) owns write and read entries s, s + GPT, ... of u: it gathers the dM_end and
// logged rows of its write entries for h and for e_u = v_u - alpha_u sum k m, and
// walks the slots whose last writer they are, loading those rows again (a whole
// token's rows do not fit in the registers across the solve).  Each slot a token
// only reads is walked by its last read.  Dot products over d_v go out as per-slice
// shares (d_wt_r, (<G, e>, <de, m>), d_alpha), summed in slice order afterwards.
constexpr int kBackThreads = 512;
constexpr int kBackEPG = 16;  // entries of each list a lane group owns: W, R <= 64
constexpr int kBackBatch = 2;  // rows of each kind a lane group loads at once

size_t back_lds_bytes(int W, int R) {
  // write lists (ids, k, L, links, words, h weights, alpha shares), read lists (ids,
  // q, words), A, Tm, alpha; per-token slices of dy, e, de, h; the groups' h and P
  constexpr int LPR = kSlice / 4;
  return ((size_t)7 * kChunk * W + 3 * kChunk * R + 2 * kChunk * kChunk + kChunk) * 4 +
         (size_t)(4 * kChunk + 2 * (kBackThreads / LPR)) * LPR * 16;
}

template <int LPR>
__device__ __forceinline__ float lane_group_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, LPR);
  return x;
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Element at a 32-bit byte offset from a wave-uniform base (one address register
// per access instead of a 64-bit pointer).
template <typename T>
__device__ __forceinline__ T& at(T* base, uint32_t byte_off) {
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ const T& at(const T* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

__global__ __launch_bounds__(kBackThreads) void chunk_back_kernel(ChunkArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = kBackThreads;
  constexpr int LPR = kSlice / 4;
  constexpr int G = NT / LPR;
  constexpr int GPT = G / C;
  static_assert(GPT * C == G && GPT * kBackEPG == 64, "lane groups per token");
  extern __shared__ int32_t lds[];
  const int W = a.W, R = a.R;
  int32_t* iw = lds;
  float* kw = reinterpret_cast<float*>(iw + C * W);
  float* lw = kw + C * W;
  int32_t* lk = reinterpret_cast<int32_t*>(lw + C * W);
  int32_t* wr = lk + C * W;
  float* wg = reinterpret_cast<float*>(wr + C * W);  // k e^(L_last - L), for h
  float* gm = wg + C * W;                            // <G - k de, m> per write entry
  int32_t* ir = reinterpret_cast<int32_t*>(gm + C * W);
  float* qr = reinterpret_cast<float*>(ir + C * R);
  int32_t* rc = reinterpret_cast<int32_t*>(qr + C * R);
  float* Am = reinterpret_cast<float*>(rc + C * R);
  float* Tl = Am + C * C;
  float* al = Tl + C * C;
  float4* dyv = reinterpret_cast<float4*>(al + C);  // [C][LPR]
  float4* eu = dyv + C * LPR;
  float4* dev = eu + C * LPR;
  float4* hv = dev + C * LPR;
  float4* partH = hv + C * LPR;  // [G][LPR]
  float4* partP = partH + G * LPR;

  const int tid = threadIdx.x;
  const int li = tid % LPR, g = tid / LPR;
  const int tl = g / GPT, sub = g % GPT;
  const int64_t walks = a.B * a.H;
  const int64_t w = blockIdx.x % walks;
  const int slice = (int)(blockIdx.x / walks);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int H = a.H;
  const uint32_t d_v = (uint32_t)a.d_v;
  const int col = slice * kSlice;
  // this walk's state and gradient rows from column col; a slot's bytes for this lane
  float* const Mw = a.state + w * (int64_t)a.N * d_v + col;
  float* const dMw = a.dM + w * (int64_t)a.N * d_v + col;
  auto row = [&](int32_t j) { return ((uint32_t)j * d_v + (uint32_t)li * 4u) * 4u; };
  const int64_t prow = (int64_t)slice * a.rows;  // this slice's rows of the shares

  for (int c = a.chunks - 1; c >= 0; --c) {
    const int64_t t0 = (int64_t)c * C;
    const int Cc = (int)(a.T - t0 < C ? a.T - t0 : C);
    const int64_t tok0 = (b * a.T + t0) * H + h;  // token t of the chunk is tok0 + t H
    auto tok = [&](int t) { return tok0 + (int64_t)t * H; };
    // the chunk's logged rows, shares and d_v, each from a uniform base
    const float* const Lg = a.log + tok0 * W * d_v + col;
    auto lrow = [&](int t, int k) {
      return (((uint32_t)t * H * W + (uint32_t)k) * d_v + (uint32_t)li * 4u) * 4u;
    };
    float* const Pr = a.pr + (prow + tok0) * R;
    float2* const Pw = a.pw + (prow + tok0) * W;
    auto rsh = [&](int e) {  // read entry e of the chunk: its share's byte offset
      const int t = e / R;
      return ((uint32_t)t * H * R + (uint32_t)(e - t * R)) * 4u;
    };
    const int64_t cm = ((int64_t)w * a.chunks + c) * C * C;
    {  // stage the chunk's lists: every load issued before the LDS stores
      constexpr int kR = C * 64 / NT;  // W, R <= 64
      int32_t v0[kR], v3[kR], v4[kR], u0[kR], u2[kR];
      float v1[kR], v2[kR], u1[kR];
#pragma unroll
      for (int i = 0; i < kR; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * W) {
          const int t = e / W, k = e - t * W;
          const int64_t gi = tok(t) * W + k;
          v0[i] = a.idx_w[gi];
          v1[i] = a.wt_w[gi];
          v2[i] = a.Lw[gi];
          v3[i] = a.link[gi];
          v4[i] = a.wrd[gi];
        }
        if (e < Cc * R) {
          const int t = e / R, k = e - t * R;
          const int64_t gi = tok(t) * R + k;
          u0[i] = a.idx_r[gi];
          u1[i] = a.wt_r[gi];
          u2[i] = a.rch[gi];
        }
      }
      float am[C * C / NT], tm[C * C / NT];
#pragma unroll
      for (int i = 0; i < C * C / NT; ++i) {
        am[i] = a.Am[cm + tid + NT * i];
        tm[i] = a.Tm[cm + tid + NT * i];
      }
#pragma unroll
      for (int i = 0; i < kR; ++i) {
        const int e = tid + NT * i;
        if (e < Cc * W) {
          iw[e] = v0[i];
          kw[e] = v1[i];
          lw[e] = v2[i];
          lk[e] = v3[i];
          wr[e] = v4[i];
        }
        if (e < Cc * R) {
          ir[e] = u0[i];
          qr[e] = u1[i];
          rc[e] = u2[i];
        }
      }
#pragma unroll
      for (int i = 0; i < C * C / NT; ++i) {
        Am[tid + NT * i] = am[i];
        Tl[tid + NT * i] = tm[i];
      }
    }
    if (tid < C) al[tid] = tid < Cc ? a.alpha[tok(tid)] : 0.0f;
    if (tid < C * LPR) {
      const int t = tid / LPR, q = tid % LPR;
      dyv[tid] = t < Cc ? reinterpret_cast<const float4*>(a.dy + tok(t) * d_v + col)[q]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // h weights along each chain, from its last writer
    for (int e = tid; e < Cc * W; e += NT) {
      if (lk[e] & kNextBit) continue;
      const float Ll = lw[e];
      for (int q = e;;) {
        wg[q] = kw[q] * expf(Ll - lw[q]);
        const int p = lk[q] & 0xffff;
        if (!p) break;
        q = p - 1;
      }
    }
    // slots the chunk only reads: each walked back by its last read (no write of the
    // chunk touches them, so this needs nothing else of the chunk).  Batches are
    // double-buffered: the next batch's rows are loaded before this batch's stores,
    // since loads and stores retire in one order and a load issued after a store
    // would wait for it.
    constexpr int kRB = kBackBatch;
    constexpr int kNB = kBackEPG / kRB;
    if (tl < Cc) {
      float4 dd[2][kRB], ff[2][kRB];
      uint32_t jr[2][kRB];
      auto load_reads = [&](int bi, int buf) {
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          const int k = sub + GPT * (bi * kRB + i);
          jr[buf][i] = row(ir[tl * R + (k < R ? k : 0)]);
        }
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          dd[buf][i] = at(reinterpret_cast<const float4*>(dMw), jr[buf][i]);
          ff[buf][i] = at(reinterpret_cast<const float4*>(Mw), jr[buf][i]);
        }
      };
      load_reads(0, 0);
#pragma unroll
      for (int bi = 0; bi < kNB; ++bi) {
        const int buf = bi & 1;
        if (bi + 1 < kNB) load_reads(bi + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          const int k = sub + GPT * (bi * kRB + i);
          if (k >= R || !(rc[tl * R + k] & kReadOnlyTail)) continue;
          float4 D = dd[buf][i];
          for (int r = tl * R + k + 1; r; r = rc[r - 1] & kPrevMask) {
            const float4 dyt = dyv[((r - 1) / R) * LPR + li];
            const float dq = lane_group_sum<LPR>(dot4(dyt, ff[buf][i]));
            if (li == 0) at(Pr, rsh(r - 1)) = dq;
            D = fma4(qr[r - 1], dyt, D);
          }
          at(reinterpret_cast<float4*>(dMw), jr[buf][i]) = D;
        }
      }
    }
    __syncthreads();  // the h weights are complete
    // this group's write entries: h and P from their dM_end and logged rows
    {
      float4 hs = make_float4(0.f, 0.f, 0.f, 0.f), ps = hs;
      if (tl < Cc) {
#pragma unroll
        for (int i0 = 0; i0 < kBackEPG; i0 += kBackBatch) {
          float4 rD[kBackBatch], rM[kBackBatch];
#pragma unroll
          for (int i = 0; i < kBackBatch; ++i) {
            const int k = sub + GPT * (i0 + i);
            const int kk = k < W ? k : 0;
            rD[i] = at(reinterpret_cast<const float4*>(dMw), row(iw[tl * W + kk]));
            rM[i] = at(reinterpret_cast<const float4*>(Lg), lrow(tl, kk));
          }
#pragma unroll
          for (int i = 0; i < kBackBatch; ++i) {
            const int k = sub + GPT * (i0 + i);
            if (k < W) {
              hs = fma4(wg[tl * W + k], rD[i], hs);
              ps = fma4(kw[tl * W + k], rM[i], ps);
            }
          }
        }
      }
      partH[g * LPR + li] = hs;
      partP[g * LPR + li] = ps;
    }
    __syncthreads();
    if (tid < C * LPR) {
      const int t = tid / LPR, q = tid % LPR;
      float4 hh = make_float4(0.f, 0.f, 0.f, 0.f), ee = hh;
      if (t < Cc) {
        float4 pp = partP[(GPT * t) * LPR + q];
        hh = partH[(GPT * t) * LPR + q];
#pragma unroll
        for (int u = 1; u < GPT; ++u) {
          hh = add4(hh, partH[(GPT * t + u) * LPR + q]);
          pp = add4(pp, partP[(GPT * t + u) * LPR + q]);
        }
        for (int s = t; s < Cc; ++s) hh = fma4(Am[s * C + t], dyv[s * LPR + q], hh);
        const float4 vv = reinterpret_cast<const float4*>(a.v + tok(t) * d_v + col)[q];
        const float at_ = al[t];
        ee = make_float4(vv.x - at_ * pp.x, vv.y - at_ * pp.y, vv.z - at_ * pp.z,
                         vv.w - at_ * pp.w);
      }
      hv[tid] = hh;
      eu[tid] = ee;
    }
    __syncthreads();
    if (tid < C * LPR) {  // de = Tm^T h
      const int t = tid / LPR, q = tid % LPR;
      float4 dd = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = t; s < Cc; ++s) dd = fma4(Tl[s * C + t], hv[s * LPR + q], dd);
      dev[tid] = dd;
      if (t < Cc) reinterpret_cast<float4*>(a.g_v + tok(t) * d_v + col)[q] = dd;
    }
    __syncthreads();

    // each written slot walked back by its last writer (double-buffered as above)
    if (tl < Cc) {
      float4 rD[2][kBackBatch], rM[2][kBackBatch];
      auto load_writes = [&](int bi, int buf) {
#pragma unroll
        for (int i = 0; i < kBackBatch; ++i) {
          const int k = sub + GPT * (bi * kBackBatch + i);
          const int kk = k < W ? k : 0;
          rD[buf][i] = at(reinterpret_cast<const float4*>(dMw), row(iw[tl * W + kk]));
          rM[buf][i] = at(reinterpret_cast<const float4*>(Lg), lrow(tl, kk));
        }
      };
      load_writes(0, 0);
#pragma unroll
      for (int bi = 0; bi < kNB; ++bi) {
        const int buf = bi & 1;
        if (bi + 1 < kNB) load_writes(bi + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < kBackBatch; ++i) {
          const int k = sub + GPT * (bi * kBackBatch + i);
          if (k >= W) continue;
          int e = tl * W + k;
          if (lk[e] & kNextBit) continue;
          const uint32_t j = row(iw[e]);
          float4 D = rD[buf][i], m = rM[buf][i], F = m;
          if (wr[e] & kPrevMask) F = at(reinterpret_cast<const float4*>(Mw), j);
          for (;;) {
            for (int r = wr[e] & kPrevMask; r; r = rc[r - 1] & kPrevMask) {  // saw the row e left
              const float4 dyt = dyv[((r - 1) / R) * LPR + li];
              const float dq = lane_group_sum<LPR>(dot4(dyt, F));
              if (li == 0) at(Pr, rsh(r - 1)) = dq;
              D = fma4(qr[r - 1], dyt, D);
            }
            const int u = e / W;
            const float ke = kw[e];
            const float4 deu = dev[u * LPR + li], euu = eu[u * LPR + li];
            const float4 dm = make_float4(D.x - ke * deu.x, D.y - ke * deu.y, D.z - ke * deu.z,
                                          D.w - ke * deu.w);
            const float ge = lane_group_sum<LPR>(dot4(D, euu));
            const float dem = lane_group_sum<LPR>(dot4(deu, m));
            const float gmv = lane_group_sum<LPR>(dot4(dm, m));
            if (li == 0) {
              at(Pw, ((uint32_t)u * H * W + (uint32_t)(e - u * W)) * 8u) = make_float2(ge, dem);
              gm[e] = gmv;
            }
            const float au = al[u];
            D = make_float4(au * dm.x, au * dm.y, au * dm.z, au * dm.w);
            F = m;  // the row before e's write
            const int p = lk[e] & 0xffff;
            if (!p) break;
            e = p - 1;
            const int us = e / W;
            m = at(reinterpret_cast<const float4*>(Lg), lrow(us, e - us * W));
          }
          for (int r = wr[e] >> 16; r; r = rc[r - 1] & kPrevMask) {  // saw the chunk-start row
            const float4 dyt = dyv[((r - 1) / R) * LPR + li];
            const float dq = lane_group_sum<LPR>(dot4(dyt, F));
            if (li == 0) at(Pr, rsh(r - 1)) = dq;
            D = fma4(qr[r - 1], dyt, D);
          }
          at(reinterpret_cast<float4*>(dMw), j) = D;
          at(reinterpret_cast<float4*>(Mw), j) = F;
        }
      }
    }
    __syncthreads();
    if (tid < Cc) {
      float s = 0.0f;
      for (int k = 0; k < W; ++k) s += gm[tid * W + k];
      a.pa[prow + tok(tid)] = s;
    }
    __syncthreads();  // every row of this chunk is stored before the previous chunk loads
  }
}

int64_t chunks_of(const sdm_dims& d) { return (d.T + kChunk - 1) / kChunk; }

struct ChunkWs {
  size_t lw, lr, link, am, tm, y, total;
};
ChunkWs chunk_ws(const sdm_dims& d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t th = (size_t)d.B * d.T * d.H;
  const size_t mats = (size_t)d.B * d.H * chunks_of(d) * kChunk * kChunk * 4;
  ChunkWs s;
  s.lw = al(th * d.W * 4);
  s.lr = al(th * d.R * 4);
  s.link = al(th * d.W * 4);
  s.am = al(mats);
  s.tm = (d.flags & SDM_FLAG_DELTA_GDN) ? al(mats) : 0;
  s.y = al(th * d.d_v * 4);
  s.total = s.lw + s.lr + s.link + s.am + s.tm + s.y;
  return s;
}

}  // namespace

// The chunk schedule pays while its (walk, 16-column slice) workgroups run in few
// rounds: the chunk walk up to 1024 of them (two per CU), the chunkwise reverse walk
// up to 256 (one per CU).  Beyond that the sliced direct walks, several small
// workgroups per CU, are faster (32,768 tokens in all: forward 6.6 vs 4.0 ms at 256
// walks and 4.6 vs 6.0 ms at 128; reverse walk 11.6 vs 9.6 ms at 64 walks and 12.2
// vs 13.9 ms at 32).
constexpr int64_t kChunkWalkBlocks = 1024;
constexpr int64_t kChunkBackBlocks = 256;
int64_t chunk_blocks(const sdm_dims& d) { return d.B * d.H * (d.d_v / kSlice); }
// Shortest walks the chunk walk takes by default: from two chunks it is at least as
// fast as the sliced walk (32 walks: 0.146 vs 0.147 ms at 64 tokens, 0.20 vs 0.35 ms at
// 128); the chunkwise reverse walk only pays from 256 tokens (0.53 vs 0.49 ms at 128).
constexpr int64_t kChunkMinT = 2 * kChunk;

// Asked for, or the key-weighted rule on an fp32 state from 64 tokens while the walks
// are few enough.
bool scan_uses_chunk(const sdm_dims& d) {
  if (d.flags & SDM_FLAG_SCAN_CHUNK) return true;
  return (d.flags & SDM_FLAG_DELTA_GDN) && !(d.flags & (SDM_FLAG_SCAN_DIRECT | SDM_FLAG_STATE_BF16)) &&
         d.T >= kChunkMinT && chunk_blocks(d) <= kChunkWalkBlocks;
}

size_t chunk_workspace_bytes(const sdm_dims& d) { return chunk_ws(d).total; }

hipError_t launch_chunk_scan(const sdm_dims& d, const ScanArgs& sa, void* ws, hipStream_t st) {
  const ChunkWs s = chunk_ws(d);
  char* p = static_cast<char*>(ws);
  ChunkArgs a;
  a.idx_w = sa.idx_w;
  a.wt_w = sa.wt_w;
  a.idx_r = sa.idx_r;
  a.wt_r = sa.wt_r;
  a.v = sa.v;
  a.alpha = sa.alpha;
  a.beta = sa.beta;
  a.Lw = reinterpret_cast<float*>(p); p += s.lw;
  a.Lr = reinterpret_cast<float*>(p); p += s.lr;
  a.link = reinterpret_cast<int32_t*>(p); p += s.link;
  a.Am = reinterpret_cast<float*>(p); p += s.am;
  a.Tm = s.tm ? reinterpret_cast<float*>(p) : nullptr; p += s.tm;
  a.y = reinterpret_cast<float*>(p);
  a.state = static_cast<float*>(sa.state);
  a.log = static_cast<float*>(sa.log);  // fp32 rows (training forward), or null
  if (a.log && sa.log_fmt != LOG_F32) return hipErrorInvalidValue;
  a.B = sa.B;
  a.T = sa.T;
  a.H = sa.H;
  a.N = sa.N;
  a.W = sa.W;
  a.R = sa.R;
  a.d_v = sa.d_v;
  a.chunks = (int32_t)chunks_of(d);
  const bool gdn = (d.flags & SDM_FLAG_DELTA_GDN) != 0;
  const int64_t walks = sa.B * sa.H;
  {
    const size_t lds = prep_lds_bytes(a.W, a.R);
    const dim3 grid((unsigned)(walks * a.chunks));
    KernelTimer kt("chunk_prep", st);
    if (gdn) {
      hipError_t e = hipFuncSetAttribute((const void*)chunk_prep_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(chunk_prep_kernel<true>, grid, dim3(256), lds, st, a);
    } else {
      hipError_t e = hipFuncSetAttribute((const void*)chunk_prep_kernel<false>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(chunk_prep_kernel<false>, grid, dim3(256), lds, st, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const size_t lds = walk_lds_bytes(a.W, a.R);
    // a walk's slices sit walks apart, so with a multiple of 8 walks they share an
    // XCD (and its L2 copy of the chunk's lists)
    const dim3 grid((unsigned)(walks * (a.d_v / kSlice)));
    KernelTimer kt("chunk_walk", st);
    auto go = [&](auto kern) {
      const hipError_t r = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (r != hipSuccess) return r;
      hipLaunchKernelGGL(kern, grid, dim3(kWalkThreads), lds, st, a);
      return hipSuccess;
    };
    if (gdn && a.log)
      e = go(chunk_walk_kernel<true, true>);
    else if (gdn)
      e = go(chunk_walk_kernel<true, false>);
    else if (a.log)
      e = go(chunk_walk_kernel<false, true>);
    else
      e = go(chunk_walk_kernel<false, false>);
    if (e != hipSuccess) return e;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_norm_gate(sa, a.y, st);
}

namespace {
struct ChunkBackWs {
  size_t lw, lr, link, am, tm, rch, wrd, gpart, dy, pr, pw, pa, total;
};
ChunkBackWs chunk_back_ws(const sdm_dims& d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t th = (size_t)d.B * d.T * d.H;
  const size_t mats = (size_t)d.B * d.H * chunks_of(d) * kChunk * kChunk * 4;
  const size_t S = (size_t)d.d_v / kSlice;
  ChunkBackWs s;
  s.lw = al(th * d.W * 4);
  s.lr = al(th * d.R * 4);
  s.link = al(th * d.W * 4);
  s.am = al(mats);
  s.tm = al(mats);
  s.rch = al(th * d.R * 4);
  s.wrd = al(th * d.W * 4);
  s.gpart = al((size_t)d.B * d.H * norm_backward_blocks(d.T) * d.d_v * 4);
  s.dy = al(th * d.d_v * 4);
  s.pr = al(S * th * d.R * 4);
  s.pw = al(S * th * d.W * 8);
  s.pa = al(S * th * 4);
  s.total = s.lw + s.lr + s.link + s.am + s.tm + s.rch + s.wrd + s.gpart + s.dy + s.pr + s.pw +
            s.pa;
  return s;
}
}  // namespace

// The key-weighted rule's backward on the chunk schedule: with SDM_FLAG_SCAN_CHUNK, or
// from 256 tokens while the walks are few enough, with an fp32 log and W, R <= 64 (the
// lane groups' entries); otherwise the sliced direct reverse walk.
bool gdn_back_uses_chunk(const sdm_dims& d) {
  if (!(d.flags & SDM_FLAG_DELTA_GDN)) return false;
  if (d.flags & (SDM_FLAG_SCAN_DIRECT | SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4)) return false;
  if (!(d.flags & SDM_FLAG_SCAN_CHUNK) &&
      (d.T < kStreamRound || chunk_blocks(d) > kChunkBackBlocks))
    return false;
  constexpr size_t kLds = 160 * 1024;
  return d.W <= 64 && d.R <= 64 && d.d_v % kSlice == 0 && back_lds_bytes(d.W, d.R) <= kLds &&
         prep_lds_bytes(d.W, d.R) <= kLds;
}

size_t chunk_backward_workspace_bytes(const sdm_dims& d) { return chunk_back_ws(d).total; }

hipError_t launch_chunk_backward(const sdm_dims& d, const ScanBackArgs& sa, float* d_norm_w,
                                 void* ws, hipStream_t st) {
  const ChunkBackWs s = chunk_back_ws(d);
  char* p = static_cast<char*>(ws);
  ChunkArgs a{};
  a.idx_w = sa.idx_w;
  a.wt_w = sa.wt_w;
  a.idx_r = sa.idx_r;
  a.wt_r = sa.wt_r;
  a.v = sa.v;
  a.alpha = sa.alpha;
  a.beta = sa.beta;
  a.Lw = reinterpret_cast<float*>(p); p += s.lw;
  a.Lr = reinterpret_cast<float*>(p); p += s.lr;
  a.link = reinterpret_cast<int32_t*>(p); p += s.link;
  a.Am = reinterpret_cast<float*>(p); p += s.am;
  a.Tm = reinterpret_cast<float*>(p); p += s.tm;
  a.rch = reinterpret_cast<int32_t*>(p); p += s.rch;
  a.wrd = reinterpret_cast<int32_t*>(p); p += s.wrd;
  float* gpart = reinterpret_cast<float*>(p); p += s.gpart;
  float* dy = reinterpret_cast<float*>(p); p += s.dy;
  a.pr = reinterpret_cast<float*>(p); p += s.pr;
  a.pw = reinterpret_cast<float2*>(p); p += s.pw;
  a.pa = reinterpret_cast<float*>(p);
  a.state = sa.state;
  a.dM = sa.d_state;
  a.dy = dy;
  a.g_v = sa.g_v;
  a.log = static_cast<float*>(const_cast<void*>(sa.log));
  a.B = sa.B;
  a.T = sa.T;
  a.rows = sa.B * sa.T * sa.H;
  a.H = sa.H;
  a.N = sa.N;
  a.W = sa.W;
  a.R = sa.R;
  a.d_v = sa.d_v;
  a.chunks = (int32_t)chunks_of(d);
  if (sa.log_fmt != LOG_F32 || sa.W > 64 || sa.R > 64 || sa.d_v % kSlice) return hipErrorInvalidValue;
  const int64_t walks = sa.B * sa.H;
  hipError_t e;
  {
    const size_t lds = prep_lds_bytes(a.W, a.R);
    KernelTimer kt("chunk_prep_back", st);
    e = hipFuncSetAttribute((const void*)chunk_prep_kernel<true, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_prep_kernel<true, true>), dim3((unsigned)(walks * a.chunks)),
                       dim3(256), lds, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_norm_backward(sa, dy, gpart, st)) != hipSuccess) return e;
  {
    const size_t lds = back_lds_bytes(a.W, a.R);
    KernelTimer kt("chunk_backward", st);
    e = hipFuncSetAttribute((const void*)chunk_back_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_back_kernel, dim3((unsigned)(walks * (a.d_v / kSlice))),
                       dim3(kBackThreads), lds, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_gdn_back_reduce(sa, a.pr, a.pw, a.pa, a.d_v / kSlice, st)) != hipSuccess)
    return e;
  if (d_norm_w) return launch_gamma_blocks(sa, gpart, d_norm_w, st);
  return hipSuccess;
}

}  // namespace sdm
