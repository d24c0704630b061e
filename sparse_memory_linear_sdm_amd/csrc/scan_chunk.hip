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
//   order: x, the reads and the chunk-end rows.  The columns of the state evolve
//   independently under both rules, so slices need no communication.  y then goes
//   through the norm/gate kernel.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kChunk = 32;
constexpr float kLogFloor = -80.0f;
constexpr int32_t kNextBit = 1 << 16;  // link word: a later writer of the slot exists
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
  int64_t B, T;
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
// writers, A, B and Tm, beta, the two slot bitmaps.
size_t prep_lds_bytes(int W, int R) {
  return ((size_t)4 * kChunk * W + 2 * kChunk * R + 3 * kChunk * kChunk + kChunk +
          2 * kFilterWords) * 4;
}

template <bool GDN>
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

// Asked for, or the key-weighted rule on an fp32 state from 256 tokens (where it is
// several times faster than the direct walk).
bool scan_uses_chunk(const sdm_dims& d) {
  if (d.flags & SDM_FLAG_SCAN_CHUNK) return true;
  return (d.flags & SDM_FLAG_DELTA_GDN) && !(d.flags & (SDM_FLAG_SCAN_DIRECT | SDM_FLAG_STATE_BF16)) &&
         d.T >= kStreamRound;
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

}  // namespace sdm
