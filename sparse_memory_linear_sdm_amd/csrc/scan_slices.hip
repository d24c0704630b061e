// Direct schedule of the key-weighted write rule (SDM_FLAG_DELTA_GDN), split over
// column slices of the state.
//
// The rule ("与 GDN 的关系" section of ai-paper-analysis.pages.dev; Gated
// DeltaNet's rule on the selected slots), per token over its write set I_w:
//   r = sum_j k_j M[j],  M[i] <- alpha M[i] + beta k_i (v - alpha r)   (i in I_w)
//   y = sum_{i in I_r} q_i M[i]   (after the writes),  out = RMSNorm(y) gamma gate
// Every term acts on each of the d_v columns on its own: column c of r, of the
// update and of y involves column c of the rows only.  A walk therefore splits into
// S independent walks over d_v/S columns; only the RMSNorm (a pass over whole rows
// afterwards) and, in the backward, the dot products over d_v (outputs, never fed
// back into the walk) need all columns.
//
// Why: one workgroup per whole walk leaves 32 workgroups on 256 CUs at the
// 1.4B-like shape, each moving its write set a few rows at a time.  Here a
// workgroup owns one slice, and its row groups hold every row of a token in flight
// at once (W, R <= 128 rows in registers), so a token costs about one memory round
// trip for the write set and one for the read set, the latter overlapped with the
// next token's write-set loads.  The norm and gate run in the walk when one slice
// covers the row (d_v <= SDM_GDN_MAX_SW), else in a pass over the raw read vectors.
//
// Sums over the row groups run in a fixed order (a wavefront butterfly, then the
// four wavefronts in order through LDS), so every result is bit-reproducible and
// the training forward equals the inference walk bit for bit.
//
// Backward (training; the m.163.com article on arXiv 2607.07386, section 八: the
// in-place update is undone in backward from the rows it overwrote), per token in
// reverse, m the logged rows, m~ = alpha m, e = v - sum_i k_i m~_i, G_i = dM[i]:
//   read  r:  d_q[r] = <dy, M[r]>,  dM[r] += q[r] dy          (M after t's writes)
//   write:    de = beta sum_i k_i G_i = d_v,  dm~_i = G_i - k_i de,
//             d_k_i = beta <G_i, e> - <de, m~_i>,  d_beta = sum_i k_i <G_i, e>,
//             d_alpha = sum_i <dm~_i, m_i>,  dM[i] = alpha dm~_i,  M[i] = m_i
// e and de are column-wise, so each slice has them whole; each slice writes its
// share of every dot product and a reduce pass sums the slices in order.  dy comes
// from the norm/gate backward of all tokens, run before the walk.
#include "sdm_internal.h"

namespace sdm {
namespace {

// Widest column slice (16, 32, 64 or 128): a group holds SW / 8 rows of each list in
// registers (W, R <= 128), so wide slices cost occupancy.  Measured with 1024 walks
// of 64 tokens (d_v = 128): 2.43 / 1.87 / 1.65 / 1.96 ms for caps 128 / 64 / 32 /
// 16; 32 walks of 4096 tokens take 16-column slices under every cap.
#ifndef SDM_GDN_MAX_SW
#define SDM_GDN_MAX_SW 32
#endif

constexpr int kNW = 4;                              // wavefronts per workgroup
constexpr int64_t kStageBytes = 256ll << 20;        // quantised-log staging bound

struct SliceArgs {
  ScanArgs s;
  float* y;                // raw read vectors [B, T, H, d_v] (y_raw, or workspace)
  float* log;              // fp32 rows: the caller's log, or a token chunk's staging area
  int64_t log_T, log_t0;   // row of (b, t, h, k) at ((b * log_T + t - log_t0) * H + h) * W + k
  int64_t t0, t1;          // tokens of this launch
  int32_t S;               // slices per walk
};

struct SliceBackArgs {
  ScanBackArgs s;
  const float* dy;         // [B, T, H, d_v]
  float* pr;               // [S][B*T*H][R]  each slice's share of d_q
  float2* pw;              // [S][B*T*H][W]  each slice's share of (<G, e>, <de, m>)
  float* pa;               // [S][B*T*H]     each slice's share of d_alpha
  int64_t rows;            // B*T*H
  int32_t S;
};

__device__ __forceinline__ float4 f4z() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ void fma4(float w, float4 m, float4& acc) {
  acc.x = fmaf(w, m.x, acc.x);
  acc.y = fmaf(w, m.y, acc.y);
  acc.z = fmaf(w, m.z, acc.z);
  acc.w = fmaf(w, m.w, acc.w);
}

// Sum over the row groups of a wavefront: lanes with the same place in their group
// (lane mod LPR).  A butterfly: every lane ends with the same bits.
template <int LPR>
__device__ __forceinline__ float wave_groups_sum(float x) {
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}
template <int LPR>
__device__ __forceinline__ float4 wave_groups_sum4(float4 v) {
  return make_float4(wave_groups_sum<LPR>(v.x), wave_groups_sum<LPR>(v.y),
                     wave_groups_sum<LPR>(v.z), wave_groups_sum<LPR>(v.w));
}
// Sum over the LPR lanes of one row slice (xor butterfly within the group).
template <int LPR>
__device__ __forceinline__ float slice_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, LPR);
  return x;
}
// The column sums of every row group: each wavefront's, then the four in order.
// Callers put a barrier between two uses of one `red`.
template <int LPR>
__device__ __forceinline__ float4 block_groups_sum(float4 v, float4 (*red)[LPR], int lane,
                                                   int wv, int li) {
  v = wave_groups_sum4<LPR>(v);
  if (lane < LPR) red[wv][li] = v;
  __syncthreads();
  float4 s = red[0][li];
#pragma unroll
  for (int q = 1; q < kNW; ++q) {
    const float4 o = red[q][li];
    s.x += o.x;
    s.y += o.y;
    s.z += o.z;
    s.w += o.w;
  }
  return s;
}

// A barrier that orders this workgroup's LDS accesses only: global loads and stores
// still in flight stay in flight (a full __syncthreads() orders them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// block_groups_sum in two halves, so that other work can go between them: each
// wavefront's sums into `red`, then (after a barrier) the four in order.
template <int LPR>
__device__ __forceinline__ void groups_put(float4 v, float4 (*red)[LPR], int lane, int wv, int li) {
  v = wave_groups_sum4<LPR>(v);
  if (lane < LPR) red[wv][li] = v;
}
template <int LPR>
__device__ __forceinline__ float4 groups_take(float4 (*red)[LPR], int li) {
  float4 s = red[0][li];
#pragma unroll
  for (int q = 1; q < kNW; ++q) {
    const float4 o = red[q][li];
    s.x += o.x;
    s.y += o.y;
    s.z += o.z;
    s.w += o.w;
  }
  return s;
}

// Forward walk of one (walk, slice): SW columns, LPR = SW/4 lanes per row (a float4
// each), G = 256/LPR row groups; group g takes rows g, g + G, ... of a token's write
// and read sets.  NORM (one slice per walk): RMSNorm and gate in the kernel.
// LOG: the training forward's fp32 log of the rows each write replaces.
template <int SW, bool BF, bool LOG, bool NORM>
__global__ __launch_bounds__(256) void gdn_slice_kernel(SliceArgs A) {
  constexpr uint32_t ES = StateT<BF>::ES;
  constexpr int LPR = SW / 4;
  constexpr int G = 256 / LPR;
  constexpr int RPG = (128 + G - 1) / G;  // rows per group for W, R up to 128
  __shared__ float4 redp[kNW][LPR];
  __shared__ float4 redy[kNW][LPR];
  const ScanArgs& a = A.s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int64_t bh = blockIdx.x / A.S;
  const int sl = (int)(blockIdx.x - bh * A.S);
  const int64_t b = bh / a.H;
  const int h = (int)(bh - b * a.H);
  const int DV = a.d_v;
  const int c0 = sl * SW + li * 4;  // this lane's first column
  char* const Mb = static_cast<char*>(a.state) + (bh * (int64_t)a.N * DV + c0) * ES;
  auto row = [&](int64_t r) { return Mb + r * (DV * ES); };
  auto tok_of = [&](int64_t t) { return (b * a.T + t) * a.H + h; };

  float4 gam = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  if (NORM && a.norm_w) gam = *reinterpret_cast<const float4*>(a.norm_w + (int64_t)h * DV + c0);

  float4 mw[RPG];  // this group's rows of the current token's write set
  {
    const int32_t* iw = a.idx_w + tok_of(A.t0) * a.W;
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.W) mw[j] = state_load<BF>(row(iw[k]));
    }
  }
  for (int64_t t = A.t0; t < A.t1; ++t) {
    const int64_t tok = tok_of(t);
    const float al = a.alpha[tok];
    const float be = a.beta[tok];
    const int32_t* iw = a.idx_w + tok * a.W;
    const float* ww = a.wt_w + tok * a.W;
    const int32_t* ir = a.idx_r + tok * a.R;
    const float* wr = a.wt_r + tok * a.R;
    const float4 vv = *reinterpret_cast<const float4*>(a.v + tok * DV + c0);
    // key-weighted prediction from the rows before this token's writes
    float4 part = f4z();
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.W) fma4(ww[k], mw[j], part);
    }
    const float4 pred = block_groups_sum<LPR>(part, redp, lane, wv, li);
    const float4 err = make_float4(vv.x - al * pred.x, vv.y - al * pred.y, vv.z - al * pred.z,
                                   vv.w - al * pred.w);
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.W) {
        const float c = be * ww[k];
        if constexpr (LOG)
          *reinterpret_cast<float4*>(
              A.log + (((b * A.log_T + t - A.log_t0) * a.H + h) * a.W + k) * DV + c0) = mw[j];
        float4 m = mw[j];
        m.x = fmaf(c, err.x, al * m.x);
        m.y = fmaf(c, err.y, al * m.y);
        m.z = fmaf(c, err.z, al * m.z);
        m.w = fmaf(c, err.w, al * m.w);
        state_store<BF>(reinterpret_cast<uint64_t>(row(iw[k])), state_round<BF>(m));
      }
    }
    __syncthreads();  // this token's rows are written before anyone reloads them
    // the read set, and the next token's write set, both after this token's writes
    float4 mr[RPG];
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.R) mr[j] = state_load<BF>(row(ir[k]));
    }
    if (t + 1 < A.t1) {
      const int32_t* iwn = a.idx_w + tok_of(t + 1) * a.W;
#pragma unroll
      for (int j = 0; j < RPG; ++j) {
        const int k = grp + j * G;
        if (k < a.W) mw[j] = state_load<BF>(row(iwn[k]));
      }
    }
    float4 acc = f4z();
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.R) fma4(wr[k], mr[j], acc);
    }
    const float4 y = block_groups_sum<LPR>(acc, redy, lane, wv, li);
    if (tid < LPR) {  // the first row group of wavefront 0 stores the slice
      if constexpr (NORM) {
        const float ss = slice_sum<LPR>(dot4(y, y));
        const float rn = rsqrtf(ss / (float)DV + a.eps);
        const float4 gt = *reinterpret_cast<const float4*>(a.gate + tok * DV + c0);
        *reinterpret_cast<float4*>(a.out + tok * DV + c0) =
            make_float4(y.x * rn * gam.x * gt.x, y.y * rn * gam.y * gt.y,
                        y.z * rn * gam.z * gt.z, y.w * rn * gam.w * gt.w);
        if (a.y_raw) *reinterpret_cast<float4*>(a.y_raw + tok * DV + c0) = y;
      } else {
        *reinterpret_cast<float4*>(A.y + tok * DV + c0) = y;
      }
    }
  }
}

// Whether id is in the ascending list s[0..n) (LDS, 1 <= n <= 128): a binary search
// of fixed length whose reads are unconditional (no branch for the wait-count pass to
// join loads in flight across).
__device__ __forceinline__ bool in_sorted(const int32_t* s, int n, int32_t id) {
  int pos = 0;  // count of entries below id
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int q = pos + step;
    const bool below = s[min(q, n) - 1] < id;
    pos = (q <= n && below) ? q : pos;
  }
  return s[min(pos, n - 1)] == id;
}

// Reverse walk of one (walk, slice); layout as the forward.  Per token, the rows of
// the write phase that the token does not also read are loaded together with the
// read phase's rows and the logged rows (one round trip); the few it does read (a
// search of its read ids, staged in LDS) are reloaded after the read phase's
// barrier.  The previous token's small operands are loaded one token ahead.  Loads
// of padding entries (k beyond W or R) are clamped to a real entry and discarded,
// so the batch is straight-line code and its loads retire in order.
template <int SW, int FMT>
__global__ __launch_bounds__(256) void gdn_slice_backward_kernel(SliceBackArgs A) {
  constexpr int LPR = SW / 4;
  constexpr int G = 256 / LPR;
  constexpr int RPG = (128 + G - 1) / G;
  __shared__ float4 red1[kNW][LPR];
  __shared__ float4 red2[kNW][LPR];
  __shared__ float rda[kNW];
  __shared__ int32_t rid[128];  // this token's read ids
  const ScanBackArgs& a = A.s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int64_t bh = blockIdx.x / A.S;
  const int sl = (int)(blockIdx.x - bh * A.S);
  const int64_t b = bh / a.H;
  const int h = (int)(bh - b * a.H);
  const int DV = a.d_v;
  const int c0 = sl * SW + li * 4;
  const int q0 = sl * LPR + li;  // this lane's float4 of a row
  float* const M = a.state + bh * (int64_t)a.N * DV + c0;
  float* const dM = a.d_state + bh * (int64_t)a.N * DV + c0;
  auto ld = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
  auto st = [](float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; };
  auto kw_of = [&](int j) { return min(grp + j * G, a.W - 1); };  // clamped entries
  auto kr_of = [&](int j) { return min(grp + j * G, a.R - 1); };

  struct Ops {
    float4 dy, vv;
    float al, be;
    float ww[RPG], wr[RPG];
    int32_t iw[RPG], ir[RPG];
    int32_t rfull;  // read id number tid (staging)
  };
  auto load_ops = [&](int64_t t, Ops& o) {
    const int64_t tok = (b * a.T + t) * a.H + h;
    o.dy = ld(A.dy + tok * DV + c0);
    o.vv = ld(a.v + tok * DV + c0);
    o.al = a.alpha[tok];
    o.be = a.beta[tok];
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      o.ww[j] = a.wt_w[tok * a.W + kw_of(j)];
      o.iw[j] = a.idx_w[tok * a.W + kw_of(j)];
      o.wr[j] = a.wt_r[tok * a.R + kr_of(j)];
      o.ir[j] = a.idx_r[tok * a.R + kr_of(j)];
    }
    o.rfull = a.idx_r[tok * a.R + min(tid, a.R - 1)];
  };

  Ops op;
  load_ops(a.T - 1, op);
  for (int64_t t = a.T - 1; t >= 0; --t) {
    const int64_t tok = (b * a.T + t) * a.H + h;
    if (tid < a.R) rid[tid] = op.rfull;
    __syncthreads();  // read ids staged; the previous token's restores precede the loads
    // ---- one batch: logged rows, the read rows, the write rows' gradients ----
    float4 ms[RPG], m[RPG], g[RPG], gs[RPG];
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      ms[j] = log_load(a.log, a.log_scale, FMT, tok * a.W + kw_of(j), DV, q0);
      const int64_t r = (int64_t)op.ir[j] * DV;
      m[j] = ld(M + r);
      g[j] = ld(dM + r);
    }
    uint32_t late = 0;  // write rows this token also reads: their dM after the read phase
#pragma unroll
    for (int j = 0; j < RPG; ++j)
      late |= (uint32_t)in_sorted(rid, a.R, op.iw[j]) << j;
#pragma unroll
    for (int j = 0; j < RPG; ++j) gs[j] = ld(dM + (int64_t)op.iw[j] * DV);
    Ops on;
    load_ops(t > 0 ? t - 1 : t, on);
    // the read rows are used here, whatever entries are real: their loads stay in this
    // batch (the compiler would otherwise sink some into the branches that store)
#pragma unroll
    for (int j = 0; j < RPG; ++j)
      asm volatile("" ::"v"(m[j].x), "v"(m[j].y), "v"(m[j].z), "v"(m[j].w), "v"(g[j].x),
                   "v"(g[j].y), "v"(g[j].z), "v"(g[j].w));
    // ---- read (the state after token t's writes) ----
    // (every entry computes, padding ones included, so that no load is sunk into a
    // branch; only real entries store)
    float dq[RPG];
    float4 nr[RPG];
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      dq[j] = slice_sum<LPR>(dot4(op.dy, m[j]));
      nr[j] = g[j];
      fma4(op.wr[j], op.dy, nr[j]);
    }
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      if (k < a.R) {
        if (li == 0) A.pr[(sl * A.rows + tok) * a.R + k] = dq[j];
        st(dM + (int64_t)op.ir[j] * DV, nr[j]);
      }
    }
    __syncthreads();  // the write phase may take rows this phase updated
    // ---- write, undone ----
#pragma unroll
    for (int j = 0; j < RPG; ++j)
      if (((late >> j) & 1u) && grp + j * G < a.W) gs[j] = ld(dM + (int64_t)op.iw[j] * DV);
    float4 pk = f4z(), sg = f4z();
    float kwj[RPG];  // the write weights, 0 for padding entries
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      kwj[j] = grp + j * G < a.W ? op.ww[j] : 0.0f;
      fma4(kwj[j], ms[j], pk);
      fma4(kwj[j], gs[j], sg);
    }
    groups_put<LPR>(pk, red1, lane, wv, li);
    groups_put<LPR>(sg, red2, lane, wv, li);
    lds_barrier();
    pk = groups_take<LPR>(red1, li);  // sum k m
    sg = groups_take<LPR>(red2, li);  // sum k G
    const float al = op.al, be = op.be;
    const float4 e = make_float4(op.vv.x - al * pk.x, op.vv.y - al * pk.y, op.vv.z - al * pk.z,
                                 op.vv.w - al * pk.w);
    const float4 de = make_float4(be * sg.x, be * sg.y, be * sg.z, be * sg.w);
    if (tid < LPR) st(a.g_v + tok * DV + c0, de);
    float da = 0.0f;
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
      const int k = grp + j * G;
      const bool real = k < a.W;
      const float kw = kwj[j];
      const float4 mm = ms[j], gg = gs[j];
      const float4 dmt = make_float4(gg.x - kw * de.x, gg.y - kw * de.y, gg.z - kw * de.z,
                                     gg.w - kw * de.w);
      const float ge = slice_sum<LPR>(dot4(gg, e));
      const float dem = slice_sum<LPR>(dot4(de, mm));
      const float dj = slice_sum<LPR>(dot4(dmt, mm));
      da += real ? dj : 0.0f;
      if (real) {
        if (li == 0) A.pw[(sl * A.rows + tok) * a.W + k] = make_float2(ge, dem);
        const int64_t r = (int64_t)op.iw[j] * DV;
        st(dM + r, make_float4(al * dmt.x, al * dmt.y, al * dmt.z, al * dmt.w));
        st(M + r, mm);
      }
    }
    da = wave_groups_sum<LPR>(da);  // every lane of a group holds its group's sum
    if (lane == 0) rda[wv] = da;
    lds_barrier();
    if (tid == 0) A.pa[sl * A.rows + tok] = (rda[0] + rda[1]) + (rda[2] + rda[3]);
    op = on;
  }
}

// Per token: the slices' shares summed in slice order.
__global__ __launch_bounds__(256) void gdn_slice_reduce_kernel(SliceBackArgs A) {
  const ScanBackArgs& a = A.s;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= A.rows) return;
  for (int k = lane; k < a.R; k += 64) {
    float s = 0.0f;
    for (int q = 0; q < A.S; ++q) s += A.pr[(q * A.rows + tok) * a.R + k];
    a.g_wt_r[tok * a.R + k] = s;
  }
  const float al = a.alpha[tok], be = a.beta[tok];
  float db = 0.0f;
  for (int k = lane; k < a.W; k += 64) {
    float ge = 0.0f, dem = 0.0f;
    for (int q = 0; q < A.S; ++q) {
      const float2 p = A.pw[(q * A.rows + tok) * a.W + k];
      ge += p.x;
      dem += p.y;
    }
    a.g_wt_w[tok * a.W + k] = be * ge - al * dem;
    db = fmaf(a.wt_w[tok * a.W + k], ge, db);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) db += __shfl_xor(db, off);
  if (lane == 0) {
    float da = 0.0f;
    for (int q = 0; q < A.S; ++q) da += A.pa[q * A.rows + tok];
    a.g_alpha[tok] = da;
    a.g_beta[tok] = db;
  }
}

template <int SW>
void launch_back_sw(const SliceBackArgs& A, dim3 grid, hipStream_t s) {
  if (A.s.log_fmt == LOG_FP8)
    hipLaunchKernelGGL((gdn_slice_backward_kernel<SW, LOG_FP8>), grid, dim3(256), 0, s, A);
  else if (A.s.log_fmt == LOG_INT4)
    hipLaunchKernelGGL((gdn_slice_backward_kernel<SW, LOG_INT4>), grid, dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL((gdn_slice_backward_kernel<SW, LOG_F32>), grid, dim3(256), 0, s, A);
}

template <int SW>
void launch_fwd_sw(const SliceArgs& A, dim3 grid, bool norm, hipStream_t s) {
  const ScanArgs& a = A.s;
  const bool log = A.log != nullptr;
  if (a.state_bf16 && norm)
    hipLaunchKernelGGL((gdn_slice_kernel<SW, true, false, true>), grid, dim3(256), 0, s, A);
  else if (a.state_bf16)
    hipLaunchKernelGGL((gdn_slice_kernel<SW, true, false, false>), grid, dim3(256), 0, s, A);
  else if (log && norm)
    hipLaunchKernelGGL((gdn_slice_kernel<SW, false, true, true>), grid, dim3(256), 0, s, A);
  else if (log)
    hipLaunchKernelGGL((gdn_slice_kernel<SW, false, true, false>), grid, dim3(256), 0, s, A);
  else if (norm)
    hipLaunchKernelGGL((gdn_slice_kernel<SW, false, false, true>), grid, dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL((gdn_slice_kernel<SW, false, false, false>), grid, dim3(256), 0, s, A);
}

auto al256 = [](size_t x) { return (x + 255) & ~(size_t)255; };

// Tokens per launch of a training forward whose quantised log is staged in fp32.
int64_t stage_tokens(const sdm_dims& d) {
  const int64_t per_tok = d.B * (int64_t)d.H * d.W * d.d_v * 4;
  int64_t tc = kStageBytes / per_tok;
  tc = tc < 1 ? 1 : tc;
  return d.T < tc ? d.T : tc;
}

}  // namespace

// Slices per walk: powers of two until the grid reaches 256 workgroups, slices of
// at least 16 columns, at most SDM_GDN_MAX_SW.
int gdn_slices(const sdm_dims& d) {
  const int64_t walks = d.B * (int64_t)d.H;
  int S = 1;
  while (d.d_v / (2 * S) >= 16 && walks * S < 256) S *= 2;
  while (d.d_v / S > SDM_GDN_MAX_SW) S *= 2;
  return S;
}

// Inference over several slices: the raw read vectors for the norm pass (when the
// caller keeps none).  Training (the caller's y_raw is required): the fp32 staging
// of a token chunk's rows when the log is quantised.
size_t gdn_slice_workspace_bytes(const sdm_dims& d, bool train) {
  if (train)
    return (d.flags & (SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4))
               ? al256((size_t)d.B * stage_tokens(d) * d.H * d.W * d.d_v * 4)
               : 0;
  return gdn_slices(d) > 1 ? al256((size_t)d.B * d.T * d.H * d.d_v * 4) : 0;
}

hipError_t launch_gdn_slices(const sdm_dims& d, const ScanArgs& a, void* ws, hipStream_t st) {
  const int S = gdn_slices(d);
  const int SW = a.d_v / S;
  const bool norm = S == 1;
  const bool qlog = a.log && a.log_fmt != LOG_F32;
  if (a.log && a.state_bf16) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  SliceArgs A;
  A.s = a;
  A.S = S;
  A.y = a.y_raw ? a.y_raw : reinterpret_cast<float*>(base);  // training: y_raw given
  float* stage = qlog ? reinterpret_cast<float*>(base) : nullptr;
  const int64_t tc = qlog ? stage_tokens(d) : a.T;
  const dim3 grid((unsigned)(a.B * a.H * S));
  for (int64_t t0 = 0; t0 < a.T; t0 += tc) {
    A.t0 = t0;
    A.t1 = a.T - t0 < tc ? a.T : t0 + tc;
    A.log = qlog ? stage : static_cast<float*>(a.log);
    A.log_T = qlog ? A.t1 - t0 : a.T;
    A.log_t0 = qlog ? t0 : 0;
    {
      KernelTimer kt("gdn_slices", st);
      switch (SW) {
        case 16: launch_fwd_sw<16>(A, grid, norm, st); break;
        case 32: launch_fwd_sw<32>(A, grid, norm, st); break;
#if SDM_GDN_MAX_SW >= 64
        case 64: launch_fwd_sw<64>(A, grid, norm, st); break;
#endif
#if SDM_GDN_MAX_SW >= 128
        case 128: launch_fwd_sw<128>(A, grid, norm, st); break;
#endif
        default: return hipErrorInvalidValue;
      }
    }
    if (qlog) {
      const hipError_t e = launch_log_quantize(a, stage, t0, A.t1 - t0, st);
      if (e != hipSuccess) return e;
    }
  }
  if (!norm) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_norm_gate(a, A.y, st);
  }
  return hipGetLastError();
}

namespace {
struct SliceBackLayout {
  size_t gpart, dy, pr, pw, pa, total;
};
SliceBackLayout slice_back_layout(const sdm_dims& d) {
  const size_t rows = (size_t)d.B * d.T * d.H;
  const size_t S = (size_t)gdn_slices(d);
  SliceBackLayout L;
  size_t s = 0;
  L.gpart = s;
  s += al256((size_t)d.B * d.H * norm_backward_blocks(d.T) * d.d_v * 4);
  L.dy = s;
  s += al256(rows * d.d_v * 4);
  L.pr = s;
  s += al256(S * rows * d.R * 4);
  L.pw = s;
  s += al256(S * rows * d.W * 8);
  L.pa = s;
  s += al256(S * rows * 4);
  L.total = s;
  return L;
}
}  // namespace

size_t gdn_slice_backward_workspace_bytes(const sdm_dims& d) { return slice_back_layout(d).total; }

hipError_t launch_gdn_slice_backward(const sdm_dims& d, const ScanBackArgs& a, float* d_norm_w,
                                     void* ws, hipStream_t st) {
  const SliceBackLayout L = slice_back_layout(d);
  char* base = static_cast<char*>(ws);
  const int S = gdn_slices(d);
  SliceBackArgs A;
  A.s = a;
  A.S = S;
  A.rows = a.B * a.T * a.H;
  float* gpart = reinterpret_cast<float*>(base + L.gpart);
  float* dy = reinterpret_cast<float*>(base + L.dy);
  A.dy = dy;
  A.pr = reinterpret_cast<float*>(base + L.pr);
  A.pw = reinterpret_cast<float2*>(base + L.pw);
  A.pa = reinterpret_cast<float*>(base + L.pa);
  hipError_t e = launch_norm_backward(a, dy, gpart, st);
  if (e != hipSuccess) return e;
  {
    const dim3 grid((unsigned)(a.B * a.H * S));
    KernelTimer kt("gdn_slices_backward", st);
    switch (a.d_v / S) {
      case 16: launch_back_sw<16>(A, grid, st); break;
      case 32: launch_back_sw<32>(A, grid, st); break;
#if SDM_GDN_MAX_SW >= 64
      case 64: launch_back_sw<64>(A, grid, st); break;
#endif
#if SDM_GDN_MAX_SW >= 128
      case 128: launch_back_sw<128>(A, grid, st); break;
#endif
      default: return hipErrorInvalidValue;
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_gdn_back_reduce(a, A.pr, A.pw, A.pa, S, st)) != hipSuccess) return e;
  if (d_norm_w) return launch_gamma_blocks(a, gpart, d_norm_w, st);
  return hipSuccess;
}

hipError_t launch_gdn_back_reduce(const ScanBackArgs& a, float* pr, float2* pw, float* pa, int S,
                                  hipStream_t st) {
  SliceBackArgs A;
  A.s = a;
  A.dy = nullptr;
  A.pr = pr;
  A.pw = pw;
  A.pa = pa;
  A.rows = a.B * a.T * a.H;
  A.S = S;
  KernelTimer kt("gdn_back_reduce", st);
  hipLaunchKernelGGL(gdn_slice_reduce_kernel, dim3((unsigned)((A.rows + 3) / 4)), dim3(256), 0, st,
                     A);
  return hipGetLastError();
}

}  // namespace sdm
