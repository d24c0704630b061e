// Recurrent sparse scan for long token runs: slot-owner lane groups.
// State rows are fp32, or bf16 with fp32 arithmetic (SDM_FLAG_STATE_BF16).
//
// What is computed is the recurrence of the method ("Sparse Delta Memory" summary
// on paper.rainbus.top, method paragraph, steps 2-3; ai-paper-analysis.pages.dev,
// sections "步骤 2" and "步骤 3"): per (batch, head) memory and tokens in order,
//   write slot i (weight k):  M[i] <- (1 - c)(alpha_t M[i]) + c v_t,  c = beta_t k
//   read:                     y_t = sum_i q^(i) M[i]   (after the token's writes)
// with unselected slots never touched.
//
// How it is scheduled on gfx950:
//  * Every slot belongs to exactly one lane group (hash of the slot id).  A lane
//    group is LPG lanes covering one SW-float segment of d_v (one float4 each).
//    The lane groups of a walk are split over `parts` workgroups, so that a few
//    dozen walks still put one workgroup on every CU.
//  * A bucketing pre-pass lays the accesses of each walk out as per-group streams
//    in token order (writes before reads within a token), split into rounds of
//    ROUND tokens.  Because a slot's column chunk is only ever loaded and stored by
//    one thread, program order alone orders every read-after-write and
//    write-after-write on that address: no cross-wave synchronisation is needed
//    for the state.
//  * Each lane group keeps BQ row loads in flight; repeated slots inside a batch
//    are forwarded in registers.
//  * Two schedules of the reads:
//      stream:    every read sits in its owner's stream and adds q * M[i] into an
//                 LDS ring of per-token partial sums (float atomics);
//      two-phase: only reads whose slot a later token of the round rewrites stay in
//                 the owner streams; all others are summed per token in registers
//                 once the round's writes are done (see two_phase_scan_kernel).
//    Each part writes its own partial read vectors; a small kernel sums the parts,
//    normalises and gates.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int ROUND = kStreamRound;  // tokens per round (ring half)
// two-phase training forward: accesses in flight per lane group (32- / 16-float slices;
// 8 spills registers at 16)
constexpr int BQ_TRAIN32 = 8, BQ_TRAIN16 = 6;
constexpr int MAX_GT = kStreamMaxGT;  // lane groups per walk
constexpr uint32_t SLOT_MASK = 0xFFFFFFu;
static_assert(ROUND <= 256, "token-in-round must fit the entry's top 8 bits");

// Owner-stream entry: slot ids < 2^24 (at most 1024^2 here) share a word with the
// token's place in its round; softmax weights are >= 0, so their sign bit is free
// for the read flag.
__device__ __forceinline__ uint2 make_entry(uint32_t slot, int tt, float q, bool read) {
  return make_uint2(slot | ((uint32_t)tt << 24), __float_as_uint(q) | (read ? 0x80000000u : 0u));
}

__device__ __forceinline__ uint32_t group_of(uint32_t slot, int log2gt) {
  return (slot * 2654435761u) >> (32 - log2gt);
}

// ---------------------------------------------------------------------------
// Pre-pass 1: per (walk, round) histogram of accesses per group.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bucket_count_kernel(StreamArgs a) {
  __shared__ int cnt[MAX_GT];
  const int64_t w = blockIdx.x / a.rounds;
  const int r = (int)(blockIdx.x - w * a.rounds);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  for (int g = threadIdx.x; g < a.GT; g += 256) cnt[g] = 0;
  __syncthreads();
  const int64_t t_lo = (int64_t)r * ROUND;
  const int nt = (int)min<int64_t>(ROUND, a.Tc - t_lo);
  const int per = a.W + a.R;
  const int n = nt * per;  // at most 256 x 256 accesses: 32-bit indexing
  const int64_t tok0 = (b * a.T + a.t0 + t_lo) * a.H + h;
  constexpr int U = 4;  // ids loaded per thread before their atomics
  for (int e0 = threadIdx.x; e0 < n; e0 += 256 * U) {
    uint32_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(e0 + u * 256, n - 1);
      const int t = e / per, k = e - t * per;
      const int64_t tok = tok0 + (int64_t)t * a.H;
      s[u] = (uint32_t)(k < a.W ? a.idx_w[tok * a.W + k] : a.idx_r[tok * a.R + (k - a.W)]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (e0 + u * 256 < n) atomicAdd(&cnt[group_of(s[u], a.log2GT)], 1);
  }
  __syncthreads();
  int* out = a.counts + ((int64_t)w * a.rounds + r) * a.GT;
  for (int g = threadIdx.x; g < a.GT; g += 256) out[g] = cnt[g];
}

// ---------------------------------------------------------------------------
// Pre-pass 2: per walk, stream offsets of every (group, round), groups laid out
// one after another.  offsets[w][g][r] for r in [0, rounds] (last = group end).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bucket_offsets_kernel(StreamArgs a) {
  __shared__ int tot[MAX_GT];
  __shared__ int part[1024];
  const int64_t w = blockIdx.x;
  const int tid = threadIdx.x;
  const int* cnt = a.counts + (int64_t)w * a.rounds * a.GT;
  for (int g = tid; g < a.GT; g += 1024) {
    int acc = 0;
    for (int r = 0; r < a.rounds; ++r) acc += cnt[(int64_t)r * a.GT + g];
    tot[g] = acc;
  }
  __syncthreads();
  // exclusive prefix over groups: each thread owns a contiguous run
  const int per = (a.GT + 1023) / 1024;
  int run = 0;
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g < a.GT) run += tot[g];
  }
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - run;  // exclusive
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g < a.GT) {
      const int t = tot[g];
      tot[g] = base;
      base += t;
    }
  }
  __syncthreads();
  for (int g = tid; g < a.GT; g += 1024) {
    int acc = tot[g];
    int* o = a.offsets + ((int64_t)w * a.GT + g) * (a.rounds + 1);
    for (int r = 0; r < a.rounds; ++r) {
      o[r] = acc;
      acc += cnt[(int64_t)r * a.GT + g];
    }
    o[a.rounds] = acc;
  }
}

// Pre-pass 2 for walks with many groups x rounds (few long walks: one workgroup per
// walk would sum them alone): the same offsets from two kernels over blocks of 256
// groups.  2a: each thread sums one group's counts over the rounds.  2b: each block
// adds up the totals of the walk's earlier groups, scans its own 256, and writes its
// groups' running sums over the rounds.  Integer sums: the result is the one above.
__global__ __launch_bounds__(256) void bucket_totals_kernel(StreamArgs a) {
  const int nb = (a.GT + 255) / 256;
  const int64_t w = blockIdx.x / nb;
  const int g = (int)(blockIdx.x - w * nb) * 256 + (int)threadIdx.x;
  if (g >= a.GT) return;
  const int* cnt = a.counts + (int64_t)w * a.rounds * a.GT + g;
  int acc = 0;
  for (int r = 0; r < a.rounds; ++r) acc += cnt[(int64_t)r * a.GT];
  a.totals[(int64_t)w * a.GT + g] = acc;
}

__global__ __launch_bounds__(256) void bucket_offsets_wide_kernel(StreamArgs a) {
  __shared__ int sh[256];
  const int nb = (a.GT + 255) / 256;
  const int64_t w = blockIdx.x / nb;
  const int g0 = (int)(blockIdx.x - w * nb) * 256;
  const int tid = threadIdx.x;
  const int* tot = a.totals + (int64_t)w * a.GT;
  // totals of the walk's groups before this block
  int before = 0;
  for (int g = tid; g < g0; g += 256) before += tot[g];
  sh[tid] = before;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  const int base0 = sh[0];
  __syncthreads();
  // exclusive prefix of this block's totals
  const int g = g0 + tid;
  const int mine = g < a.GT ? tot[g] : 0;
  sh[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  if (g >= a.GT) return;
  int acc = base0 + sh[tid] - mine;
  const int* cnt = a.counts + (int64_t)w * a.rounds * a.GT + g;
  int* o = a.offsets + ((int64_t)w * a.GT + g) * (a.rounds + 1);
  for (int r = 0; r < a.rounds; ++r) {
    o[r] = acc;
    acc += cnt[(int64_t)r * a.GT];
  }
  o[a.rounds] = acc;
}

// Offsets pass: one workgroup per walk, or the two-kernel form when a walk has many
// groups x rounds.
hipError_t launch_offsets(const StreamArgs& a, int64_t walks, hipStream_t st) {
  if ((int64_t)a.GT * a.rounds <= 65536) {
    KernelTimer kt("bucket_offsets", st);
    hipLaunchKernelGGL(bucket_offsets_kernel, dim3((unsigned)walks), dim3(1024), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(walks * ((a.GT + 255) / 256)));
  {
    KernelTimer kt("bucket_totals", st);
    hipLaunchKernelGGL(bucket_totals_kernel, grid, dim3(256), 0, st, a);
  }
  KernelTimer kt("bucket_offsets", st);
  hipLaunchKernelGGL(bucket_offsets_wide_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pre-pass 3: scatter the accesses of one (walk, round) into the streams.  One
// wavefront walks the round's tokens in order; LDS cursors hand out positions.
// Within one instruction all slots are distinct (a token's write ids are distinct,
// and so are its read ids), and writes are issued before reads, so accesses of
// one slot keep token order with writes first.  TRAIN: the entry's second word
// holds the access's position in the token's id list instead of its weight.
// ---------------------------------------------------------------------------
template <bool TRAIN>
__global__ __launch_bounds__(64) void bucket_scatter_kernel(StreamArgs a) {
  constexpr int D = 4;   // tokens whose ids are loaded ahead of their placement
  constexpr int KC = 2;  // 64-wide chunks of W and R (up to 128)
  __shared__ int cur[MAX_GT];
  const int64_t w = blockIdx.x / a.rounds;
  const int r = (int)(blockIdx.x - w * a.rounds);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int lane = threadIdx.x;
  for (int g = lane; g < a.GT; g += 64)
    cur[g] = a.offsets[((int64_t)w * a.GT + g) * (a.rounds + 1) + r];
  __syncthreads();
  uint2* ent = a.entries + w * a.walk_entries;
  const int64_t t_lo = (int64_t)r * ROUND;
  const int nt = (int)min<int64_t>(ROUND, a.Tc - t_lo);
  const int64_t tok0 = (b * a.T + a.t0 + t_lo) * a.H + h;  // token tt -> tok0 + tt*H
  // ids and entry words (weight bits, or the position) of the writes (x*) and reads
  // (r*) of D tokens
  uint32_t xs[D][KC], xq[D][KC], rs[D][KC], rq[D][KC];
  auto fetch = [&](int tb, uint32_t (&fs)[D][KC], uint32_t (&fq)[D][KC], uint32_t (&gs)[D][KC],
                   uint32_t (&gq)[D][KC]) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int64_t tok = tok0 + (int64_t)min(tb + u, nt - 1) * a.H;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int kw = min(c * 64 + lane, a.W - 1), kr = min(c * 64 + lane, a.R - 1);
        fs[u][c] = (uint32_t)a.idx_w[tok * a.W + kw];
        fq[u][c] = TRAIN ? (uint32_t)kw : __float_as_uint(a.wt_w[tok * a.W + kw]);
        gs[u][c] = (uint32_t)a.idx_r[tok * a.R + kr];
        gq[u][c] = TRAIN ? (uint32_t)kr : __float_as_uint(a.wt_r[tok * a.R + kr]);
      }
    }
  };
  fetch(0, xs, xq, rs, rq);
  for (int tb = 0; tb < nt; tb += D) {
    uint32_t ns[D][KC], nq[D][KC], ms[D][KC], mq[D][KC];
    fetch(tb + D, ns, nq, ms, mq);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int tt = tb + u;
      if (tt >= nt) break;
      // writes before reads: a slot's accesses keep token order, writes first
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (c * 64 + lane < a.W) {
          const int pos = atomicAdd(&cur[group_of(xs[u][c], a.log2GT)], 1);
          ent[pos] = make_entry(xs[u][c], tt, __uint_as_float(xq[u][c]), false);
        }
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (c * 64 + lane < a.R) {
          const int pos = atomicAdd(&cur[group_of(rs[u][c], a.log2GT)], 1);
          ent[pos] = make_entry(rs[u][c], tt, __uint_as_float(rq[u][c]), true);
        }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        xs[u][c] = ns[u][c];
        xq[u][c] = nq[u][c];
        rs[u][c] = ms[u][c];
        rq[u][c] = mq[u][c];
      }
  }
}

// ---------------------------------------------------------------------------
// The scan proper.  Workgroup = (walk, slice, part); NT threads; SW floats per
// slice; LPG = SW/4 lanes per group; GW = NT/LPG groups; batches of BQ accesses.
// Per round the slice of v and the gates of the round's tokens are staged in LDS,
// so a batch only holds its BQ state rows in registers while they are in flight.
// TRAIN (training forward, fp32 state): entries carry each access's position in its
// token's id list; the weight is loaded by (token, position), and every write also
// stores the row it replaces to the write log.
// ---------------------------------------------------------------------------
template <int NT, int SW, int BQ, bool BF, bool TRAIN>
__global__ __launch_bounds__(NT) void stream_scan_kernel(StreamArgs a) {
  static_assert(!(TRAIN && BF), "the write log is kept for fp32 state");
  constexpr uint32_t ES = StateT<BF>::ES;
  constexpr int LPG = SW / 4;
  constexpr int GW = NT / LPG;
  constexpr int EPL = (BQ + LPG - 1) / LPG;  // entries loaded per lane per batch
  // Read partial sums, one padded row of YS words per token.  Column 4*l + c of a
  // lane l sits at word c*LPG + l, so one atomic instruction's lanes of a group hit
  // consecutive banks, and the padding staggers the tokens' rows across banks.
  constexpr int YS = SW + 8;
  __shared__ __attribute__((aligned(16))) float yr[2 * ROUND * YS];
  __shared__ __attribute__((aligned(16))) float vs[ROUND * SW];      // v slice of the round
  __shared__ float2 gab[ROUND];                                      // (alpha, beta)

  const int tid = threadIdx.x;
  const int li = tid % LPG;
  const int g = tid / LPG;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % a.parts);
  const int64_t ws = wg / a.parts;
  const int sl = (int)(ws % a.S);
  const int64_t w = ws / a.S;
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int gg = p * GW + g;
  const int dv = a.d_v;

  for (int x = tid; x < 2 * ROUND * YS; x += NT) yr[x] = 0.0f;

  // state of this walk as a uniform base; rows addressed by 32-bit byte offsets
  char* Mb = static_cast<char*>(a.state) + w * (int64_t)a.N * dv * ES;
  const uint32_t col_bytes = (uint32_t)(sl * SW + li * 4) * ES;
  const uint32_t row_bytes = (uint32_t)dv * ES;
  const uint2* ent = a.entries + w * a.walk_entries;
  const int* offs = a.offsets + ((int64_t)w * a.GT + gg) * (a.rounds + 1);
  const int64_t tok_base = (b * a.T + a.t0) * a.H + h;  // token t -> tok_base + t*H
  const int64_t log_base = (b * a.log_T + a.log_t0) * a.H + h;  // TRAIN: log row of t
  float4* trash = a.trash + wg * NT + tid;

  for (int r = 0; r < a.rounds; ++r) {
    const int half = r & 1;
    const int64_t t_lo = (int64_t)r * ROUND;
    const int nt = (int)min<int64_t>(ROUND, a.Tc - t_lo);
    // stage v slice and gates of this round's tokens
    for (int x = tid; x < nt * LPG; x += NT) {
      const int tt = x / LPG, c4 = x % LPG;
      const int64_t tok = tok_base + (t_lo + tt) * a.H;
      *reinterpret_cast<float4*>(vs + tt * SW + c4 * 4) =
          *reinterpret_cast<const float4*>(a.v + tok * dv + sl * SW + c4 * 4);
    }
    for (int x = tid; x < nt; x += NT) {
      const int64_t tok = tok_base + (t_lo + x) * a.H;
      gab[x] = make_float2(a.alpha[tok], a.beta[tok]);
    }
    __syncthreads();

    const int beg = offs[r];
    const int end = offs[r + 1];
    uint2 e[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) e[q] = ent[max(min(beg + q * LPG + li, end - 1), 0)];
    // once per round: the first batch's entries are complete before the batch loop,
    // so the loop header carries no pending load
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int i = beg; i < end; i += BQ) {
      // next batch's entries travel with this batch's row loads
      uint2 en[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) en[q] = ent[min(i + BQ + q * LPG + li, end - 1)];
      uint32_t slot[BQ], tk[BQ];
      float wq[BQ];
      int kk[BQ];                 // TRAIN: position in the token's id list
      uint32_t wrm = 0, vam = 0;  // bit j: access j is a valid write / is valid
      float4 mv[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int src = j % LPG, q = j / LPG;
        const uint32_t ex = group_bcast<LPG>(e[q].x, src);
        const uint32_t ey = group_bcast<LPG>(e[q].y, src);
        slot[j] = min(ex & SLOT_MASK, (uint32_t)a.N - 1u);  // stays in bounds
        tk[j] = ex >> 24;                                   // token within the round
        if constexpr (TRAIN) {
          tk[j] = min(tk[j], (uint32_t)nt - 1u);
          kk[j] = min((int)(ey & 0x7fffffffu), ((ey >> 31) ? a.R : a.W) - 1);
          const int64_t tok = tok_base + (t_lo + tk[j]) * a.H;
          wq[j] = (ey >> 31) ? a.wt_r[tok * a.R + kk[j]] : a.wt_w[tok * a.W + kk[j]];
        } else {
          wq[j] = __uint_as_float(ey & 0x7fffffffu);
        }
        const bool valid = i + j < end;
        vam |= (uint32_t)valid << j;
        wrm |= (uint32_t)(valid && !(ey >> 31)) << j;
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j)
        mv[j] = state_load<BF>(Mb + (slot[j] * row_bytes + col_bytes));
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        float4 val = mv[j];
#pragma unroll
        for (int jj = 0; jj < j; ++jj) {
          const bool fwd = ((wrm >> jj) & 1u) && slot[jj] == slot[j];
          val.x = fwd ? mv[jj].x : val.x;
          val.y = fwd ? mv[jj].y : val.y;
          val.z = fwd ? mv[jj].z : val.z;
          val.w = fwd ? mv[jj].w : val.w;
        }
        const bool isw = (wrm >> j) & 1u;
        if constexpr (TRAIN) {
          if (isw) {
            const int64_t lr = log_base + (t_lo + tk[j]) * a.H;
            *reinterpret_cast<float4*>(a.log + (lr * a.W + kk[j]) * dv + sl * SW + li * 4) = val;
          }
        }
        {
          // every access stores once (the vector-memory counter then stays static);
          // accesses that do not write go to this lane's trash slot
          const float2 ab = gab[tk[j]];
          const float4 vv = *reinterpret_cast<const float4*>(vs + tk[j] * SW + li * 4);
          const float c = ab.y * wq[j];
          const float oc = 1.0f - c;
          float4 nv;
          nv.x = fmaf(c, vv.x, oc * (ab.x * val.x));
          nv.y = fmaf(c, vv.y, oc * (ab.x * val.y));
          nv.z = fmaf(c, vv.z, oc * (ab.x * val.z));
          nv.w = fmaf(c, vv.w, oc * (ab.x * val.w));
          val.x = isw ? nv.x : val.x;
          val.y = isw ? nv.y : val.y;
          val.z = isw ? nv.z : val.z;
          val.w = isw ? nv.w : val.w;
          val = state_round<BF>(val);  // the stored value (exact for non-writes)
          uint64_t dst = isw ? reinterpret_cast<uint64_t>(Mb + (slot[j] * row_bytes + col_bytes))
                             : reinterpret_cast<uint64_t>(trash);
          asm volatile("" : "+v"(dst));  // keep one unconditional store: hide the select
          state_store<BF>(dst, val);
        }
        if (!isw && ((vam >> j) & 1u)) {
          float* y = yr + (half * ROUND + tk[j]) * YS + li;
          atomicAdd(y + 0 * LPG, wq[j] * val.x);
          atomicAdd(y + 1 * LPG, wq[j] * val.y);
          atomicAdd(y + 2 * LPG, wq[j] * val.z);
          atomicAdd(y + 3 * LPG, wq[j] * val.w);
        }
        mv[j] = val;  // value after this access (forward source for later ones)
      }
#pragma unroll
      for (int q = 0; q < EPL; ++q) e[q] = en[q];
    }
    __syncthreads();
    // flush this round's partial read vectors and clear the ring half
    for (int x = tid; x < nt * LPG; x += NT) {
      const int tt = x / LPG, c4 = x % LPG;
      float* src = yr + (half * ROUND + tt) * YS + c4;
      const int64_t yi = ((((int64_t)p * a.B + b) * a.Tc + t_lo + tt) * a.H + h) * dv +
                         sl * SW + c4 * 4;
      *reinterpret_cast<float4*>(a.y_part + yi) =
          make_float4(src[0], src[LPG], src[2 * LPG], src[3 * LPG]);
      src[0] = 0.f;
      src[LPG] = 0.f;
      src[2 * LPG] = 0.f;
      src[3 * LPG] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Two-phase schedule, pre-pass 3: scatter one (walk, round) in REVERSE token order.
// An LDS bitmap over the N slots holds "written by a later token of this round".
// A read whose slot is in it is "dirty": it must be served by the slot's owner at
// its place in the stream (it sees a value that a later write of the round
// replaces).  Every other read is clean and is served after the round's writes by
// the read phase of the part that owns its slot.  The owner streams get the writes
// and the dirty reads only, packed at the end of each (group, round) segment;
// begins[] records where each packed segment starts.  Each token's clean reads are
// written grouped by owning part, cstart[] giving where each part's run begins.
// Positions are handed out downwards, so a slot's accesses keep token order with
// writes before reads.
// ---------------------------------------------------------------------------
// The token loop is latency-bound (one wavefront, one token at a time), so the ids
// and weights of the next D tokens are loaded while the current D are placed.
// KC = number of 64-wide chunks of W and R (1 or 2).  TRAIN: owner-stream entries
// carry the access's position in its token's id list instead of its weight (clean
// reads keep their weights).
template <int KC, int D, bool TRAIN>
__global__ __launch_bounds__(64) void bucket_scatter_rev_kernel(StreamArgs a) {
  extern __shared__ uint32_t dyn[];
  int* cur = reinterpret_cast<int*>(dyn);
  uint32_t* bm = dyn + a.GT;
  const int nbw = (a.N + 31) >> 5;
  const int64_t w = blockIdx.x / a.rounds;
  const int r = (int)(blockIdx.x - w * a.rounds);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int lane = threadIdx.x;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int g = lane; g < a.GT; g += 64)
    cur[g] = a.offsets[((int64_t)w * a.GT + g) * (a.rounds + 1) + r + 1];
  for (int i = lane; i < nbw; i += 64) bm[i] = 0u;
  __syncthreads();
  uint2* ent = a.entries + w * a.walk_entries;
  const int64_t t_lo = (int64_t)r * ROUND;
  const int64_t t_hi = min<int64_t>(a.Tc, t_lo + ROUND);
  const int64_t tok0 = (b * a.T + a.t0) * a.H + h;  // token t -> tok0 + t*H

  // ids / weight bits of the reads (r*) and writes (x*) of D tokens
  uint32_t rs[D][KC], rq[D][KC], xs[D][KC], xq[D][KC];
  auto fetch = [&](int64_t tb, uint32_t (&fs)[D][KC], uint32_t (&fq)[D][KC],
                   uint32_t (&gs)[D][KC], uint32_t (&gq)[D][KC]) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int64_t tok = tok0 + max<int64_t>(tb - u, t_lo) * a.H;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int kr = min(c * 64 + lane, a.R - 1), kw = min(c * 64 + lane, a.W - 1);
        fs[u][c] = (uint32_t)a.idx_r[tok * a.R + kr];
        fq[u][c] = __float_as_uint(a.wt_r[tok * a.R + kr]);
        gs[u][c] = (uint32_t)a.idx_w[tok * a.W + kw];
        gq[u][c] = __float_as_uint(a.wt_w[tok * a.W + kw]);
      }
    }
  };
  fetch(t_hi - 1, rs, rq, xs, xq);
  for (int64_t tb = t_hi - 1; tb >= t_lo; tb -= D) {
    uint32_t ns[D][KC], nq[D][KC], ms[D][KC], mq[D][KC];
    fetch(tb - D, ns, nq, ms, mq);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int64_t t = tb - u;
      if (t < t_lo) break;
      const int64_t ltok = (b * a.Tc + t) * a.H + h;  // chunk-local token row
      const int tt = (int)(t - t_lo);
      int pk[KC];  // owning part of a clean read, -1 otherwise
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const uint32_t sr = rs[u][c];
        pk[c] = -1;
        if (c * 64 + lane < a.R) {
          const uint32_t grp = group_of(sr, a.log2GT);
          if ((bm[sr >> 5] >> (sr & 31u)) & 1u) {
            const int pos = atomicSub(&cur[grp], 1) - 1;
            ent[pos] = make_entry(sr, tt,
                                  __uint_as_float(TRAIN ? (uint32_t)(c * 64 + lane) : rq[u][c]),
                                  true);
          } else {
            pk[c] = (int)(grp >> a.log2GW);
          }
        }
      }
      // clean reads grouped by owning part: a ballot per part gives every lane its
      // place, then one store per lane; lane p records where part p's run starts
      int* cs = a.cstart + ltok * (a.parts + 1);
      uint2* cl = a.clean + ltok * a.R;
      int base = 0, csv = 0;
      int cpos[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) cpos[c] = 0;
      for (int p = 0; p < a.parts; ++p) {  // parts < 64 (plan_stream)
        csv = lane == p ? base : csv;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bool mine = pk[c] == p;
          const unsigned long long m = __ballot(mine);
          cpos[c] = mine ? base + __popcll(m & below) : cpos[c];
          base += __popcll(m);
        }
      }
      csv = lane == a.parts ? base : csv;
      if (lane <= a.parts) cs[lane] = csv;
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (pk[c] >= 0) cl[cpos[c]] = make_uint2(rs[u][c], rq[u][c]);
      __syncthreads();
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c * 64 + lane < a.W) {
          const uint32_t sw = xs[u][c];
          const int pos = atomicSub(&cur[group_of(sw, a.log2GT)], 1) - 1;
          ent[pos] = make_entry(sw, tt,
                                __uint_as_float(TRAIN ? (uint32_t)(c * 64 + lane) : xq[u][c]),
                                false);
          atomicOr(&bm[sw >> 5], 1u << (sw & 31u));
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        rs[u][c] = ns[u][c];
        rq[u][c] = nq[u][c];
        xs[u][c] = ms[u][c];
        xq[u][c] = mq[u][c];
      }
  }
  for (int g = lane; g < a.GT; g += 64)
    a.begins[((int64_t)w * a.GT + g) * a.rounds + r] = cur[g];
}

// ---------------------------------------------------------------------------
// Two-phase scan.  Workgroup = (walk, slice, part); the part's lane groups own its
// share of the walk's slots.  Per round of ROUND tokens:
//   write phase: owners run their streams (writes and dirty reads) in batches of
//                BQ, dirty reads add q*M[i] into an LDS ring;
//   read phase:  each lane group takes whole tokens, loads the token's clean reads
//                of this part's slots BR rows at a time and sums them in registers,
//                adds the ring's dirty part and writes the part's y.  Barriers
//                separate the phases (the reads see the round's writes; the next
//                round's writes come after the reads).  Parts never touch each
//                other's slots, so they need no synchronisation with one another.
// ---------------------------------------------------------------------------
// F8: fp8 state (codes plane, then one exponent byte per 32-column block; SW >= 32).
template <int NT, int SW, int BQ, int BR, bool BF, bool TRAIN, bool F8 = false>
__global__ __launch_bounds__(NT) void two_phase_scan_kernel(StreamArgs a) {
  static_assert(!(TRAIN && BF), "the write log is kept for fp32 state");
  static_assert(!(F8 && (BF || TRAIN || SW < 32)), "fp8 state: inference, 32-column blocks");
  constexpr uint32_t ES = F8 ? 1u : StateT<BF>::ES;
  constexpr int LPG = SW / 4;
  constexpr int GW = NT / LPG;
  constexpr int EPL = (BQ + LPG - 1) / LPG;
  constexpr int RPL = (BR + LPG - 1) / LPG;  // clean reads loaded per lane per batch
  constexpr int YS = SW + 8;
  __shared__ __attribute__((aligned(16))) float yr[ROUND * YS];  // dirty-read sums
  __shared__ __attribute__((aligned(16))) float vs[ROUND * SW];  // v slice of the round
  __shared__ float2 gab[ROUND];                                  // (alpha, beta)

  const int tid = threadIdx.x;
  const int li = tid % LPG;
  const int g = tid / LPG;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % a.parts);
  const int64_t ws = wg / a.parts;
  const int sl = (int)(ws % a.S);
  const int64_t w = ws / a.S;
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int gg = p * GW + g;
  const int dv = a.d_v;

  for (int x = tid; x < ROUND * YS; x += NT) yr[x] = 0.0f;

  char* Mb = static_cast<char*>(a.state) + w * (int64_t)a.N * dv * ES;
  const uint32_t col_bytes = (uint32_t)(sl * SW + li * 4) * ES;
  const uint32_t row_bytes = (uint32_t)dv * ES;
  // F8: this lane's block exponent of row r at Eb + r * erow
  uint8_t* const Eb = F8 ? static_cast<uint8_t*>(a.state) + a.B * a.H * (int64_t)a.N * dv +
                               w * (int64_t)a.N * (dv / 32) + (sl * SW + li * 4) / 32
                         : nullptr;
  const uint32_t erow = (uint32_t)dv / 32;
  auto load_row = [&](uint32_t r) {
    if constexpr (F8)
      return fp8_decode4(*reinterpret_cast<const uint32_t*>(Mb + (r * row_bytes + col_bytes)),
                         Eb[r * erow]);
    else
      return state_load<BF>(Mb + (r * row_bytes + col_bytes));
  };
  const uint2* ent = a.entries + w * a.walk_entries;
  const int* offs = a.offsets + ((int64_t)w * a.GT + gg) * (a.rounds + 1);
  const int* begs = a.begins + ((int64_t)w * a.GT + gg) * a.rounds;
  const int64_t tok_base = (b * a.T + a.t0) * a.H + h;  // token t -> tok_base + t*H
  const int64_t log_base = (b * a.log_T + a.log_t0) * a.H + h;  // TRAIN: log row of t
  float* y_out = a.y_part + (int64_t)p * a.B * a.Tc * a.H * dv + sl * SW + li * 4;
  float4* trash = a.trash + wg * NT + tid;

  for (int r = 0; r < a.rounds; ++r) {
    const int64_t t_lo = (int64_t)r * ROUND;
    const int nt = (int)min<int64_t>(ROUND, a.Tc - t_lo);
    for (int x = tid; x < nt * LPG; x += NT) {
      const int tt = x / LPG, c4 = x % LPG;
      const int64_t tok = tok_base + (t_lo + tt) * a.H;
      *reinterpret_cast<float4*>(vs + tt * SW + c4 * 4) =
          *reinterpret_cast<const float4*>(a.v + tok * dv + sl * SW + c4 * 4);
    }
    for (int x = tid; x < nt; x += NT) {
      const int64_t tok = tok_base + (t_lo + x) * a.H;
      gab[x] = make_float2(a.alpha[tok], a.beta[tok]);
    }
    __syncthreads();

    // ---- write phase ----
    const int beg = begs[r];
    const int end = offs[r + 1];
    uint2 e[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) e[q] = ent[max(min(beg + q * LPG + li, end - 1), 0)];
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop header carries no pending load
    for (int i = beg; i < end; i += BQ) {
      uint2 en[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) en[q] = ent[min(i + BQ + q * LPG + li, end - 1)];
      uint32_t slot[BQ], tk[BQ];
      float wq[BQ];
      int kk[BQ];  // TRAIN: position in the token's id list
      uint32_t wrm = 0, vam = 0;
      float4 mv[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int src = j % LPG, q = j / LPG;
        const uint32_t ex = group_bcast<LPG>(e[q].x, src);
        const uint32_t ey = group_bcast<LPG>(e[q].y, src);
        slot[j] = min(ex & SLOT_MASK, (uint32_t)a.N - 1u);
        tk[j] = ex >> 24;
        if constexpr (TRAIN) {
          tk[j] = min(tk[j], (uint32_t)nt - 1u);
          kk[j] = min((int)(ey & 0x7fffffffu), ((ey >> 31) ? a.R : a.W) - 1);
          const int64_t tok = tok_base + (t_lo + tk[j]) * a.H;
          wq[j] = (ey >> 31) ? a.wt_r[tok * a.R + kk[j]] : a.wt_w[tok * a.W + kk[j]];
        } else {
          wq[j] = __uint_as_float(ey & 0x7fffffffu);
        }
        const bool valid = i + j < end;
        vam |= (uint32_t)valid << j;
        wrm |= (uint32_t)(valid && !(ey >> 31)) << j;
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) mv[j] = load_row(slot[j]);
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        float4 val = mv[j];
#pragma unroll
        for (int jj = 0; jj < j; ++jj) {
          const bool fwd = ((wrm >> jj) & 1u) && slot[jj] == slot[j];
          val.x = fwd ? mv[jj].x : val.x;
          val.y = fwd ? mv[jj].y : val.y;
          val.z = fwd ? mv[jj].z : val.z;
          val.w = fwd ? mv[jj].w : val.w;
        }
        const bool isw = (wrm >> j) & 1u;
        if constexpr (TRAIN) {  // the row as it was before this write, to the log
          if (isw) {
            const int64_t lr = log_base + (t_lo + tk[j]) * a.H;
            *reinterpret_cast<float4*>(a.log + (lr * a.W + kk[j]) * dv + sl * SW + li * 4) = val;
          }
        }
        {
          const float2 ab = gab[tk[j]];
          const float4 vv = *reinterpret_cast<const float4*>(vs + tk[j] * SW + li * 4);
          const float c = ab.y * wq[j];
          const float oc = 1.0f - c;
          float4 nv;
          nv.x = fmaf(c, vv.x, oc * (ab.x * val.x));
          nv.y = fmaf(c, vv.y, oc * (ab.x * val.y));
          nv.z = fmaf(c, vv.z, oc * (ab.x * val.z));
          nv.w = fmaf(c, vv.w, oc * (ab.x * val.w));
          val.x = isw ? nv.x : val.x;
          val.y = isw ? nv.y : val.y;
          val.z = isw ? nv.z : val.z;
          val.w = isw ? nv.w : val.w;
          uint64_t dst = isw ? reinterpret_cast<uint64_t>(Mb + (slot[j] * row_bytes + col_bytes))
                             : reinterpret_cast<uint64_t>(trash);
          if constexpr (F8) {  // requantised (values of non-writes unchanged)
            const Fp8Row q = fp8_quantize(val);
            val = q.val;
            uint64_t edst = isw ? reinterpret_cast<uint64_t>(Eb + slot[j] * erow)
                                : reinterpret_cast<uint64_t>(trash) + 8;
            asm volatile("" : "+v"(dst), "+v"(edst));
            *reinterpret_cast<__attribute__((address_space(1))) uint32_t*>(dst) = q.codes;
            if ((li & 7) == 0)
              *reinterpret_cast<__attribute__((address_space(1))) uint8_t*>(edst) = (uint8_t)q.s;
          } else {
            val = state_round<BF>(val);  // the stored value (exact for non-writes)
            asm volatile("" : "+v"(dst));  // keep one unconditional store: hide the select
            state_store<BF>(dst, val);
          }
        }
        if (!isw && ((vam >> j) & 1u)) {  // dirty read: its value at this point of the stream
          float* y = yr + tk[j] * YS + li;
          atomicAdd(y + 0 * LPG, wq[j] * val.x);
          atomicAdd(y + 1 * LPG, wq[j] * val.y);
          atomicAdd(y + 2 * LPG, wq[j] * val.z);
          atomicAdd(y + 3 * LPG, wq[j] * val.w);
        }
        mv[j] = val;
      }
#pragma unroll
      for (int q = 0; q < EPL; ++q) e[q] = en[q];
    }
    __syncthreads();

    // ---- read phase: whole tokens per lane group, sums in registers ----
    for (int tt = g; tt < nt; tt += GW) {
      const int64_t ltok = (b * a.Tc + t_lo + tt) * a.H + h;
      const int* cs = a.cstart + ltok * (a.parts + 1) + p;
      const int cb = cs[0], ce = cs[1];
      const uint2* cl = a.clean + ltok * a.R;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cb < ce) {
        uint2 c[RPL];
#pragma unroll
        for (int q = 0; q < RPL; ++q) c[q] = cl[min(cb + q * LPG + li, ce - 1)];
        for (int i = cb; i < ce; i += BR) {
          // next batch's ids travel with this batch's row loads
          uint2 cn[RPL];
#pragma unroll
          for (int q = 0; q < RPL; ++q) cn[q] = cl[min(i + BR + q * LPG + li, ce - 1)];
          uint32_t rs[BR];
          float rq[BR];
          float4 rv[BR];
#pragma unroll
          for (int j = 0; j < BR; ++j) {
            const uint32_t si = group_bcast<LPG>(c[j / LPG].x, j % LPG);
            const float qi = __uint_as_float(group_bcast<LPG>(c[j / LPG].y, j % LPG));
            rs[j] = min(si, (uint32_t)a.N - 1u);
            rq[j] = i + j < ce ? qi : 0.0f;  // the tail repeats the last row with weight 0
          }
#pragma unroll
          for (int j = 0; j < BR; ++j) rv[j] = load_row(rs[j]);
#pragma unroll
          for (int j = 0; j < BR; ++j) {
            acc.x = fmaf(rq[j], rv[j].x, acc.x);
            acc.y = fmaf(rq[j], rv[j].y, acc.y);
            acc.z = fmaf(rq[j], rv[j].z, acc.z);
            acc.w = fmaf(rq[j], rv[j].w, acc.w);
          }
#pragma unroll
          for (int q = 0; q < RPL; ++q) c[q] = cn[q];
        }
      }
      float* ring = yr + tt * YS + li;
      const float4 y = make_float4(acc.x + ring[0], acc.y + ring[LPG], acc.z + ring[2 * LPG],
                                   acc.w + ring[3 * LPG]);
      ring[0] = 0.f;
      ring[LPG] = 0.f;
      ring[2 * LPG] = 0.f;
      ring[3 * LPG] = 0.f;
      *reinterpret_cast<float4*>(y_out + ltok * dv) = y;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sum of the parts, RMSNorm over d_v and the output gate; one wavefront per
// (token, head), each lane DV/64 columns (DV >= 64) or a row of 4 (DV < 64).
// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void norm_gate_kernel(StreamArgs a) {
  constexpr int LPR = DV / 4 < 64 ? DV / 4 : 64;  // lanes per row
  constexpr int CPL = DV / LPR;                  // columns per lane (multiple of 4)
  constexpr int RPW = 64 / LPR;                  // rows per wavefront
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, li = lane % LPR;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + sub;
  const int64_t rows = a.B * a.Tc * a.H;
  const bool ok = row < rows;
  // a chunk's rows fit 32 bits (its buffers are bounded near 2 GiB): 32-bit index
  // arithmetic, far cheaper per lane than 64-bit division
  const uint32_t rr = ok ? (uint32_t)row : 0u;
  const uint32_t h = rr % (uint32_t)a.H;
  const uint32_t bt = rr / (uint32_t)a.H;
  const uint32_t b = bt / (uint32_t)a.Tc, t = bt - b * (uint32_t)a.Tc;
  const int64_t grow = ((int64_t)b * a.T + a.t0 + t) * a.H + h;  // row of the full [B,T,H] arrays
  float y[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) y[c] = 0.0f;
#pragma unroll 4
  for (int p = 0; p < a.parts; ++p) {
    const float* src = a.y_part + ((int64_t)p * rows + rr) * DV + li * CPL;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + c);
      y[c] += v.x;
      y[c + 1] += v.y;
      y[c + 2] += v.z;
      y[c + 3] += v.w;
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) ss += y[c] * y[c];
  for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LPR);
  const float rn = rsqrtf(ss / (float)DV + a.eps);
  if (!ok) return;
  const float* gt = a.gate + grow * DV + li * CPL;
  float* o = a.out + grow * DV + li * CPL;
  float* yo = a.y_raw ? a.y_raw + grow * DV + li * CPL : nullptr;
#pragma unroll
  for (int c = 0; c < CPL; c += 4) {
    const float4 gv = *reinterpret_cast<const float4*>(gt + c);
    float4 nw = make_float4(1.f, 1.f, 1.f, 1.f);
    if (a.norm_w) nw = *reinterpret_cast<const float4*>(a.norm_w + h * DV + li * CPL + c);
    float4 ov;
    ov.x = y[c] * rn * nw.x * gv.x;
    ov.y = y[c + 1] * rn * nw.y * gv.y;
    ov.z = y[c + 2] * rn * nw.z * gv.z;
    ov.w = y[c + 3] * rn * nw.w * gv.w;
    *reinterpret_cast<float4*>(o + c) = ov;
    if (yo) *reinterpret_cast<float4*>(yo + c) = make_float4(y[c], y[c + 1], y[c + 2], y[c + 3]);
  }
}

// Training forward with a quantised log: the walk left the chunk's replaced rows in
// fp32 in the staging area ([B][Tc of the plan][H][W] rows); encode each row with its
// absmax into the caller's log at its global place.  One workgroup per (b, t, h) of
// the chunk, its W rows RPB at a time, LPR lanes per row.
template <int DV>
__global__ __launch_bounds__(256) void log_quantize_kernel(StreamArgs a, ScanArgs sa) {
  constexpr int LPR = DV / 4;      // one float4 per lane (at most a wavefront per row)
  constexpr int RPB = 256 / LPR;   // rows per pass
  const uint32_t bth = blockIdx.x;  // (b * Tc + t) * H + h; a chunk's count fits 32 bits
  const uint32_t h = bth % (uint32_t)a.H;
  const uint32_t bt = bth / (uint32_t)a.H;
  const uint32_t b = bt / (uint32_t)a.Tc, t = bt - b * (uint32_t)a.Tc;
  const float4* src =
      reinterpret_cast<const float4*>(a.log + (((int64_t)b * a.log_T + t) * a.H + h) * a.W * DV);
  const int64_t r0 = (((int64_t)b * a.T + a.t0 + t) * a.H + h) * a.W;
  const int li = threadIdx.x % LPR;
  for (int k = threadIdx.x / LPR; k < a.W; k += RPB)  // a row's lanes share k
    log_store<LPR>(sa.log, sa.log_scale, sa.log_fmt, r0 + k, DV, src[k * LPR + li], li);
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace

StreamPlan plan_stream(const sdm_dims& d, int64_t N, int64_t stage_bytes) {
  (void)N;
  StreamPlan pl;
  pl.stage_bytes = stage_bytes;
  const int64_t walks = d.B * (int64_t)d.H;
  pl.two_phase = !(d.flags & SDM_FLAG_SCAN_STREAM);
  pl.SW = d.d_v >= 32 ? 32 : d.d_v;
  // Two-phase: 256-byte column slices (fp32) where the grid still reaches one
  // workgroup per CU with at most 4 parts.  Longer row segments per access move
  // faster through HBM; more parts would multiply the partial read vectors.
  if (pl.two_phase && d.d_v % 64 == 0 && walks * (d.d_v / 64) * 4 >= 256) pl.SW = 64;
  pl.S = d.d_v / pl.SW;
  pl.NT = 1024;
  const int lpg = pl.SW / 4;
  const int gw = pl.NT / lpg;
  // the lane groups of a walk are split over `parts` workgroups until the grid
  // reaches one workgroup per CU
  int parts = 1;
  // (parts stay below 64: the reverse bucketing pass gives each part's start a lane)
  while (walks * pl.S * parts < 256 && gw * parts * 2 <= MAX_GT && parts * 2 < 64) parts *= 2;
  pl.parts = parts;
  pl.GT = gw * parts;
  pl.log2GT = ilog2(pl.GT);
  // token chunk: bound the per-token buffers to ~2 GiB
  const int64_t per_tok = walks * ((d.W + d.R) * 8 + (int64_t)parts * d.d_v * 4 +
                                   (pl.two_phase ? d.R * 8 + (parts + 1) * 4 : 0) + stage_bytes);
  int64_t tc = (2ll << 30) / per_tok;
  tc = tc < ROUND ? ROUND : (tc / ROUND) * ROUND;
  pl.Tc = d.T < tc ? d.T : tc;
  pl.rounds = (int)((pl.Tc + ROUND - 1) / ROUND);
  return pl;
}

namespace {

// Byte offsets of the scan's buffers inside the workspace (256-byte aligned).
struct StreamLayout {
  size_t counts, offsets, totals, entries, y_part, trash, begins, clean, cstart, stage, total;
};

StreamLayout stream_layout(const sdm_dims& d, const StreamPlan& pl) {
  const int64_t walks = d.B * (int64_t)d.H;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  StreamLayout L;
  size_t s = 0;
  L.counts = s;
  s += al((size_t)walks * pl.rounds * pl.GT * 4);
  L.offsets = s;
  s += al((size_t)walks * pl.GT * (pl.rounds + 1) * 4);
  L.totals = s;
  s += al((size_t)walks * pl.GT * 4);
  L.entries = s;
  s += al((size_t)walks * pl.Tc * (d.W + d.R) * 8);
  L.y_part = s;
  s += al((size_t)pl.parts * walks * pl.Tc * d.d_v * 4);
  L.trash = s;
  s += al((size_t)walks * pl.S * pl.parts * pl.NT * 16);
  L.begins = L.clean = L.cstart = s;
  if (pl.two_phase) {
    L.begins = s;
    s += al((size_t)walks * pl.GT * pl.rounds * 4);
    L.clean = s;
    s += al((size_t)walks * pl.Tc * d.R * 8);
    L.cstart = s;
    s += al((size_t)walks * pl.Tc * (pl.parts + 1) * 4);
  }
  L.stage = s;
  s += al((size_t)walks * pl.Tc * pl.stage_bytes);
  L.total = s;
  return L;
}

}  // namespace

hipError_t launch_stream_buckets(const StreamArgs& a, int64_t walks, bool train,
                                 hipStream_t st) {
  {
    KernelTimer kt("bucket_count", st);
    hipLaunchKernelGGL(bucket_count_kernel, dim3((unsigned)(walks * a.rounds)), dim3(256), 0, st,
                       a);
  }
  const hipError_t e = launch_offsets(a, walks, st);
  if (e != hipSuccess) return e;
  KernelTimer kt("bucket_scatter", st);
  if (train)
    hipLaunchKernelGGL(bucket_scatter_kernel<true>, dim3((unsigned)(walks * a.rounds)), dim3(64),
                       0, st, a);
  else
    hipLaunchKernelGGL(bucket_scatter_kernel<false>, dim3((unsigned)(walks * a.rounds)),
                       dim3(64), 0, st, a);
  return hipGetLastError();
}

size_t stream_workspace_bytes(const sdm_dims& d, const StreamPlan& pl) {
  return stream_layout(d, pl).total;
}

hipError_t launch_stream_scan(const ScanArgs& sa, const StreamPlan& pl, void* ws,
                              hipStream_t st) {
  StreamArgs a;
  a.idx_w = sa.idx_w;
  a.wt_w = sa.wt_w;
  a.idx_r = sa.idx_r;
  a.wt_r = sa.wt_r;
  a.v = sa.v;
  a.gate = sa.gate;
  a.alpha = sa.alpha;
  a.beta = sa.beta;
  a.norm_w = sa.norm_w;
  a.state = sa.state;
  a.out = sa.out;
  a.y_raw = sa.y_raw;
  // training forward: the rows replaced by each write, stored by the slot's owner, in
  // fp32 to the caller's log, or (quantised formats) to a chunk-sized staging area that
  // log_quantize_kernel encodes into the caller's log after the walk
  const bool train = sa.log != nullptr;
  const bool qlog = train && sa.log_fmt != LOG_F32;
  if (train && (sa.state_bf16 || sa.state_fp8)) return hipErrorInvalidValue;
  if (sa.state_fp8 && !pl.two_phase) return hipErrorInvalidValue;
  if (qlog && pl.stage_bytes < (int64_t)sa.W * sa.d_v * 4) return hipErrorInvalidValue;
  a.B = sa.B;
  a.T = sa.T;
  a.H = sa.H;
  a.N = sa.N;
  a.W = sa.W;
  a.R = sa.R;
  a.d_v = sa.d_v;
  a.eps = sa.eps;
  a.S = pl.S;
  a.parts = pl.parts;
  a.GT = pl.GT;
  a.log2GT = pl.log2GT;
  a.log2GW = ilog2(pl.GT / pl.parts);
  const int64_t walks = sa.B * (int64_t)sa.H;
  sdm_dims dd{};
  dd.B = sa.B;
  dd.H = sa.H;
  dd.W = sa.W;
  dd.R = sa.R;
  dd.d_v = sa.d_v;
  const StreamLayout L = stream_layout(dd, pl);
  char* base = static_cast<char*>(ws);
  a.counts = reinterpret_cast<int*>(base + L.counts);
  a.offsets = reinterpret_cast<int*>(base + L.offsets);
  a.totals = reinterpret_cast<int*>(base + L.totals);
  a.entries = reinterpret_cast<uint2*>(base + L.entries);
  a.y_part = reinterpret_cast<float*>(base + L.y_part);
  a.trash = reinterpret_cast<float4*>(base + L.trash);
  a.begins = reinterpret_cast<int*>(base + L.begins);
  a.clean = reinterpret_cast<uint2*>(base + L.clean);
  a.cstart = reinterpret_cast<int*>(base + L.cstart);
  a.log = qlog ? reinterpret_cast<float*>(base + L.stage) : static_cast<float*>(sa.log);
  for (int64_t t0 = 0; t0 < sa.T; t0 += pl.Tc) {
    a.t0 = t0;
    a.Tc = sa.T - t0 < pl.Tc ? sa.T - t0 : pl.Tc;
    a.log_T = qlog ? pl.Tc : sa.T;
    a.log_t0 = qlog ? 0 : t0;
    a.rounds = (int)((a.Tc + ROUND - 1) / ROUND);
    a.walk_entries = a.Tc * (sa.W + sa.R);

    {
      KernelTimer kt("bucket_count", st);
      hipLaunchKernelGGL(bucket_count_kernel, dim3((unsigned)(walks * a.rounds)), dim3(256), 0,
                         st, a);
    }
    {
      const hipError_t e = launch_offsets(a, walks, st);
      if (e != hipSuccess) return e;
    }
    if (pl.two_phase) {
      const size_t lds = (size_t)pl.GT * 4 + (size_t)((sa.N + 31) / 32) * 4;
      const bool narrow = sa.W <= 64 && sa.R <= 64;
      const void* rev =
          narrow ? (train ? reinterpret_cast<const void*>(bucket_scatter_rev_kernel<1, 8, true>)
                          : reinterpret_cast<const void*>(bucket_scatter_rev_kernel<1, 8, false>))
                 : (train ? reinterpret_cast<const void*>(bucket_scatter_rev_kernel<2, 4, true>)
                          : reinterpret_cast<const void*>(bucket_scatter_rev_kernel<2, 4, false>));
      if (lds > 65536) {  // slot bitmaps beyond 64 KiB (N > ~500k) need the larger LDS limit
        const hipError_t e = hipFuncSetAttribute(rev, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
      }
      const dim3 rg((unsigned)(walks * a.rounds));
      {
        KernelTimer kt("bucket_scatter_rev", st);
        if (narrow && train)
          hipLaunchKernelGGL((bucket_scatter_rev_kernel<1, 8, true>), rg, dim3(64), lds, st, a);
        else if (narrow)
          hipLaunchKernelGGL((bucket_scatter_rev_kernel<1, 8, false>), rg, dim3(64), lds, st, a);
        else if (train)
          hipLaunchKernelGGL((bucket_scatter_rev_kernel<2, 4, true>), rg, dim3(64), lds, st, a);
        else
          hipLaunchKernelGGL((bucket_scatter_rev_kernel<2, 4, false>), rg, dim3(64), lds, st, a);
      }
      {  // the walk takes its loop bounds from the bucketing outputs: launch it only on them
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const dim3 grid((unsigned)(walks * pl.S * pl.parts));
      KernelTimer kt("two_phase_scan", st);
      if (train && pl.SW == 64)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 64, BQ_TRAIN32, 8, false, true>), grid,
                           dim3(1024), 0, st, a);
      else if (train && pl.SW == 32)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 32, BQ_TRAIN32, 8, false, true>), grid,
                           dim3(1024), 0, st, a);
      else if (train)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 16, BQ_TRAIN16, 8, false, true>), grid,
                           dim3(1024), 0, st, a);
      else if (pl.SW == 64 && sa.state_fp8)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 64, 8, 8, false, false, true>), grid,
                           dim3(1024), 0, st, a);
      else if (pl.SW == 32 && sa.state_fp8)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 32, 8, 8, false, false, true>), grid,
                           dim3(1024), 0, st, a);
      else if (sa.state_fp8)
        return hipErrorInvalidValue;  // blocks of 32 columns need 32-column slices
      else if (pl.SW == 64 && sa.state_bf16)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 64, 8, 8, true, false>), grid, dim3(1024), 0, st,
                           a);
      else if (pl.SW == 64)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 64, 8, 8, false, false>), grid, dim3(1024), 0, st,
                           a);
      else if (pl.SW == 32 && sa.state_bf16)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 32, 8, 8, true, false>), grid, dim3(1024), 0, st,
                           a);
      else if (pl.SW == 32)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 32, 8, 8, false, false>), grid, dim3(1024), 0, st,
                           a);
      else if (sa.state_bf16)
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 16, 8, 8, true, false>), grid, dim3(1024), 0, st,
                           a);
      else
        hipLaunchKernelGGL((two_phase_scan_kernel<1024, 16, 8, 8, false, false>), grid, dim3(1024), 0, st,
                           a);
    } else {
      {
        KernelTimer kt("bucket_scatter", st);
        if (train)
          hipLaunchKernelGGL(bucket_scatter_kernel<true>, dim3((unsigned)(walks * a.rounds)),
                             dim3(64), 0, st, a);
        else
          hipLaunchKernelGGL(bucket_scatter_kernel<false>, dim3((unsigned)(walks * a.rounds)),
                             dim3(64), 0, st, a);
      }
      {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const dim3 grid((unsigned)(walks * pl.S * pl.parts));
      KernelTimer kt("stream_scan", st);
      if (train && pl.SW == 32)
        hipLaunchKernelGGL((stream_scan_kernel<1024, 32, 6, false, true>), grid, dim3(1024), 0, st,
                           a);
      else if (train)
        hipLaunchKernelGGL((stream_scan_kernel<1024, 16, 6, false, true>), grid, dim3(1024), 0, st,
                           a);
      else if (pl.SW == 32 && sa.state_bf16)
        hipLaunchKernelGGL((stream_scan_kernel<1024, 32, 8, true, false>), grid, dim3(1024), 0, st, a);
      else if (pl.SW == 32)
        hipLaunchKernelGGL((stream_scan_kernel<1024, 32, 8, false, false>), grid, dim3(1024), 0, st, a);
      else if (sa.state_bf16)
        hipLaunchKernelGGL((stream_scan_kernel<1024, 16, 8, true, false>), grid, dim3(1024), 0, st, a);
      else
        hipLaunchKernelGGL((stream_scan_kernel<1024, 16, 8, false, false>), grid, dim3(1024), 0, st, a);
    }
    if (qlog) {
      const dim3 qg((unsigned)(sa.B * a.Tc * sa.H));
      KernelTimer kt("log_quantize", st);
      switch (sa.d_v) {
        case 16: hipLaunchKernelGGL(log_quantize_kernel<16>, qg, dim3(256), 0, st, a, sa); break;
        case 32: hipLaunchKernelGGL(log_quantize_kernel<32>, qg, dim3(256), 0, st, a, sa); break;
        case 64: hipLaunchKernelGGL(log_quantize_kernel<64>, qg, dim3(256), 0, st, a, sa); break;
        case 128: hipLaunchKernelGGL(log_quantize_kernel<128>, qg, dim3(256), 0, st, a, sa); break;
        case 256: hipLaunchKernelGGL(log_quantize_kernel<256>, qg, dim3(256), 0, st, a, sa); break;
        default: return hipErrorInvalidValue;
      }
    }
    const int64_t rows = sa.B * a.Tc * sa.H;
    // rows per 256-thread block: 4 wavefronts x (64 / lanes per row)
    const int lpr = sa.d_v / 4 < 64 ? sa.d_v / 4 : 64;
    const int64_t rpb = 4 * (64 / lpr);
    const dim3 ng((unsigned)((rows + rpb - 1) / rpb));
    KernelTimer kt("norm_gate", st);
    switch (sa.d_v) {
      case 16: hipLaunchKernelGGL(norm_gate_kernel<16>, ng, dim3(256), 0, st, a); break;
      case 32: hipLaunchKernelGGL(norm_gate_kernel<32>, ng, dim3(256), 0, st, a); break;
      case 64: hipLaunchKernelGGL(norm_gate_kernel<64>, ng, dim3(256), 0, st, a); break;
      case 128: hipLaunchKernelGGL(norm_gate_kernel<128>, ng, dim3(256), 0, st, a); break;
      case 256: hipLaunchKernelGGL(norm_gate_kernel<256>, ng, dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


hipError_t launch_log_quantize(const ScanArgs& sa, const float* stage, int64_t t0, int64_t Tc,
                               hipStream_t st) {
  StreamArgs a = {};
  a.log = const_cast<float*>(stage);
  a.log_T = Tc;
  a.T = sa.T;
  a.t0 = t0;
  a.Tc = Tc;
  a.H = sa.H;
  a.W = sa.W;
  const dim3 grid((unsigned)(sa.B * Tc * sa.H));
  KernelTimer kt("log_quantize", st);
  switch (sa.d_v) {
    case 16: hipLaunchKernelGGL(log_quantize_kernel<16>, grid, dim3(256), 0, st, a, sa); break;
    case 32: hipLaunchKernelGGL(log_quantize_kernel<32>, grid, dim3(256), 0, st, a, sa); break;
    case 64: hipLaunchKernelGGL(log_quantize_kernel<64>, grid, dim3(256), 0, st, a, sa); break;
    case 128: hipLaunchKernelGGL(log_quantize_kernel<128>, grid, dim3(256), 0, st, a, sa); break;
    case 256: hipLaunchKernelGGL(log_quantize_kernel<256>, grid, dim3(256), 0, st, a, sa); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norm_gate(const ScanArgs& sa, const float* y, hipStream_t st) {
  StreamArgs a = {};
  a.gate = sa.gate;
  a.norm_w = sa.norm_w;
  a.out = sa.out;
  a.y_raw = sa.y_raw;
  a.y_part = const_cast<float*>(y);
  a.B = sa.B;
  a.T = sa.T;
  a.t0 = 0;
  a.Tc = sa.T;
  a.H = sa.H;
  a.d_v = sa.d_v;
  a.eps = sa.eps;
  a.parts = 1;
  const int64_t rows = sa.B * sa.T * sa.H;
  const int lpr = sa.d_v / 4 < 64 ? sa.d_v / 4 : 64;
  const int64_t rpb = 4 * (64 / lpr);
  const dim3 ng((unsigned)((rows + rpb - 1) / rpb));
  KernelTimer kt("norm_gate", st);
  switch (sa.d_v) {
    case 16: hipLaunchKernelGGL(norm_gate_kernel<16>, ng, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(norm_gate_kernel<32>, ng, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(norm_gate_kernel<64>, ng, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(norm_gate_kernel<128>, ng, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL(norm_gate_kernel<256>, ng, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sdm
