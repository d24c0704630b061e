// Backward of the recurrent sparse scan on the slot-owner stream schedule: the
// reverse walk of scan_backward.hip (same arithmetic, the same write log), made
// parallel over slots so that a few dozen long walks still fill the chip.
//
// Per (b, h) memory, tokens in reverse, each token's read undone before its write
// (the m.163.com article on arXiv 2607.07386, section 八: the in-place update is
// undone in backward from the rows it overwrote):
//   read  r:  d_q[r] = <dy, M[i]>,  dM[i] += q[r] dy           (M after t's writes)
//   write k:  m = logged row, c = beta k, G = dM[i]:
//             d_v += c G,  dc = <G, v - alpha m>,  gm = <G, m>,
//             d_k = beta dc,  d_beta += k dc,  d_alpha += (1 - c) gm,
//             dM[i] = alpha (1 - c) G,  M[i] = m
//
// Schedule (mirrors the forward stream schedule of scan_stream.hip):
//  * The forward's bucketing pre-passes lay each walk's accesses out per lane group
//    (hash of the slot id), in token order with writes before reads, in rounds of
//    kStreamRound tokens; here each entry carries the access's position in its
//    token's id list.  A lane group walks its segments backwards, so every slot
//    sees its accesses in exactly reverse order, and a slot's M and dM rows are
//    only ever touched by one thread per column chunk: program order is the only
//    ordering the state needs.
//  * Lane groups cover SW-float column slices of d_v.  Every dot product above is
//    an output only, so each slice writes its partial dot per access and a reduce
//    pass sums the slices in a fixed order (d_q, d_k, d_alpha, d_beta are then
//    reproducible bit for bit).  d_v is a scatter from slot owners to tokens: it is
//    summed per round in an LDS ring with float atomics, per part, so it is
//    reproducible only up to fp32 summation order.
//  * dy (RMSNorm and gate backward) is computed per token before the walk and
//    staged per round in LDS with v and (alpha, beta).
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int ROUND = kStreamRound;
constexpr uint32_t SLOT_MASK = 0xFFFFFFu;
constexpr int PREP_TOK = 256;  // tokens per norm/gate block (d_gamma partial granule)
constexpr int kNT = 1024;      // threads of a reverse-walk workgroup
// accesses a lane group keeps in flight: fp32 log / quantised log (decoding takes
// registers)
#ifndef SDM_BACK_BQ
#define SDM_BACK_BQ 4
#endif
constexpr int BQ_F32 = SDM_BACK_BQ;
constexpr int BQ_Q = 4;

struct BackStreamArgs {
  ScanBackArgs s;
  const uint2* entries;  // [walks][walk_entries]
  const int* offsets;    // [walks][GT][rounds + 1]
  float* dy;             // [B][Tc][H][d_v]
  float2* pw;            // [S*parts][B][Tc][H][W]  per (slice, part) (dc, gm) of each write
  float* pr;             // [S*parts][B][Tc][H][R]  per (slice, part) d_q of each read
  float* dv_part;        // [parts][B][Tc][H][d_v]
  float* gpart;          // [B*H][gblocks][d_v]  d_gamma partials
  int64_t t0, Tc, walk_entries, rows_c;  // rows_c = B*Tc*H
  int32_t S, parts, GT, rounds, gblocks, pblocks;
};

__device__ __forceinline__ float4 f4s(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Sum over an LPG-lane group (LPG = 4 or 8), every lane gets it: quad swaps by DPP,
// then the other quad of the 8 by row_half_mirror.  A fixed pairing, so the sum
// has one rounding order.
template <int LPG>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
  if (LPG >= 8)  // row_half_mirror: the other quad of the 8-lane half-row
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));
  if (LPG == 16)  // row_mirror: the other half of the 16-lane row
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));
  return x;
}

// Sum over the LPR lanes of one row (xor butterfly).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, LPR);
  return x;
}

// ---------------------------------------------------------------------------
// Norm/gate backward of the chunk's tokens: dy and d_gate per token, and one d_gamma
// partial per (walk, PREP_TOK-token block), summed in a fixed order.
// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void back_prep_kernel(BackStreamArgs A) {
  constexpr int LPR = DV / 4;
  constexpr int G = 256 / LPR;
  __shared__ float4 red[G][LPR];
  const ScanBackArgs& a = A.s;
  const int tid = threadIdx.x, li = tid % LPR, grp = tid / LPR;
  const int64_t w = blockIdx.x / A.pblocks;
  const int blk = (int)(blockIdx.x - w * A.pblocks);
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const float4 gam = a.norm_w ? reinterpret_cast<const float4*>(a.norm_w + (int64_t)h * DV)[li]
                              : f4s(1.0f);
  float4 dgam = f4s(0.0f);
  const int64_t t_hi = min<int64_t>(A.Tc, (int64_t)(blk + 1) * PREP_TOK);
#pragma unroll 4  // several tokens' loads in flight; d_gamma keeps its summation order
  for (int64_t t = (int64_t)blk * PREP_TOK + grp; t < t_hi; t += G) {
    const int64_t tok = (b * a.T + A.t0 + t) * a.H + h;
    const int64_t tokc = (b * A.Tc + t) * a.H + h;
    const float4 y = reinterpret_cast<const float4*>(a.y_raw + tok * DV)[li];
    const float4 gt = reinterpret_cast<const float4*>(a.gate + tok * DV)[li];
    const float4 dout = reinterpret_cast<const float4*>(a.d_out + tok * DV)[li];
    const float s = rsqrtf(row_sum<LPR>(dot4(y, y)) / (float)DV + a.eps);
    const float4 yh = make_float4(y.x * s, y.y * s, y.z * s, y.w * s);
    const float4 u = make_float4(dout.x * gam.x * gt.x, dout.y * gam.y * gt.y,
                                 dout.z * gam.z * gt.z, dout.w * gam.w * gt.w);
    const float mu = row_sum<LPR>(dot4(u, yh)) / (float)DV;
    reinterpret_cast<float4*>(A.dy + tokc * DV)[li] =
        make_float4(s * (u.x - yh.x * mu), s * (u.y - yh.y * mu), s * (u.z - yh.z * mu),
                    s * (u.w - yh.w * mu));
    reinterpret_cast<float4*>(a.g_gate + tok * DV)[li] =
        make_float4(dout.x * yh.x * gam.x, dout.y * yh.y * gam.y, dout.z * yh.z * gam.z,
                    dout.w * yh.w * gam.w);
    dgam.x += dout.x * yh.x * gt.x;
    dgam.y += dout.y * yh.y * gt.y;
    dgam.z += dout.z * yh.z * gt.z;
    dgam.w += dout.w * yh.w * gt.w;
  }
  red[grp][li] = dgam;
  __syncthreads();
  if (grp == 0) {
    float4 sv = red[0][li];
    for (int q = 1; q < G; ++q) {
      const float4 o = red[q][li];
      sv.x += o.x;
      sv.y += o.y;
      sv.z += o.z;
      sv.w += o.w;
    }
    const int64_t gb = A.t0 / PREP_TOK + blk;  // chunks start on block boundaries
    reinterpret_cast<float4*>(A.gpart + (w * A.gblocks + gb) * DV)[li] = sv;
  }
}

// ---------------------------------------------------------------------------
// The reverse walk.  Workgroup = (walk, slice, part); NT threads; SW floats per
// slice; LPG = SW/4 lanes per group; GW = NT/LPG groups; batches of BQ accesses
// taken from the end of the group's round segment backwards.
// Each round is walked in sub-rounds of SUB tokens, last first.  A group's segment
// is in token order, so a sub-round's accesses are the next run of it going down.
// Per sub-round the workgroup stages dy, v and the gates of its tokens, collects the
// partial dots of every access in LDS at (token, id position) -- each access has one
// owner, so no atomics -- and d_v in an LDS ring, then writes them out as whole rows.
// ---------------------------------------------------------------------------
constexpr int SUB = 64;  // tokens per sub-round

template <int NT, int SW, int BQ, int LF>
__global__ __launch_bounds__(NT) void stream_backward_kernel(BackStreamArgs A) {
  constexpr int LPG = SW / 4;
  constexpr int GW = NT / LPG;
  constexpr int EPL = (BQ + LPG - 1) / LPG;  // entries loaded per lane per batch
  constexpr int YS = SW + 8;  // padded d_v ring row (column 4l + c of lane l at c*LPG + l)
  __shared__ __attribute__((aligned(16))) float dvr[SUB * YS];
  __shared__ __attribute__((aligned(16))) float dys[SUB * SW];
  __shared__ __attribute__((aligned(16))) float vs[SUB * SW];
  __shared__ float2 gab[SUB];                                        // (alpha, beta)
  __shared__ float pdq[SUB * SDM_MAX_COUNT];                         // [token][R] d_q
  __shared__ __attribute__((aligned(8))) float2 pdc[SUB * SDM_MAX_COUNT];  // [token][W] (dc, gm)

  const ScanBackArgs& a = A.s;
  const int tid = threadIdx.x;
  const int li = tid % LPG;
  const int g = tid / LPG;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % A.parts);
  const int64_t ws = wg / A.parts;
  const int sl = (int)(ws % A.S);
  const int64_t w = ws / A.S;
  const int64_t b = w / a.H;
  const int h = (int)(w - b * a.H);
  const int gg = p * GW + g;
  const int dv = a.d_v;

  for (int x = tid; x < SUB * YS; x += NT) dvr[x] = 0.0f;
  for (int x = tid; x < SUB * a.R; x += NT) pdq[x] = 0.0f;
  for (int x = tid; x < SUB * a.W; x += NT) pdc[x] = make_float2(0.0f, 0.0f);

  char* Mb = reinterpret_cast<char*>(a.state + w * (int64_t)a.N * dv);
  char* Gb = reinterpret_cast<char*>(a.d_state + w * (int64_t)a.N * dv);
  const uint32_t col_bytes = (uint32_t)(sl * SW + li * 4) * 4u;
  const uint32_t row_bytes = (uint32_t)dv * 4u;
  const int c4 = sl * LPG + li;  // this lane's column / 4
  const uint2* ent = A.entries + w * A.walk_entries;
  const int last = (int)A.walk_entries - 1;
  const int* offs = A.offsets + ((int64_t)w * A.GT + gg) * (A.rounds + 1);
  const int64_t tok_base = (b * a.T + A.t0) * a.H + h;  // chunk token t -> tok_base + t*H
  const int64_t tokc_base = b * A.Tc * a.H + h;         // chunk row of t: tokc_base + t*H
  const int64_t u = (int64_t)sl * A.parts + p;         // this workgroup's partial-dot plane
  float2* pw = A.pw + u * A.rows_c * a.W;
  float* pr = A.pr + u * A.rows_c * a.R;

  for (int r = A.rounds - 1; r >= 0; --r) {
    const int64_t t_lo = (int64_t)r * ROUND;
    const int nt = (int)min<int64_t>(ROUND, A.Tc - t_lo);
    const int beg = offs[r];
    const int end = offs[r + 1];
    // entry at stream position pos, clamped into the walk's entries
    auto at = [&](int pos) { return max(min(max(pos, beg), min(end - 1, last)), 0); };
    int i = end;  // this group's accesses below i are still to be undone
    for (int s_lo = ((nt - 1) / SUB) * SUB; s_lo >= 0; s_lo -= SUB) {
      const int ns = min(SUB, nt - s_lo);
      for (int x = tid; x < ns * LPG; x += NT) {
        const int tt = x / LPG, q4 = x % LPG;
        const int64_t tok = tok_base + (t_lo + s_lo + tt) * a.H;
        const int64_t tokc = tokc_base + (t_lo + s_lo + tt) * a.H;
        *reinterpret_cast<float4*>(vs + tt * SW + q4 * 4) =
            *reinterpret_cast<const float4*>(a.v + tok * dv + sl * SW + q4 * 4);
        *reinterpret_cast<float4*>(dys + tt * SW + q4 * 4) =
            *reinterpret_cast<const float4*>(A.dy + tokc * dv + sl * SW + q4 * 4);
      }
      for (int x = tid; x < ns; x += NT) {
        const int64_t tok = tok_base + (t_lo + s_lo + x) * a.H;
        gab[x] = make_float2(a.alpha[tok], a.beta[tok]);
      }
      __syncthreads();

      uint2 e[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) e[q] = ent[at(i - 1 - q * LPG - li)];
      while (i > beg) {
        uint2 en[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) en[q] = ent[at(i - BQ - 1 - q * LPG - li)];
        uint32_t slot[BQ];
        int tk[BQ], kk[BQ];
        uint32_t rdm = 0, vam = 0;  // bit j: access j is a read / belongs to this sub-round
        float wq[BQ];
        float4 X[BQ], Gd[BQ];  // M (reads) or the logged row (writes); dM
#pragma unroll
        for (int j = 0; j < BQ; ++j) {
          const int src = j % LPG, q = j / LPG;
          const uint32_t ex = group_bcast<LPG>(e[q].x, src);
          const uint32_t ey = group_bcast<LPG>(e[q].y, src);
          const bool rd = ey >> 31;
          const int tr = min((int)(ex >> 24), nt - 1);  // token within the round
          slot[j] = min(ex & SLOT_MASK, (uint32_t)a.N - 1u);
          tk[j] = min(max(tr - s_lo, 0), ns - 1);       // token within the sub-round
          kk[j] = min((int)(ey & 0x7fffffffu), (rd ? a.R : a.W) - 1);
          rdm |= (uint32_t)rd << j;
          // tokens never increase going down a segment: the valid accesses are a prefix
          vam |= (uint32_t)(i - 1 - j >= beg && tr >= s_lo) << j;
        }
        const int m = __builtin_ctz(~vam);  // accesses of this sub-round in the batch
        if (m == 0) break;
#pragma unroll
        for (int j = 0; j < BQ; ++j) {
          const bool rd = (rdm >> j) & 1u;
          const int64_t tok = tok_base + (t_lo + s_lo + tk[j]) * a.H;
          wq[j] = rd ? a.wt_r[tok * a.R + kk[j]] : a.wt_w[tok * a.W + kk[j]];
          const uint32_t off = slot[j] * row_bytes + col_bytes;
          if constexpr (LF == LOG_F32) {
            const float4* src =
                rd ? reinterpret_cast<const float4*>(Mb + off)
                   : reinterpret_cast<const float4*>(static_cast<const float*>(a.log) +
                                                     (tok * a.W + kk[j]) * dv) +
                         c4;
            X[j] = *src;
          } else {
            X[j] = rd ? *reinterpret_cast<const float4*>(Mb + off)
                      : log_load(a.log, a.log_scale, LF, tok * a.W + kk[j], dv, c4);
          }
          Gd[j] = *reinterpret_cast<const float4*>(Gb + off);
        }
#pragma unroll
        for (int j = 0; j < BQ; ++j) {
          if (!((vam >> j) & 1u)) continue;
          // the latest earlier access of this slot in the batch left M in X and dM in Gd
          float4 mv = X[j], gv = Gd[j];
#pragma unroll
          for (int jj = 0; jj < j; ++jj) {
            const bool fwd = ((vam >> jj) & 1u) && slot[jj] == slot[j];
            mv.x = fwd ? X[jj].x : mv.x;
            mv.y = fwd ? X[jj].y : mv.y;
            mv.z = fwd ? X[jj].z : mv.z;
            mv.w = fwd ? X[jj].w : mv.w;
            gv.x = fwd ? Gd[jj].x : gv.x;
            gv.y = fwd ? Gd[jj].y : gv.y;
            gv.z = fwd ? Gd[jj].z : gv.z;
            gv.w = fwd ? Gd[jj].w : gv.w;
          }
          const uint32_t off = slot[j] * row_bytes + col_bytes;
          if ((rdm >> j) & 1u) {
            const float4 d = *reinterpret_cast<const float4*>(dys + tk[j] * SW + li * 4);
            const float dq = group_sum<LPG>(dot4(d, mv));
            const float q = wq[j];
            float4 n;
            n.x = fmaf(q, d.x, gv.x);
            n.y = fmaf(q, d.y, gv.y);
            n.z = fmaf(q, d.z, gv.z);
            n.w = fmaf(q, d.w, gv.w);
            *reinterpret_cast<float4*>(Gb + off) = n;
            if (li == 0) pdq[tk[j] * a.R + kk[j]] = dq;
            X[j] = mv;
            Gd[j] = n;
          } else {
            const float4 mm = X[j];
            const float2 ab = gab[tk[j]];
            const float4 vv = *reinterpret_cast<const float4*>(vs + tk[j] * SW + li * 4);
            const float c = ab.y * wq[j];
            const float oc = 1.0f - c;
            const float4 er = make_float4(vv.x - ab.x * mm.x, vv.y - ab.x * mm.y,
                                          vv.z - ab.x * mm.z, vv.w - ab.x * mm.w);
            const float dc = group_sum<LPG>(dot4(gv, er));
            const float gm = group_sum<LPG>(dot4(gv, mm));
            float* y = dvr + tk[j] * YS + li;
            atomicAdd(y + 0 * LPG, c * gv.x);
            atomicAdd(y + 1 * LPG, c * gv.y);
            atomicAdd(y + 2 * LPG, c * gv.z);
            atomicAdd(y + 3 * LPG, c * gv.w);
            const float f = ab.x * oc;
            const float4 n = make_float4(f * gv.x, f * gv.y, f * gv.z, f * gv.w);
            *reinterpret_cast<float4*>(Gb + off) = n;
            *reinterpret_cast<float4*>(Mb + off) = mm;
            if (li == 0) pdc[tk[j] * a.W + kk[j]] = make_float2(dc, gm);
            Gd[j] = n;
          }
        }
        i -= m;
        if (m < BQ) break;  // the rest of the segment belongs to earlier sub-rounds
#pragma unroll
        for (int q = 0; q < EPL; ++q) e[q] = en[q];
      }
      __syncthreads();
      // this workgroup's d_v and partial dots of the sub-round's tokens, whole rows;
      // the LDS rows are cleared for the next sub-round
      for (int x = tid; x < ns * LPG; x += NT) {
        const int tt = x / LPG, q4 = x % LPG;
        float* src = dvr + tt * YS + q4;
        const int64_t tokc = tokc_base + (t_lo + s_lo + tt) * a.H;
        *reinterpret_cast<float4*>(A.dv_part + ((int64_t)p * A.rows_c + tokc) * dv + sl * SW +
                                   q4 * 4) = make_float4(src[0], src[LPG], src[2 * LPG], src[3 * LPG]);
        src[0] = 0.f;
        src[LPG] = 0.f;
        src[2 * LPG] = 0.f;
        src[3 * LPG] = 0.f;
      }
      for (int x = tid; x < ns * a.R; x += NT) {
        const int tt = x / a.R, k = x - tt * a.R;
        const int64_t tokc = tokc_base + (t_lo + s_lo + tt) * a.H;
        pr[tokc * a.R + k] = pdq[x];
        pdq[x] = 0.0f;
      }
      for (int x = tid; x < ns * a.W; x += NT) {
        const int tt = x / a.W, k = x - tt * a.W;
        const int64_t tokc = tokc_base + (t_lo + s_lo + tt) * a.H;
        pw[tokc * a.W + k] = pdc[x];
        pdc[x] = make_float2(0.0f, 0.0f);
      }
      // the next sub-round's staging writes only dys / vs / gab, which nothing reads now
    }
  }
}

// ---------------------------------------------------------------------------
// Per token: sum the slices' partial dots and the parts' d_v in a fixed order,
// then d_k = beta dc, d_beta = sum_k k dc, d_alpha = sum_k (1 - beta k) gm.
// One wavefront per token row of the chunk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__global__ __launch_bounds__(256) void back_reduce_kernel(BackStreamArgs A) {
  const ScanBackArgs& a = A.s;
  // one row per wavefront (uniform, so the index arithmetic is scalar); a chunk's
  // rows fit 32 bits
  const uint32_t row32 =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int64_t row = row32;
  if (row >= A.rows_c) return;
  const int lane = threadIdx.x & 63;
  const uint32_t bt = row32 / (uint32_t)a.H;
  const int h = (int)(row32 - bt * (uint32_t)a.H);
  const uint32_t b = bt / (uint32_t)A.Tc;
  const uint32_t t = bt - b * (uint32_t)A.Tc;
  const int64_t tok = ((int64_t)b * a.T + A.t0 + t) * a.H + h;
  const float be = a.beta[tok];
  float db = 0.0f, da = 0.0f;
  for (int k = lane; k < a.W; k += 64) {
    float dc = 0.0f, gm = 0.0f;
#pragma unroll 8  // the planes' loads go out together; the sums keep their order
    for (int u = 0; u < A.S * A.parts; ++u) {
      const float2 x = A.pw[((int64_t)u * A.rows_c + row) * a.W + k];
      dc += x.x;
      gm += x.y;
    }
    const float kw = a.wt_w[tok * a.W + k];
    a.g_wt_w[tok * a.W + k] = be * dc;
    db += kw * dc;
    da += (1.0f - be * kw) * gm;
  }
  db = wave_sum(db);
  da = wave_sum(da);
  if (lane == 0) {
    a.g_alpha[tok] = da;
    a.g_beta[tok] = db;
  }
  for (int k = lane; k < a.R; k += 64) {
    float dq = 0.0f;
#pragma unroll 8
    for (int u = 0; u < A.S * A.parts; ++u) dq += A.pr[((int64_t)u * A.rows_c + row) * a.R + k];
    a.g_wt_r[tok * a.R + k] = dq;
  }
  const int dv = a.d_v;
  for (int q4 = lane; q4 < dv / 4; q4 += 64) {
    float4 sv = f4s(0.0f);
#pragma unroll 4
    for (int p = 0; p < A.parts; ++p) {
      const float4 o =
          *reinterpret_cast<const float4*>(A.dv_part + ((int64_t)p * A.rows_c + row) * dv + q4 * 4);
      sv.x += o.x;
      sv.y += o.y;
      sv.z += o.z;
      sv.w += o.w;
    }
    *reinterpret_cast<float4*>(a.g_v + tok * dv + q4 * 4) = sv;
  }
}

// d_norm_w[h] = sum over batch entries, then over token blocks, of the partials.
__global__ __launch_bounds__(256) void gamma_blocks_kernel(const float* __restrict__ part,
                                                           int64_t B, int32_t H, int32_t DV,
                                                           int32_t gblocks,
                                                           float* __restrict__ d_norm_w) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)H * DV) return;
  const int64_t h = e / DV, c = e - h * DV;
  // partials in (batch, block) order; the loads of 8 terms are issued together (the
  // sum keeps its order, so the result is the same bit for bit)
  float s = 0.0f;
  for (int64_t b = 0; b < B; ++b) {
    const float* pb = part + (b * H + h) * gblocks * DV + c;
#pragma unroll 8
    for (int q = 0; q < gblocks; ++q) s += pb[(int64_t)q * DV];
  }
  d_norm_w[e] = s;
}

template <int SW>
void launch_walk_sw(int fmt, dim3 grid, hipStream_t st, const BackStreamArgs& A) {
  if (fmt == LOG_F32)
    hipLaunchKernelGGL((stream_backward_kernel<kNT, SW, BQ_F32, LOG_F32>), grid, dim3(kNT), 0, st,
                       A);
  else if (fmt == LOG_FP8)
    hipLaunchKernelGGL((stream_backward_kernel<kNT, SW, BQ_Q, LOG_FP8>), grid, dim3(kNT), 0, st, A);
  else
    hipLaunchKernelGGL((stream_backward_kernel<kNT, SW, BQ_Q, LOG_INT4>), grid, dim3(kNT), 0, st,
                       A);
}

void launch_walk(int sw, int fmt, dim3 grid, hipStream_t st, const BackStreamArgs& A) {
  if (sw == 64)
    launch_walk_sw<64>(fmt, grid, st, A);
  else if (sw == 32)
    launch_walk_sw<32>(fmt, grid, st, A);
  else
    launch_walk_sw<16>(fmt, grid, st, A);
}

struct BackPlan {
  int SW, S, parts, GT, log2GT, rounds, gblocks;
  int64_t Tc;
};

int ilog2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

BackPlan back_plan(const sdm_dims& d) {
  BackPlan pl;
  const int64_t walks = d.B * (int64_t)d.H;
  pl.SW = d.d_v >= 32 ? 32 : d.d_v;
  // 256-byte column slices where at most 4 parts fill the grid (as the forward)
  if (d.d_v % 64 == 0 && walks * (d.d_v / 64) * 4 >= 256) pl.SW = 64;
  pl.S = d.d_v / pl.SW;
  const int gw = kNT / (pl.SW / 4);
  int parts = 1;
  while (walks * pl.S * parts < 256 && gw * parts * 2 <= kStreamMaxGT) parts *= 2;
  pl.parts = parts;
  pl.GT = gw * parts;
  pl.log2GT = ilog2i(pl.GT);
  // token chunk: bound the per-token buffers to ~2 GiB
  const int64_t per_tok = walks * ((int64_t)(d.W + d.R) * 8 + (int64_t)d.d_v * 4 +
                                   (int64_t)pl.S * parts * (d.W * 8 + d.R * 4) +
                                   (int64_t)parts * d.d_v * 4);
  int64_t tc = (2ll << 30) / per_tok;
  tc = tc < ROUND ? ROUND : (tc / ROUND) * ROUND;
  pl.Tc = d.T < tc ? d.T : tc;
  pl.rounds = (int)((pl.Tc + ROUND - 1) / ROUND);
  pl.gblocks = (int)((d.T + PREP_TOK - 1) / PREP_TOK);
  return pl;
}

struct BackLayout {
  size_t counts, offsets, totals, entries, dy, pw, pr, dv_part, gpart, total;
};

BackLayout back_layout(const sdm_dims& d, const BackPlan& pl) {
  const int64_t walks = d.B * (int64_t)d.H;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BackLayout L;
  size_t s = 0;
  L.counts = s;
  s += al((size_t)walks * pl.rounds * pl.GT * 4);
  L.offsets = s;
  s += al((size_t)walks * pl.GT * (pl.rounds + 1) * 4);
  L.totals = s;
  s += al((size_t)walks * pl.GT * 4);
  L.entries = s;
  s += al((size_t)walks * pl.Tc * (d.W + d.R) * 8);
  L.dy = s;
  s += al((size_t)walks * pl.Tc * d.d_v * 4);
  L.pw = s;
  s += al((size_t)pl.S * pl.parts * walks * pl.Tc * d.W * 8);
  L.pr = s;
  s += al((size_t)pl.S * pl.parts * walks * pl.Tc * d.R * 4);
  L.dv_part = s;
  s += al((size_t)pl.parts * walks * pl.Tc * d.d_v * 4);
  L.gpart = s;
  s += al((size_t)walks * pl.gblocks * d.d_v * 4);
  L.total = s;
  return L;
}

}  // namespace

int norm_backward_blocks(int64_t T) { return (int)((T + PREP_TOK - 1) / PREP_TOK); }

hipError_t launch_norm_backward(const ScanBackArgs& sa, float* dy, float* gpart, hipStream_t st) {
  BackStreamArgs A{};
  A.s = sa;
  A.dy = dy;
  A.gpart = gpart;
  A.t0 = 0;
  A.Tc = sa.T;
  A.gblocks = norm_backward_blocks(sa.T);
  A.pblocks = A.gblocks;
  const dim3 grid((unsigned)(sa.B * (int64_t)sa.H * A.pblocks));
  KernelTimer kt("back_prep", st);
  switch (sa.d_v) {
    case 16: hipLaunchKernelGGL(back_prep_kernel<16>, grid, dim3(256), 0, st, A); break;
    case 32: hipLaunchKernelGGL(back_prep_kernel<32>, grid, dim3(256), 0, st, A); break;
    case 64: hipLaunchKernelGGL(back_prep_kernel<64>, grid, dim3(256), 0, st, A); break;
    case 128: hipLaunchKernelGGL(back_prep_kernel<128>, grid, dim3(256), 0, st, A); break;
    case 256: hipLaunchKernelGGL(back_prep_kernel<256>, grid, dim3(256), 0, st, A); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gamma_blocks(const ScanBackArgs& sa, const float* gpart, float* d_norm_w,
                               hipStream_t st) {
  const int64_t n = (int64_t)sa.H * sa.d_v;
  KernelTimer kt("gamma_sum", st);
  hipLaunchKernelGGL(gamma_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     gpart, sa.B, sa.H, sa.d_v, norm_backward_blocks(sa.T), d_norm_w);
  return hipGetLastError();
}

// The backward has one slot-owner schedule: SDM_FLAG_SCAN_STREAM and
// SDM_FLAG_SCAN_TWO_PHASE both select it.
// The slot-owner reverse walk from ROUND tokens, unless the walks alone fill the chip
// (kDirectWalks): then one lock-step workgroup per walk is faster.
bool backward_uses_stream(const sdm_dims& d) {
  if (d.flags & SDM_FLAG_SCAN_DIRECT) return false;
  if (d.flags & (SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_TWO_PHASE)) return true;
  return d.T >= ROUND && d.B * d.H < kDirectWalks;
}

size_t stream_backward_workspace_bytes(const sdm_dims& d) {
  return back_layout(d, back_plan(d)).total;
}

hipError_t launch_stream_backward(const sdm_dims& d, const ScanBackArgs& sa, float* d_norm_w,
                                  void* ws, hipStream_t st) {
  const BackPlan pl = back_plan(d);
  const BackLayout L = back_layout(d, pl);
  char* base = static_cast<char*>(ws);
  const int64_t walks = sa.B * (int64_t)sa.H;

  StreamArgs k{};  // bucketing pre-passes
  k.idx_w = sa.idx_w;
  k.wt_w = sa.wt_w;
  k.idx_r = sa.idx_r;
  k.wt_r = sa.wt_r;
  k.counts = reinterpret_cast<int*>(base + L.counts);
  k.offsets = reinterpret_cast<int*>(base + L.offsets);
  k.totals = reinterpret_cast<int*>(base + L.totals);
  k.entries = reinterpret_cast<uint2*>(base + L.entries);
  k.B = sa.B;
  k.T = sa.T;
  k.H = sa.H;
  k.N = sa.N;
  k.W = sa.W;
  k.R = sa.R;
  k.d_v = sa.d_v;
  k.S = pl.S;
  k.parts = pl.parts;
  k.GT = pl.GT;
  k.log2GT = pl.log2GT;
  k.log2GW = ilog2i(pl.GT / pl.parts);

  BackStreamArgs A;
  A.s = sa;
  A.entries = k.entries;
  A.offsets = k.offsets;
  A.dy = reinterpret_cast<float*>(base + L.dy);
  A.pw = reinterpret_cast<float2*>(base + L.pw);
  A.pr = reinterpret_cast<float*>(base + L.pr);
  A.dv_part = reinterpret_cast<float*>(base + L.dv_part);
  A.gpart = reinterpret_cast<float*>(base + L.gpart);
  A.S = pl.S;
  A.parts = pl.parts;
  A.GT = pl.GT;
  A.gblocks = pl.gblocks;

  const int64_t nchunks = (sa.T + pl.Tc - 1) / pl.Tc;
  for (int64_t ci = nchunks - 1; ci >= 0; --ci) {
    k.t0 = ci * pl.Tc;
    k.Tc = sa.T - k.t0 < pl.Tc ? sa.T - k.t0 : pl.Tc;
    k.rounds = (int)((k.Tc + ROUND - 1) / ROUND);
    k.walk_entries = k.Tc * (sa.W + sa.R);
    hipError_t e = launch_stream_buckets(k, walks, true, st);
    if (e != hipSuccess) return e;

    A.t0 = k.t0;
    A.Tc = k.Tc;
    A.walk_entries = k.walk_entries;
    A.rows_c = sa.B * k.Tc * sa.H;
    A.rounds = k.rounds;
    A.pblocks = (int)((k.Tc + PREP_TOK - 1) / PREP_TOK);
    {
      const dim3 grid((unsigned)(walks * A.pblocks));
      KernelTimer kt("back_prep", st);
      switch (sa.d_v) {
        case 16: hipLaunchKernelGGL(back_prep_kernel<16>, grid, dim3(256), 0, st, A); break;
        case 32: hipLaunchKernelGGL(back_prep_kernel<32>, grid, dim3(256), 0, st, A); break;
        case 64: hipLaunchKernelGGL(back_prep_kernel<64>, grid, dim3(256), 0, st, A); break;
        case 128: hipLaunchKernelGGL(back_prep_kernel<128>, grid, dim3(256), 0, st, A); break;
        case 256: hipLaunchKernelGGL(back_prep_kernel<256>, grid, dim3(256), 0, st, A); break;
        default: return hipErrorInvalidValue;
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
      const dim3 grid((unsigned)(walks * pl.S * pl.parts));
      KernelTimer kt("stream_backward", st);
      launch_walk(pl.SW, sa.log_fmt, grid, st, A);
    }
    {
      KernelTimer kt("back_reduce", st);
      hipLaunchKernelGGL(back_reduce_kernel, dim3((unsigned)((A.rows_c + 3) / 4)), dim3(256), 0,
                         st, A);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d_norm_w) {
    const int64_t n = (int64_t)sa.H * sa.d_v;
    KernelTimer kt("gamma_sum", st);
    hipLaunchKernelGGL(gamma_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       A.gpart, sa.B, sa.H, sa.d_v, pl.gblocks, d_norm_w);
  }
  return hipGetLastError();
}

}  // namespace sdm
