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
//   3. rank the candidates by (exact fp64 score desc, slot id asc), keep `count`;
//   4. return the ids ascending with softmax weights of their scores.
//
// One wavefront per problem, everything in registers but a 256-bin histogram and
// small staging areas in LDS:
//  * a top-k is an exact selection by value bins (wave min/max, 256 equal-width
//    bins, the bin holding the k-th best refined at most three times, the rest
//    ranked exactly), then compaction and a register bitonic sort of the k
//    survivors;
//  * the candidates' fp32-rounded sums never decrease with their exact sums, so
//    they are binned on those and only the members of the last bin are ordered by
//    exact fp64 sum and id;
//  * all cross-lane traffic (reductions, scans, sorting exchanges) moves through
//    DPP and the permlane swaps, never through the LDS crossbar.
#include "sdm_internal.h"

namespace sdm {
namespace {

// ---------------------------------------------------------------------------
// Candidate table: for every count c in [1, 128] the pairs (r1, r2) with
// (r1+1)(r2+1) <= c, row by row, packed as r1 << 8 | r2.  Built at compile time.
// ---------------------------------------------------------------------------
constexpr int cand_count(int c) {
  int s = 0;
  for (int a = 1; a <= c; ++a) s += c / a;
  return s;
}
constexpr int cand_total() {
  int s = 0;
  for (int c = 1; c <= SDM_MAX_COUNT; ++c) s += cand_count(c);
  return s;
}
constexpr int kCandTotal = cand_total();

struct CandTable {
  uint16_t off[SDM_MAX_COUNT + 2];
  uint16_t rc[kCandTotal];
};

constexpr CandTable make_cand_table() {
  CandTable t{};
  int p = 0;
  t.off[0] = 0;
  t.off[1] = 0;
  for (int c = 1; c <= SDM_MAX_COUNT; ++c) {
    t.off[c] = (uint16_t)p;
    for (int r1 = 0; r1 < c; ++r1)
      for (int r2 = 0; (r1 + 1) * (r2 + 1) <= c; ++r2) t.rc[p++] = (uint16_t)(r1 << 8 | r2);
  }
  t.off[SDM_MAX_COUNT + 1] = (uint16_t)p;
  return t;
}

__device__ const CandTable kCand = make_cand_table();

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

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Cross-lane moves without the LDS crossbar: DPP within rows of 16 lanes
// (quad_perm, row shifts under bank masks, row rotation, row broadcasts) and the
// gfx950 permlane swaps across rows and halves of the wavefront.
// dpp<CTRL>(old, src): lane i gets src of the lane CTRL names, or `old` where that
// lane is outside the row or masked off.
template <int CTRL, int RM = 0xf, int BM = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, RM, BM, false);
}

// x of lane (this lane ^ M)
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if constexpr (M == 1) {
    return dpp<0xB1>(x, x);  // quad_perm(1,0,3,2)
  } else if constexpr (M == 2) {
    return dpp<0x4E>(x, x);  // quad_perm(2,3,0,1)
  } else if constexpr (M == 4) {
    const uint32_t t = dpp<0x104, 0xf, 0x5>(x, x);  // banks 0,2: row_shl 4
    return dpp<0x114, 0xf, 0xA>(t, x);              // banks 1,3: row_shr 4
  } else if constexpr (M == 8) {
    return dpp<0x128>(x, x);  // row_ror 8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
  }
}
// the same with a distance that is a constant after unrolling
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int m) {
  switch (m) {
    case 1: return xor_lane<1>(x);
    case 2: return xor_lane<2>(x);
    case 4: return xor_lane<4>(x);
    case 8: return xor_lane<8>(x);
    case 16: return xor_lane<16>(x);
    default: return xor_lane<32>(x);
  }
}
__device__ __forceinline__ float xor_lane(float x, int m) {
  return __uint_as_float(xor_lane(__float_as_uint(x), m));
}
__device__ __forceinline__ uint64_t xor_lane(uint64_t x, int m) {
  return ((uint64_t)xor_lane((uint32_t)(x >> 32), m) << 32) | xor_lane((uint32_t)x, m);
}
__device__ __forceinline__ double xor_lane(double x, int m) {
  return __longlong_as_double((long long)xor_lane((uint64_t)__double_as_longlong(x), m));
}

// Inclusive prefix over the wavefront: Hillis-Steele within rows (row_shr 1, 2, 4,
// 8), then the last lane of row 0 / 2 into rows 1 / 3 (row_bcast 15) and lane 31
// into rows 2, 3 (row_bcast 31).  `id` is the identity of `op`.
template <class F>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id, F op) {
  v = op(v, dpp<0x111>(id, v));
  v = op(v, dpp<0x112>(id, v));
  v = op(v, dpp<0x114>(id, v));
  v = op(v, dpp<0x118>(id, v));
  v = op(v, dpp<0x142, 0xa>(id, v));
  v = op(v, dpp<0x143, 0xc>(id, v));
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  return (int)wave_scan((uint32_t)x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// wave-uniform results (read from lane 63)
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

__device__ __forceinline__ float wave_min(float x) {
  const uint32_t r = wave_scan(__float_as_uint(x), 0x7f800000u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}
__device__ __forceinline__ float wave_max(float x) {
  const uint32_t r = wave_scan(__float_as_uint(x), 0xff800000u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}

// fp64 -> uint64 whose unsigned order is the double order (-0 folded onto +0).
__device__ __forceinline__ uint64_t ord64(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  if ((u << 1) == 0) u = 0;
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Exact order of the selections: larger key first, then smaller id.
__device__ __forceinline__ bool better(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Choose exactly `need` of the valid elements (bit q of `valid`, KPL per lane): the best
// under `better` on (key, id), where key(q) gives element q's 64-bit key (evaluated only
// for the few elements that reach the exact ranking).  fv[q] is a float that never
// decreases along that order; it is only used to bin.  Each round bins the remaining candidates into 256 equal-width
// bins over their [min, max]; the bins above the one holding the need-th best are taken,
// the bins below are dropped, and the rest continue.  Whatever remains after three rounds
// (or once few are left) is ranked exactly.  Binning is monotone, so the result is exact.
// hist: 256 words of LDS; tk/ti: LDS room for 64 (key, id) pairs.  RANGE: lo0 / hi0 are
// the wave's min / max of the valid elements already (used by the first round).
template <int KPL, bool RANGE, class KeyF>
__device__ __attribute__((always_inline)) uint32_t select_exact(const float (&fv)[KPL], KeyF key,
                                                                const uint32_t (&id)[KPL],
                                                                uint32_t valid, int need,
                                                                uint32_t* hist, uint64_t* tk,
                                                                uint32_t* ti, float lo0 = 0.0f,
                                                                float hi0 = 0.0f) {
  const int lane = lane_id();
  uint32_t sel = 0, cand = valid;
  int nc = wave_sum(__popc(cand));
  for (int round = 0; round < 3; ++round) {
    if (nc == need) return sel | cand;
    if (nc <= 32) break;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    if (RANGE && round == 0) {
      lo = lo0;
      hi = hi0;
    } else {
#pragma unroll
      for (int q = 0; q < KPL; ++q)
        if ((cand >> q) & 1u) {
          lo = fminf(lo, fv[q]);
          hi = fmaxf(hi, fv[q]);
        }
      lo = wave_min(lo);
      hi = wave_max(hi);
    }
    // any positive scale keeps the binning monotone, so the hardware reciprocal will do
    const float scale = 256.0f * __builtin_amdgcn_rcpf(hi - lo);
    if (!(hi > lo) || !(scale > 0.0f) || !(scale < __builtin_inff())) break;
    // bin = clamp(fv * scale - lo * scale, 0, 255): a correctly rounded fma is monotone
    // in fv, and the conversion of whatever med3 makes of a NaN stays in [0, 255]
    const float off = -lo * scale;
    int bin[KPL];
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      bin[q] = (int)__builtin_amdgcn_fmed3f(fmaf(fv[q], scale, off), 0.0f, 255.0f);
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0, 0, 0, 0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if ((cand >> q) & 1u) atomicAdd(&hist[bin[q]], 1u);
    __syncthreads();
    // lane l owns bins 255-4l (highest) .. 252-4l
    const uint4 hv = reinterpret_cast<const uint4*>(hist)[63 - lane];
    const int local = (int)(hv.x + hv.y + hv.z + hv.w);
    const int incl = wave_incl_scan(local);
    const int excl = incl - local;
    const int L = __ffsll((long long)__ballot(incl >= need)) - 1;
    int bstar = 0, rest = 0, inbin = 0;
    if (lane == L) {
      int acc = excl;
      const int c3 = (int)hv.w, c2 = (int)hv.z, c1 = (int)hv.y, c0 = (int)hv.x;
      if (acc + c3 >= need) {
        bstar = 255 - 4 * lane;
        inbin = c3;
      } else if ((acc += c3) + c2 >= need) {
        bstar = 254 - 4 * lane;
        inbin = c2;
      } else if ((acc += c2) + c1 >= need) {
        bstar = 253 - 4 * lane;
        inbin = c1;
      } else {
        acc += c1;
        bstar = 252 - 4 * lane;
        inbin = c0;
      }
      rest = need - acc;
    }
    bstar = __builtin_amdgcn_readlane(bstar, L);
    need = __builtin_amdgcn_readlane(rest, L);
    nc = __builtin_amdgcn_readlane(inbin, L);  // the candidates left for the next round
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KPL; ++q) {
      const bool c = (cand >> q) & 1u;
      sel |= (uint32_t)(c && bin[q] > bstar) << q;
      cand &= ~((uint32_t)(!(c && bin[q] == bstar)) << q);
    }
  }
  // Exact ranking of the remaining candidates.
  const int cl = __popc(cand);
  if (nc == need) return sel | cand;
  if (nc <= 64) {
    // compacted into LDS, each ranked by one lane against all of them, the verdicts
    // handed back through LDS
    const int p0 = wave_incl_scan(cl) - cl;
    int pos = p0;
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if ((cand >> q) & 1u) {
        tk[pos] = key(q);
        ti[pos] = id[q];
        ++pos;
      }
    __syncthreads();
    bool verdict = false;
    if (lane < nc) {
      const uint64_t ke = tk[lane];
      const uint32_t ie = ti[lane];
      int rank = 0;
      for (int u = 0; u < nc; ++u) rank += better(tk[u], ti[u], ke, ie) ? 1 : 0;
      verdict = rank < need;
    }
    __syncthreads();
    if (lane < nc) ti[lane] = verdict;
    __syncthreads();
    pos = p0;
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if ((cand >> q) & 1u) {
        if (ti[pos]) sel |= 1u << q;
        ++pos;
      }
    __syncthreads();
    return sel;
  }
  // More than 64 left (many equal or nearly equal keys): take the best remaining one
  // `need` times, each by a wave-wide reduction under `better`.  Ids are distinct, so
  // every round has one winner, which its lane moves from `cand` to `sel`.
  for (int r = 0; r < need; ++r) {
    bool has = false;
    uint64_t bk = 0;
    uint32_t bi = 0;
    int bq = 0;
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if ((cand >> q) & 1u) {
        const uint64_t k = key(q);
        if (!has || better(k, id[q], bk, bi)) {
          bk = k;
          bi = id[q];
          bq = q;
          has = true;
        }
      }
    uint64_t wk = bk;
    uint32_t wi = bi, wh = has;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t ok = xor_lane(wk, o);
      const uint32_t oi = xor_lane(wi, o), oh = xor_lane(wh, o);
      if (oh && (!wh || better(ok, oi, wk, wi))) {
        wk = ok;
        wi = oi;
        wh = 1;
      }
    }
    if (has && bk == wk && bi == wi) {
      sel |= 1u << bq;
      cand &= ~(1u << bq);
    }
  }
  return sel;
}

// Bitonic sort of NE = 64*EPL unsigned keys (element e = lane + 64*r in v[r]) so
// that larger keys come first.  Keys are distinct except for equal padding keys, so
// each exchange takes the partner's key exactly when it is larger and this position
// keeps the larger of the pair, or smaller and this position keeps the smaller.
template <int EPL, class K>
__device__ __attribute__((always_inline)) void bitonic_desc(K (&v)[EPL]) {
  const int lane = lane_id();
  constexpr int NE = 64 * EPL;
#pragma unroll
  for (int size = 2; size <= NE; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {  // partner in the same lane
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int e = lane + 64 * r;
          const int pr = r ^ (stride >> 6);
          if (pr > r) {
            const bool desc = (e & size) == 0;
            const K lo = v[r], hi = v[pr];
            const bool sw = (hi > lo) == desc;
            v[r] = sw ? hi : lo;
            v[pr] = sw ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int e = lane + 64 * r;
          const K o = xor_lane(v[r], stride);
          const bool desc = (e & size) == 0;
          const bool lower = (e & stride) == 0;
          // in a descending run the lower position keeps the larger key
          const bool keep_max = (desc == lower);
          v[r] = ((o > v[r]) == keep_max) ? o : v[r];
        }
      }
    }
  }
}

// Best k (<= 128) of the n values of one half, by (value desc, index asc).
// Writes the sorted survivors to val[0..k) / idx[0..k) (LDS).  A half whose values all
// tie has the closed form indices 0..k-1 (the exact ranking would compare every pair);
// returns whether that was the case.
template <int KPL>
__device__ __attribute__((always_inline)) bool half_topk(const float* __restrict__ src, int n, int k, uint32_t* hist,
                          uint64_t* stage, float* val, uint32_t* idx) {
  const int lane = lane_id();
  uint32_t key[KPL];
  float fv[KPL];
  uint64_t ek[KPL];
  uint32_t ei[KPL];
  uint32_t valid = 0;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int i = lane * KPL + q;
    const bool ok = i < n;
    fv[q] = ok ? src[i] : 0.0f;
    key[q] = ok ? ord32(fv[q]) : 0u;
    ek[q] = key[q];
    ei[q] = (uint32_t)i;
    valid |= (uint32_t)ok << q;
  }
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < KPL; ++q)
    if ((valid >> q) & 1u) {
      lo = fminf(lo, fv[q]);
      hi = fmaxf(hi, fv[q]);
    }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lo == hi) {  // every value ties (an all-zero input row): indices 0..k-1
    for (int e = lane; e < k; e += 64) {
      val[e] = lo;
      idx[e] = (uint32_t)e;
    }
    __syncthreads();
    return true;
  }
  uint64_t* tk = stage;
  uint32_t* ti = reinterpret_cast<uint32_t*>(stage + 64);
  const uint32_t sel = select_exact<KPL, true>(fv, [&](int q) { return ek[q]; }, ei, valid, k,
                                               hist, tk, ti, lo, hi);
  const int sel_local = __popc(sel);
  int pos = wave_incl_scan(sel_local) - sel_local;
#pragma unroll
  for (int q = 0; q < KPL; ++q)
    if ((sel >> q) & 1u) {
      const uint32_t i = (uint32_t)(lane * KPL + q);
      stage[pos++] = ((uint64_t)key[q] << 32) | (0xffffffffu - i);
    }
  __syncthreads();
  if (k <= 64) {
    uint64_t v[1] = {lane < k ? stage[lane] : 0ull};
    bitonic_desc<1>(v);
    if (lane < k) {
      val[lane] = unord32((uint32_t)(v[0] >> 32));
      idx[lane] = 0xffffffffu - (uint32_t)v[0];
    }
  } else {
    uint64_t v[2] = {stage[lane], lane + 64 < k ? stage[lane + 64] : 0ull};
    bitonic_desc<2>(v);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = lane + 64 * r;
      if (e < k) {
        val[e] = unord32((uint32_t)(v[r] >> 32));
        idx[e] = 0xffffffffu - (uint32_t)v[r];
      }
    }
  }
  __syncthreads();
  return false;
}

// Combine the two sorted top-k lists into the best `count` slots; KPC candidates
// per lane.  Writes ascending ids and softmax weights to oi / ow.
template <int KPC>
__device__ __attribute__((always_inline)) void combine(int n, int k, int count, const float* av, const uint32_t* ai,
                        const float* bv, const uint32_t* bi, uint32_t* hist, uint64_t* stage,
                        int32_t* __restrict__ oi, float* __restrict__ ow) {
  const int lane = lane_id();
  const int c0 = kCand.off[count];
  const int nc = kCand.off[count + 1] - c0;
  float fa[KPC], fb[KPC], fv[KPC];
  uint32_t id[KPC];
  uint32_t valid = 0;
#pragma unroll
  for (int q = 0; q < KPC; ++q) {
    const int c = lane * KPC + q;
    const uint32_t rc = c < nc ? kCand.rc[c0 + c] : 0xffffu;
    const int r1 = (int)(rc >> 8), r2 = (int)(rc & 255u);
    const bool ok = c < nc && r1 < k && r2 < k;
    fa[q] = ok ? av[r1] : 0.0f;
    fb[q] = ok ? bv[r2] : 0.0f;
    fv[q] = fa[q] + fb[q];  // fp32-rounded sum: never decreases with the exact one
    id[q] = ok ? ai[r1] * (uint32_t)n + bi[r2] : 0u;
    valid |= (uint32_t)ok << q;
  }
  // the exact sum of two fp32 values in fp64
  auto exact = [&](int q) { return (double)fa[q] + (double)fb[q]; };
  uint64_t* tk = stage;
  uint32_t* ti = reinterpret_cast<uint32_t*>(stage + 64);
  const uint32_t sel = select_exact<KPC, false>(
      fv, [&](int q) { return ord64(exact(q)); }, id, valid, count, hist, tk, ti);
  // compaction of the `count` survivors as (id, exact score)
  uint32_t* cid = reinterpret_cast<uint32_t*>(stage);
  double* csc = reinterpret_cast<double*>(stage + 64);  // after 128 ids
  const int sel_local = __popc(sel);
  int pos = wave_incl_scan(sel_local) - sel_local;
#pragma unroll
  for (int q = 0; q < KPC; ++q)
    if ((sel >> q) & 1u) {
      cid[pos] = id[q];
      csc[pos] = exact(q);
      ++pos;
    }
  __syncthreads();
  // sort survivors by id ascending (a descending sort of complemented ids)
  static_assert(SDM_MAX_HALF * SDM_MAX_HALF <= (1 << 20) && SDM_MAX_COUNT <= 128,
                "ids and positions must fit the 32-bit sort key");
  const int ne = count <= 64 ? 1 : 2;
  double smax = -__builtin_inf();
  for (int e = lane; e < count; e += 64) smax = fmax(smax, csc[e]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) smax = fmax(smax, xor_lane(smax, o));
  float wsum = 0.0f;
  // key: (id descending-complemented, position), +1 so that padding (0) sorts last;
  // ids < 2^20 and positions < 128
  auto sort_key = [&](int e) -> uint32_t {
    return e < count ? ((((0xFFFFFu - cid[e]) << 7) | (uint32_t)e) + 1u) : 0u;
  };
  if (ne == 1) {
    uint32_t v[1] = {sort_key(lane)};
    bitonic_desc<1>(v);
    const uint32_t kk = v[0] - 1u;
    float w = 0.0f;
    if (lane < count) w = expf((float)(csc[kk & 127u] - smax));
    wsum = w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wsum += xor_lane(wsum, o);
    if (lane < count) {
      oi[lane] = (int32_t)(0xFFFFFu - (kk >> 7));
      ow[lane] = w / wsum;
    }
  } else {
    uint32_t v[2] = {sort_key(lane), sort_key(lane + 64)};
    bitonic_desc<2>(v);
    float w[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = lane + 64 * r;
      w[r] = e < count ? expf((float)(csc[(v[r] - 1u) & 127u] - smax)) : 0.0f;
    }
    wsum = w[0] + w[1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wsum += xor_lane(wsum, o);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = lane + 64 * r;
      if (e < count) {
        oi[e] = (int32_t)(0xFFFFFu - ((v[r] - 1u) >> 7));
        ow[e] = w[r] / wsum;
      }
    }
  }
}

// 64-bit staging words: exact-ranking room for 64 (key, id) pairs (96 words), the half
// top-k survivors (128 keys) or the combine's survivors (128 ids + 128 doubles).
constexpr int kStageWords = 192;

// Waves per SIMD to compile for: 8 (at most 64 VGPRs, which the instantiations for
// n <= 384 and counts whose candidates fit 5 per lane, W and R up to about 66, meet
// without spilling; 4.5 KB of LDS per wave lets 8 fit), else no bound.
constexpr int sel_waves(int kpl, int kpc) { return kpl <= 6 && kpc <= 5 ? 8 : 1; }

// One wavefront per (row, head, role).  LDS: histogram, staging, two top-k lists.
template <int KPL, int KPC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sel_waves(KPL, KPC)))) void select_kernel(const float* __restrict__ scores, int64_t rows,
                                                    int H, int n, int W, int R,
                                                    int64_t out_row0, int32_t* __restrict__ idx_w,
                                                    float* __restrict__ wt_w,
                                                    int32_t* __restrict__ idx_r,
                                                    float* __restrict__ wt_r) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ __attribute__((aligned(16))) uint64_t stage[kStageWords];
  __shared__ float tv[2][SDM_MAX_COUNT];
  __shared__ uint32_t ti[2][SDM_MAX_COUNT];

  const int64_t prob = blockIdx.x;
  const int role = (int)(prob & 1);  // 0 = write, 1 = read
  const int64_t rh = prob >> 1;
  const int64_t r = rh / H;
  const int h = (int)(rh - r * H);
  if (r >= rows) return;
  const int count = role ? R : W;
  const int k = count < n ? count : n;
  const float* half = scores + (r * H + h) * (int64_t)(4 * n) + role * 2 * n;
  const bool flat0 = half_topk<KPL>(half, n, k, hist, stage, tv[0], ti[0]);
  const bool flat1 = half_topk<KPL>(half + n, n, k, hist, stage, tv[1], ti[1]);
  const int64_t base = ((out_row0 + r) * H + h) * (int64_t)count;
  int32_t* const oi = (role ? idx_r : idx_w) + base;
  float* const ow = (role ? wt_r : wt_w) + base;
  if (flat0 && flat1) {  // every slot score ties: slots 0..count-1, equal weights
    for (int e = lane_id(); e < count; e += 64) {
      oi[e] = e;
      ow[e] = 1.0f / (float)count;
    }
    return;
  }
  combine<KPC>(n, k, count, tv[0], ti[0], tv[1], ti[1], hist, stage, oi, ow);
}

template <int KPL>
hipError_t launch_kpl(const float* scores, int64_t rows, int H, int n, int W, int R,
                      int64_t out_row0, int32_t* idx_w, float* wt_w, int32_t* idx_r,
                      float* wt_r, hipStream_t s) {
  const int maxc = W > R ? W : R;
  const int nc = cand_count(maxc);
  const int kpc = (nc + 63) / 64;
  const dim3 grid((unsigned)(rows * H * 2));
  KernelTimer kt("select", s);
#define SDM_SEL_LAUNCH(KPC)                                                                   \
  hipLaunchKernelGGL((select_kernel<KPL, KPC>), grid, dim3(64), 0, s, scores, rows, H, n, W, R, \
                     out_row0, idx_w, wt_w, idx_r, wt_r)
  if (kpc <= 1) SDM_SEL_LAUNCH(1);
  else if (kpc <= 2) SDM_SEL_LAUNCH(2);
  else if (kpc <= 5) SDM_SEL_LAUNCH(5);
  else SDM_SEL_LAUNCH(11);
#undef SDM_SEL_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const sdm_dims& d, const float* scores, int64_t rows, int64_t out_row0,
                         int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                         hipStream_t s) {
  const int kpl = (d.n + 63) / 64;
#define SDM_KPL(K) \
  return launch_kpl<K>(scores, rows, d.H, d.n, d.W, d.R, out_row0, idx_w, wt_w, idx_r, wt_r, s)
  if (kpl <= 1) SDM_KPL(1);
  if (kpl <= 2) SDM_KPL(2);
  if (kpl <= 4) SDM_KPL(4);
  if (kpl <= 6) SDM_KPL(6);
  if (kpl <= 8) SDM_KPL(8);
  SDM_KPL(16);
#undef SDM_KPL
}

}  // namespace sdm
