// Projection GEMM of the SDM selection pass with the gate epilogue.
//
// Y = x W_proj^T (one dense contraction for every projection of every head:
// "Sparse Delta Memory" summary on paper.rainbus.top, method paragraph, step 1,
// W_k, W_q in R^{d x 2 sqrt(N)}; steps 2 and 4 for W_a, W_b and the gate vector).
// Both operands are K-contiguous, so the bf16 path feeds MFMA 32x32x16 tiles
// straight from LDS.  The epilogue routes each column of a head's P-column block:
//   [0, 4n)            half-scores          -> scores (fp32)
//   [4n, 4n+d_v)       value v              -> v
//   [4n+d_v, 4n+2d_v)  gate pre-activation  -> gate = act(.)
//   4n+2d_v            a  -> alpha = exp(-A softplus(a + b_dt))   (step 2)
//   4n+2d_v+1          b  -> beta  = sigmoid(b)
#include "sdm_internal.h"

namespace sdm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// Destination of one output column: element (m, c) goes to base[m * stride],
// transformed by `kind` (0 copy, 1 sigmoid, 2 silu, 3 forget gate, 4 input gate).
struct ColDst {
  float* base;
  int64_t stride;
  int kind;
  float A, bdt;
};

__device__ __forceinline__ ColDst column_dst(const ProjDst& d, int c) {
  const int h = c / d.P;
  const int p = c - h * d.P;
  const int n4 = 4 * d.n;
  ColDst o;
  o.A = 0.0f;
  o.bdt = 0.0f;
  if (p < n4) {  // half-scores, rows relative to the staging buffer's first row
    o.base = d.scores + (-d.scores_row0 * d.H + h) * n4 + p;
    o.stride = (int64_t)d.H * n4;
    o.kind = 0;
  } else if (p < n4 + 2 * d.d_v) {
    const bool is_v = p < n4 + d.d_v;
    o.base = (is_v ? d.v + (p - n4) : d.gate + (p - n4 - d.d_v)) + (int64_t)h * d.d_v;
    o.stride = (int64_t)d.H * d.d_v;
    o.kind = is_v ? 0 : (d.gate_act == SDM_GATE_SIGMOID ? 1 : d.gate_act == SDM_GATE_SILU ? 2 : 0);
  } else {
    const bool is_a = p == n4 + 2 * d.d_v;
    o.base = (is_a ? d.alpha : d.beta) + h;
    o.stride = d.H;
    o.kind = is_a ? 3 : 4;
    if (is_a) {
      o.A = d.A[h];
      o.bdt = d.b_dt[h];
    }
  }
  return o;
}

__device__ __forceinline__ float column_value(const ColDst& o, float val) {
  switch (o.kind) {
    case 1: return sigmoid_f(val);
    case 2: return val * sigmoid_f(val);
    case 3: return expf(-o.A * softplus_f(val + o.bdt));
    case 4: return sigmoid_f(val);
    default: return val;
  }
}

// Store through a ColDst; rows beyond M and columns beyond Ncol are skipped.
__device__ __forceinline__ void epilogue_store(const ProjDst& d, int64_t m, int c, float val) {
  const ColDst o = column_dst(d, c);
  o.base[m * o.stride] = column_value(o, val);
}

// ---------------------------------------------------------------------------
// bf16 path: 256x256 block tile, K-step 64, 8 waves (2 x 4) each owning 128x64
// as 4x2 MFMA 32x32x16 blocks (each A fragment feeds 2 MFMAs, each B fragment 4).
// The next K-tile is fetched into registers while the current one is multiplied
// out of LDS (double-buffered, one barrier per K-step).  LDS rows are padded by
// 16 B.  Tiles are handed out XCD by XCD in groups of GROUP_M row tiles, so the
// blocks resident on one XCD share A and B slices through its L2.  The epilogue
// goes through LDS so that every store writes a 16-byte row segment.
// ---------------------------------------------------------------------------
// Tile shape: WM x WN waves, each owning FM x FN MFMA 32x32 blocks; BK columns of K
// per pipeline stage.
template <int WM_, int WN_, int FM_, int FN_, int BK_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, FM = FM_, FN = FN_;
  static constexpr int BM = WM * FM * 32, BN = WN * FN * 32, BK = BK_, LDK = BK + 8;
  static constexpr int NTH = WM * WN * 64;
  static constexpr int CPR = BK / 8;                  // 16-byte chunks per tile row
  static constexpr int A_CHUNKS = BM * BK / 8 / NTH;  // 16-byte chunks per thread per K-tile
  static constexpr int B_CHUNKS = BN * BK / 8 / NTH;
  static constexpr int A_BYTES = BM * LDK * 2, B_BYTES = BN * LDK * 2;
  static constexpr int LDS = 2 * (A_BYTES + B_BYTES);  // double-buffered A and B
  static_assert(A_CHUNKS * NTH * 8 == BM * BK && B_CHUNKS * NTH * 8 == BN * BK, "even split");
  static_assert(LDS >= WM * WN * 32 * 36 * 4, "epilogue patches fit in the tile buffers");
};
using BigTile = Tile<2, 4, 4, 2, 64>;     // 256 x 256, 8 waves of 128 x 64
// 64 x 64, 4 waves of 32 x 32, for few rows (decoding); the longer K-step halves the
// steps of each workgroup's serial K loop while two workgroups still fit a CU's LDS
using SmallTile = Tile<2, 2, 1, 1, 128>;
constexpr int GROUP_M = 4;
constexpr int NXCD = 8;

// XCD-aware grouped tile order: consecutive workgroups go to different XCDs, so
// each XCD gets a contiguous range of tiles, walked GROUP_M row tiles at a time.
// Returns false for the padding blocks of the grid.
template <int BM, int BN>
__device__ __forceinline__ bool tile_of_block(int64_t M, int Ncol, int64_t& tile_m, int& tile_n) {
  const int ntn = (Ncol + BN - 1) / BN;
  const int64_t ntm = (M + BM - 1) / BM;
  const int64_t total = ntm * ntn;
  const int64_t per_xcd = (total + NXCD - 1) / NXCD;
  const int64_t t = (int64_t)(blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  if (t >= total) return false;
  const int64_t grp = t / ((int64_t)GROUP_M * ntn);
  const int64_t first_m = grp * GROUP_M;
  const int gm_rows = (int)min<int64_t>(GROUP_M, ntm - first_m);
  const int64_t in_grp = t - grp * GROUP_M * ntn;
  tile_m = (first_m + in_grp % gm_rows) * BM;  // local row within [0, M)
  tile_n = (int)(in_grp / gm_rows) * BN;
  return true;
}

// Epilogue through LDS: each wave writes one 32x32 block at a time into a private
// padded LDS patch (32 rows of 36 floats; register r of lane l of a 32x32 MFMA
// block holds row (r/4)*8 + (l/32)*4 + r%4, column l%32), then every lane stores
// 4-column row segments: one 16-byte store where the 4 columns are plain copies
// into consecutive addresses, else one routed store per column.  `lds` is free
// (every wave is past its last read of the tile buffers) and holds 32*36 floats
// per wave.
template <int FM, int FN, int WN>
__device__ __forceinline__ void epilogue(floatx16 (&acc)[FM][FN], float* lds, int64_t tile_m,
                                         int tile_n, int64_t row0, int64_t M, int Ncol,
                                         const ProjDst& dst) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  float* patch = lds + wave * (32 * 36);
  const int sr = lane >> 3;        // row within an 8-row group
  const int sc = (lane & 7) * 4;   // first of this lane's 4 columns
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cb = tile_n + wn * FN * 32 + j * 32;  // first column of the block
    // this lane's 4 columns: contiguous float4 destination if all are plain copies
    // of one region of one head
    const int c0 = cb + sc;
    ColDst od[4];
    bool vec = c0 + 3 < Ncol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      od[e] = column_dst(dst, min(c0 + e, Ncol - 1));
      vec = vec && od[e].kind == 0 && od[e].stride == od[0].stride &&
            od[e].base == od[0].base + e;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        patch[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * 36 + (lane & 31)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = q * 8 + sr;
        const int64_t lm = tile_m + wm * FM * 32 + i * 32 + rr;
        const float4 v = *reinterpret_cast<const float4*>(patch + rr * 36 + sc);
        if (lm < M) {
          if (vec) {
            *reinterpret_cast<float4*>(od[0].base + (row0 + lm) * od[0].stride) = v;
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c0 + e < Ncol) od[e].base[(row0 + lm) * od[e].stride] = column_value(od[e], vv[e]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <class TL>
__global__ __launch_bounds__(TL::NTH) void proj_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp, int64_t row0, int64_t M,
    int Ncol, int K, ProjDst dst) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, LDK = TL::LDK, NTH = TL::NTH;
  constexpr int CPR = TL::CPR, A_CHUNKS = TL::A_CHUNKS, B_CHUNKS = TL::B_CHUNKS;
  constexpr int FM = TL::FM, FN = TL::FN;
  __shared__ __attribute__((aligned(16))) char smem[TL::LDS];
  auto As = [&](int buf) {
    return reinterpret_cast<uint16_t*>(smem + buf * (TL::A_BYTES + TL::B_BYTES));
  };
  auto Bs = [&](int buf) {
    return reinterpret_cast<uint16_t*>(smem + buf * (TL::A_BYTES + TL::B_BYTES) + TL::A_BYTES);
  };

  int64_t tile_m;
  int tile_n;
  if (!tile_of_block<BM, BN>(M, Ncol, tile_m, tile_n)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int it = 0; it < A_CHUNKS; ++it) {
      const int q = tid + it * NTH;
      const int r = q / CPR, kc = (q % CPR) * 8;
      const int64_t gm = tile_m + r;
      ra[it] = (gm < M && k0 + kc < K)
                   ? *reinterpret_cast<const uint4*>(X + (row0 + gm) * (int64_t)K + k0 + kc)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < B_CHUNKS; ++it) {
      const int q = tid + it * NTH;
      const int r = q / CPR, kc = (q % CPR) * 8;
      const int gn = tile_n + r;
      rb[it] = (gn < Ncol && k0 + kc < K)
                   ? *reinterpret_cast<const uint4*>(Wp + (int64_t)gn * K + k0 + kc)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int it = 0; it < A_CHUNKS; ++it) {
      const int q = tid + it * NTH;
      *reinterpret_cast<uint4*>(&As(buf)[(q / CPR) * LDK + (q % CPR) * 8]) = ra[it];
    }
#pragma unroll
    for (int it = 0; it < B_CHUNKS; ++it) {
      const int q = tid + it * NTH;
      *reinterpret_cast<uint4*>(&Bs(buf)[(q / CPR) * LDK + (q % CPR) * 8]) = rb[it];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  int cur = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) fetch(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const int kq = kk + (lane >> 5) * 8;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 u = *reinterpret_cast<const uint4*>(
            &As(cur)[(wm * FM * 32 + i * 32 + (lane & 31)) * LDK + kq]);
        __builtin_memcpy(&af[i], &u, 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 u = *reinterpret_cast<const uint4*>(
            &Bs(cur)[(wn * FN * 32 + j * 32 + (lane & 31)) * LDK + kq]);
        __builtin_memcpy(&bfr[j], &u, 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) stash(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  epilogue<FM, FN, TL::WN>(acc, reinterpret_cast<float*>(smem), tile_m, tile_n, row0, M, Ncol,
                           dst);
}

// ---------------------------------------------------------------------------
// bf16 path for K a multiple of 64: the same 256x256 tile and 8-wave layout, its
// operands brought into LDS by direct global->LDS loads (16 bytes per lane) instead
// of through registers, in two stages of K = 64.  A wave's load fills 1 KB of LDS at
// consecutive addresses, 8 tile rows of 128 bytes; lane l fetches the 16-byte chunk
// that lands at row l/8, slot l%8, i.e. chunk (l%8) ^ ((row >> 1) & 7) of that row.
// This XOR spreads the MFMA fragment reads (16 lanes read 16 rows at one chunk) over
// all LDS banks.  The loads are issued by inline assembly so that the compiler's
// wait-count pass, which cannot tell the two stages apart, does not wait for the
// stage in flight; the kernel waits for exactly the stage it is about to read, and
// synchronises with a bare barrier (no memory fence, which would also wait for it).
// The MFMA sequence per output is the one of proj_gemm_bf16_kernel: same results.
// ---------------------------------------------------------------------------
constexpr int DMA_BK = 64;

__global__ __launch_bounds__(512) void proj_gemm_bf16_dma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp, int64_t row0, int64_t M,
    int Ncol, int K, ProjDst dst) {
  constexpr int BM = 256, BN = 256, BK = DMA_BK, FM = 4, FN = 2, WN = 4;
  constexpr int ROWB = BK * 2;               // 128 bytes per tile row per stage
  constexpr int NI = BM * ROWB / 1024 / 8;   // loads per wave per operand per stage (4)
  constexpr int A_BYTES = BM * ROWB, ST_BYTES = (BM + BN) * ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * ST_BYTES];
  static_assert(2 * ST_BYTES >= 8 * 32 * 36 * 4, "epilogue patches fit in the stages");

  int64_t tile_m;
  int tile_n;
  if (!tile_of_block<BM, BN>(M, Ncol, tile_m, tile_n)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  auto swz = [](int r) { return (r >> 1) & 7; };

  // this lane's source rows: rows beyond M or Ncol read the last valid row instead
  // (their products are never stored)
  const uint16_t* ga[NI];
  const uint16_t* gb[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = (wave * NI + j) * 8 + lane / 8;
    const int c = (lane & 7) ^ swz(r);
    const int64_t gm = tile_m + r < M ? tile_m + r : M - 1;
    const int gn = tile_n + r < Ncol ? tile_n + r : Ncol - 1;
    ga[j] = X + (row0 + gm) * (int64_t)K + c * 8;
    gb[j] = Wp + (int64_t)gn * K + c * 8;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  // M0 holds the wave's LDS destination; one wait state between writing M0 and the
  // load that reads it
  auto dma = [](const uint16_t* g, uint32_t l) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(l))
                 : "memory", "m0");
  };
  auto issue = [&](int ks) {
    const uint32_t st = lds0 + (uint32_t)((ks & 1) * ST_BYTES);
    const int k0 = ks * BK;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      dma(ga[j] + k0, st + (wave * NI + j) * 1024);
      dma(gb[j] + k0, st + A_BYTES + (wave * NI + j) * 1024);
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / BK;
  issue(0);
  const int lr = lane & 31, hf = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    // stage ks is the only one in flight: wait for it, then the barrier makes every
    // wave's part visible and ensures every wave has finished reading stage ks - 1,
    // whose buffer the next issue overwrites
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ks + 1 < nk) issue(ks + 1);
    const char* st = smem + (ks & 1) * ST_BYTES;
#pragma unroll
    for (int sl = 0; sl < BK / 16; ++sl) {
      const int c = sl * 2 + hf;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * FM * 32 + i * 32 + lr;
        const uint4 u = *reinterpret_cast<const uint4*>(st + r * ROWB + ((c ^ swz(r)) << 4));
        __builtin_memcpy(&af[i], &u, 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * FN * 32 + j * 32 + lr;
        const uint4 u =
            *reinterpret_cast<const uint4*>(st + A_BYTES + r * ROWB + ((c ^ swz(r)) << 4));
        __builtin_memcpy(&bfr[j], &u, 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();  // the stages are free for the epilogue's patches
  epilogue<FM, FN, WN>(acc, reinterpret_cast<float*>(smem), tile_m, tile_n, row0, M, Ncol, dst);
}

// ---------------------------------------------------------------------------
// fp32 path (small layers): 64x64 tile, K-step 16, 4x4 outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void proj_gemm_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ Wp, int64_t row0, int64_t M, int Ncol,
    int K, ProjDst dst) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t tile_m = (int64_t)blockIdx.y * TM;
  const int tile_n = blockIdx.x * TN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    {
      const int r = tid >> 2, kc = (tid & 3) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = k0 + kc + e;
        const int64_t gm = tile_m + r;
        As[kc + e][r] = (gm < M && kk < K) ? X[(row0 + gm) * (int64_t)K + kk] : 0.0f;
        const int gn = tile_n + r;
        Bs[kc + e][r] = (gn < Ncol && kk < K) ? Wp[(int64_t)gn * K + kk] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = As[kk][ty * 4 + e];
        b[e] = Bs[kk][tx * 4 + e];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t lm = tile_m + ty * 4 + i;
      const int c = tile_n + tx * 4 + j;
      if (lm < M && c < Ncol) epilogue_store(dst, row0 + lm, c, acc[i][j]);
    }
}

}  // namespace

hipError_t launch_proj_gemm(const sdm_dims& d, const void* x, const void* w_proj, int64_t row0,
                            int64_t rows, const ProjDst& dst, hipStream_t s) {
  const int Ncol = d.H * dst.P;
  const int K = (int)d.d_model;
  if (d.in_dtype == SDM_DTYPE_BF16) {
    // the 256 x 256 tile when it gives the CUs enough workgroups, else 64 x 64
    const int64_t big = ((rows + BigTile::BM - 1) / BigTile::BM) *
                        ((Ncol + BigTile::BN - 1) / BigTile::BN);
    auto go = [&](auto tl) {
      using TL = decltype(tl);
      const int64_t tiles = ((rows + TL::BM - 1) / TL::BM) * ((Ncol + TL::BN - 1) / TL::BN);
      const dim3 grid((unsigned)(((tiles + NXCD - 1) / NXCD) * NXCD));
      KernelTimer kt("proj_gemm_bf16", s);
      hipLaunchKernelGGL(proj_gemm_bf16_kernel<TL>, grid, dim3(TL::NTH), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_proj),
                         row0, rows, Ncol, K, dst);
    };
    if (big >= 256 && K % DMA_BK == 0) {
      const dim3 grid((unsigned)(((big + NXCD - 1) / NXCD) * NXCD));
      KernelTimer kt("proj_gemm_bf16", s);
      hipLaunchKernelGGL(proj_gemm_bf16_dma_kernel, grid, dim3(512), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_proj),
                         row0, rows, Ncol, K, dst);
    } else if (big >= 256) {
      go(BigTile{});
    } else {
      go(SmallTile{});
    }
  } else {
    dim3 grid((Ncol + 63) / 64, (unsigned)((rows + 63) / 64));
    KernelTimer kt("proj_gemm_f32", s);
    hipLaunchKernelGGL(proj_gemm_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(w_proj), row0, rows, Ncol, K, dst);
  }
  return hipGetLastError();
}

}  // namespace sdm
