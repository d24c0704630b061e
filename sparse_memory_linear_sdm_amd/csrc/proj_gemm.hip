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

__device__ __forceinline__ void epilogue_store(const ProjDst& d, int64_t m, int c, float val) {
  const int h = c / d.P;
  const int p = c - h * d.P;
  const int n4 = 4 * d.n;
  const int64_t mh = m * d.H + h;
  if (p < n4) {
    d.scores[((m - d.scores_row0) * d.H + h) * n4 + p] = val;
  } else if (p < n4 + d.d_v) {
    d.v[mh * d.d_v + (p - n4)] = val;
  } else if (p < n4 + 2 * d.d_v) {
    float g = val;
    if (d.gate_act == SDM_GATE_SIGMOID) g = sigmoid_f(val);
    else if (d.gate_act == SDM_GATE_SILU) g = val * sigmoid_f(val);
    d.gate[mh * d.d_v + (p - n4 - d.d_v)] = g;
  } else if (p == n4 + 2 * d.d_v) {
    d.alpha[mh] = expf(-d.A[h] * softplus_f(val + d.b_dt[h]));
  } else {
    d.beta[mh] = sigmoid_f(val);
  }
}

// ---------------------------------------------------------------------------
// bf16 path: 128x128 block tile, K-step 32, 4 waves each owning 64x64 as 2x2
// MFMA 32x32x16 blocks.  LDS rows padded by 16 B to spread banks.
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;

__global__ __launch_bounds__(256) void proj_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp, int64_t row0, int64_t M,
    int Ncol, int K, ProjDst dst) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile_m = (int64_t)blockIdx.y * BM;   // local row within [0, M)
  const int tile_n = blockIdx.x * BN;

  floatx16 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // global -> LDS: each tile is 128 rows x 64 B = 512 chunks of 16 B
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = tid + it * 256;
      const int r = q >> 2;
      const int kc = (q & 3) * 8;
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      const int64_t gm = tile_m + r;
      if (gm < M && k0 + kc < K)
        va = *reinterpret_cast<const uint4*>(X + (row0 + gm) * (int64_t)K + k0 + kc);
      const int gn = tile_n + r;
      if (gn < Ncol && k0 + kc < K)
        vb = *reinterpret_cast<const uint4*>(Wp + (int64_t)gn * K + k0 + kc);
      *reinterpret_cast<uint4*>(As + r * LDK + kc) = va;
      *reinterpret_cast<uint4*>(Bs + r * LDK + kc) = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm * 64 + i * 32 + (lane & 31);
        const int rb = wn * 64 + i * 32 + (lane & 31);
        const int kq = kk + (lane >> 5) * 8;
        uint4 ua = *reinterpret_cast<const uint4*>(As + ra * LDK + kq);
        uint4 ub = *reinterpret_cast<const uint4*>(Bs + rb * LDK + kq);
        __builtin_memcpy(&af[i], &ua, 16);
        __builtin_memcpy(&bfr[i], &ub, 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // 32x32 output block layout: register r of lane l holds
  // row (r/4)*8 + (l/32)*4 + r%4, column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t lm = tile_m + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int c = tile_n + wn * 64 + j * 32 + (lane & 31);
        if (lm < M && c < Ncol) epilogue_store(dst, row0 + lm, c, acc[i][j][r]);
      }
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
    dim3 grid((Ncol + BN - 1) / BN, (unsigned)((rows + BM - 1) / BM));
    hipLaunchKernelGGL(proj_gemm_bf16_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_proj), row0,
                       rows, Ncol, K, dst);
  } else {
    dim3 grid((Ncol + 63) / 64, (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(proj_gemm_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(w_proj), row0, rows, Ncol, K, dst);
  }
  return hipGetLastError();
}

}  // namespace sdm
