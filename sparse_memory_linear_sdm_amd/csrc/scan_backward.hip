// Backward of the recurrent sparse scan and the norm/gate (steps 2-4 of the method
// in reverse) for training.
//
// The m.163.com article on arXiv 2607.07386 (section 八, memory-efficiency
// paragraph) trains with the sparse update applied in place and undone in
// backward, which needs the N x d state plus the T x W x d rows the writes
// overwrote.  The training forward (direct schedule, scan.hip) records those rows
// in a log; this kernel walks each (b, h) memory's tokens in reverse:
//   norm/gate:  s = (mean(y^2) + eps)^(-1/2), yhat = y s, u = d_out gamma gate,
//               dy = s (u - yhat mean(u yhat)), d_gate = d_out yhat gamma,
//               d_gamma += d_out yhat gate
//   read:       d_q[r] = <dy, M[r]>,  dM[r] += q[r] dy        (M after t's writes)
//   write:      with m the logged row, c = beta k, G = dM[i]:
//               d_v += c G,  dc = <G, v - alpha m>,  d_alpha += (1 - c) <G, m>,
//               d_k = beta dc,  d_beta += k dc,  dM[i] = alpha (1 - c) G,  M[i] = m
// The key-weighted rule (SDM_FLAG_DELTA_GDN) has its reverse walk in scan_slices.hip.
// The state comes back as M_0 bit for bit and dM as the gradient of M_0.
//
// One workgroup of 256 threads per walk, laid out like the direct forward: LPR =
// d_v/4 lanes per row (float4 each), G = 256/LPR row groups.  A token's read ids
// are distinct, and so are its write ids, so the groups never touch one row twice
// within a phase; barriers order the read phase, the write phase and the next
// token.  Every sum runs in a fixed order (group shuffles, then LDS in group
// order), so the gradients are bit-reproducible.
#include "sdm_internal.h"

namespace sdm {
namespace {

__device__ __forceinline__ float4 f4s(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Sum over the LPR lanes of one row group (xor butterfly: every lane gets the sum).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, LPR);
  return x;
}

template <int DV>
__global__ __launch_bounds__(256) void scan_backward_kernel(ScanBackArgs a) {
  constexpr int LPR = DV / 4;
  constexpr int G = 256 / LPR;
  constexpr int BQ = 8;           // rows a group keeps in flight
  __shared__ float4 red[G][LPR];  // per-group partial d_v of the token
  __shared__ float2 sab[G];       // per-group partial (d_alpha, d_beta)

  const int tid = threadIdx.x;
  const int li = tid % LPR;
  const int grp = tid / LPR;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.H;
  const int h = (int)(bh - b * a.H);
  float* M = a.state + bh * (int64_t)a.N * DV;
  float* dM = a.d_state + bh * (int64_t)a.N * DV;
  const float4 gam = a.norm_w ? reinterpret_cast<const float4*>(a.norm_w + (int64_t)h * DV)[li]
                              : f4s(1.0f);
  float4 dgam = f4s(0.0f);  // this lane's columns of d_gamma (kept by group 0)

  for (int64_t t = a.T - 1; t >= 0; --t) {
    const int64_t tok = (b * a.T + t) * a.H + h;
    // ---- norm and gate: every group derives dy for its own use ----
    const float4 y = reinterpret_cast<const float4*>(a.y_raw + tok * DV)[li];
    const float4 gt = reinterpret_cast<const float4*>(a.gate + tok * DV)[li];
    const float4 dout = reinterpret_cast<const float4*>(a.d_out + tok * DV)[li];
    const float s = rsqrtf(group_sum<LPR>(dot4(y, y)) / (float)DV + a.eps);
    const float4 yh = make_float4(y.x * s, y.y * s, y.z * s, y.w * s);
    const float4 u = make_float4(dout.x * gam.x * gt.x, dout.y * gam.y * gt.y,
                                 dout.z * gam.z * gt.z, dout.w * gam.w * gt.w);
    const float mu = group_sum<LPR>(dot4(u, yh)) / (float)DV;
    const float4 dy = make_float4(s * (u.x - yh.x * mu), s * (u.y - yh.y * mu),
                                  s * (u.z - yh.z * mu), s * (u.w - yh.w * mu));
    if (grp == 0) {
      reinterpret_cast<float4*>(a.g_gate + tok * DV)[li] =
          make_float4(dout.x * yh.x * gam.x, dout.y * yh.y * gam.y, dout.z * yh.z * gam.z,
                      dout.w * yh.w * gam.w);
      dgam.x += dout.x * yh.x * gt.x;
      dgam.y += dout.y * yh.y * gt.y;
      dgam.z += dout.z * yh.z * gt.z;
      dgam.w += dout.w * yh.w * gt.w;
    }
    // ---- read (the state after token t's writes) ----
    const int32_t* ir = a.idx_r + tok * a.R;
    const float* wr = a.wt_r + tok * a.R;
    for (int k0 = grp; k0 < a.R; k0 += G * BQ) {  // distinct ids: batch the row loads
      int64_t rows[BQ];
      float4 m[BQ], g[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        rows[j] = ir[k < a.R ? k : k0];
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        m[j] = reinterpret_cast<const float4*>(M + rows[j] * DV)[li];
        g[j] = reinterpret_cast<const float4*>(dM + rows[j] * DV)[li];
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        if (k >= a.R) break;
        const float dq = group_sum<LPR>(dot4(dy, m[j]));
        if (li == 0) a.g_wt_r[tok * a.R + k] = dq;
        const float q = wr[k];
        float4 n = g[j];
        n.x = fmaf(q, dy.x, n.x);
        n.y = fmaf(q, dy.y, n.y);
        n.z = fmaf(q, dy.z, n.z);
        n.w = fmaf(q, dy.w, n.w);
        reinterpret_cast<float4*>(dM + rows[j] * DV)[li] = n;
      }
    }
    __syncthreads();  // the write phase below may take rows this phase updated
    // ---- write, undone ----
    const float al = a.alpha[tok];
    const float be = a.beta[tok];
    const float4 vv = reinterpret_cast<const float4*>(a.v + tok * DV)[li];
    const int32_t* iw = a.idx_w + tok * a.W;
    const float* ww = a.wt_w + tok * a.W;
    float4 dv = f4s(0.0f);
    float da = 0.0f, db = 0.0f;
    for (int k0 = grp; k0 < a.W; k0 += G * BQ) {
      int64_t rows[BQ];
      float4 ms[BQ], gs[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        rows[j] = iw[k < a.W ? k : k0];
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        const int kk = k < a.W ? k : k0;
        ms[j] = log_load(a.log, a.log_scale, a.log_fmt, tok * a.W + kk, DV, li);
        gs[j] = reinterpret_cast<const float4*>(dM + rows[j] * DV)[li];
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        if (k >= a.W) break;
        const int64_t row = rows[j];
        const float kw = ww[k];
        const float c = be * kw;
        const float oc = 1.0f - c;
        const float4 m = ms[j];
        float4* pg = reinterpret_cast<float4*>(dM + row * DV) + li;
        const float4 g = gs[j];
        dv.x = fmaf(c, g.x, dv.x);
        dv.y = fmaf(c, g.y, dv.y);
        dv.z = fmaf(c, g.z, dv.z);
        dv.w = fmaf(c, g.w, dv.w);
        const float4 e = make_float4(vv.x - al * m.x, vv.y - al * m.y, vv.z - al * m.z,
                                     vv.w - al * m.w);
        const float dc = group_sum<LPR>(dot4(g, e));
        da += oc * group_sum<LPR>(dot4(g, m));
        db += kw * dc;
        if (li == 0) a.g_wt_w[tok * a.W + k] = be * dc;
        const float f = al * oc;
        *pg = make_float4(f * g.x, f * g.y, f * g.z, f * g.w);
        reinterpret_cast<float4*>(M + row * DV)[li] = m;
      }
    }
    red[grp][li] = dv;
    if (li == 0) sab[grp] = make_float2(da, db);
    __syncthreads();
    if (grp == 0) {
      float4 sv = red[0][li];
      float2 ab = sab[0];
      for (int q = 1; q < G; ++q) {
        const float4 o = red[q][li];
        sv.x += o.x;
        sv.y += o.y;
        sv.z += o.z;
        sv.w += o.w;
        ab.x += sab[q].x;
        ab.y += sab[q].y;
      }
      reinterpret_cast<float4*>(a.g_v + tok * DV)[li] = sv;
      if (li == 0) {
        a.g_alpha[tok] = ab.x;
        a.g_beta[tok] = ab.y;
      }
    }
    __syncthreads();  // red / sab reuse, and the next token's reads see this restore
  }
  if (grp == 0) reinterpret_cast<float4*>(a.g_gamma_part + bh * DV)[li] = dgam;
}

// d_norm_w[h] = sum over batch entries of the walks' partials, in batch order.
__global__ __launch_bounds__(256) void gamma_sum_kernel(const float* __restrict__ part,
                                                        int64_t B, int32_t H, int32_t DV,
                                                        float* __restrict__ d_norm_w) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)H * DV) return;
  float s = 0.0f;
  for (int64_t b = 0; b < B; ++b) s += part[b * H * DV + e];
  d_norm_w[e] = s;
}

}  // namespace

hipError_t launch_scan_backward(const ScanBackArgs& a, float* d_norm_w, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H));
  {
    KernelTimer kt("scan_backward", s);
    switch (a.d_v) {
#define SDM_BACK(DVV) \
  hipLaunchKernelGGL((scan_backward_kernel<DVV>), grid, dim3(256), 0, s, a);
      case 16: SDM_BACK(16) break;
      case 32: SDM_BACK(32) break;
      case 64: SDM_BACK(64) break;
      case 128: SDM_BACK(128) break;
      case 256: SDM_BACK(256) break;
#undef SDM_BACK
      default: return hipErrorInvalidValue;
    }
  }
  if (d_norm_w) {
    const int64_t n = (int64_t)a.H * a.d_v;
    KernelTimer kt("gamma_sum", s);
    hipLaunchKernelGGL(gamma_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a.g_gamma_part, a.B, a.H, a.d_v, d_norm_w);
  }
  return hipGetLastError();
}

}  // namespace sdm
