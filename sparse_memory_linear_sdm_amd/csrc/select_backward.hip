// Backward of the selection pass, down to the gradient of the projection output.
//
// Forward ("Sparse Delta Memory" summary on paper.rainbus.top, method paragraph,
// steps 1, 2 and 4; ai-paper-analysis.pages.dev, sections "步骤 1" and "步骤 2"):
//   weights w = softmax(s) over the selected slots' outer-sum scores
//   s_k = h1[i_k] + h2[j_k] (slot id i_k n + j_k), alpha = exp(-A softplus(a + b_dt)),
//   beta = sigmoid(b), gate = act(g), value v: all columns of Y = x W_proj^T.
// Reverse mode, per (token, head):
//   ds_k = w_k (dw_k - sum_l w_l dw_l);  dY[h1 i] = sum_{k: i_k = i} ds_k, dY[h2 j] alike;
//   dY[v] = dv;  dY[g] = dgate act'(g);  dY[a] = dalpha (-A alpha sigmoid(z)), z = a + b_dt;
//   dY[b] = dbeta beta (1 - beta);  dA += dalpha (-softplus(z) alpha);  db_dt += dY[a].
// SiLU output gate: dY[g] = dgate sigma(p) (1 + p (1 - sigma(p))) at the pre-activation p.
// The selected sets are piecewise constant in the scores: no gradient flows through
// the choice.  The forget pre-gate a is recomputed as x . W_a in fp32 (softplus and
// sigmoid of it are needed; the stored alpha alone loses them as alpha -> 1), and so
// is the SiLU gate's pre-activation (SiLU cannot be inverted from its output).
// Deterministic: the sums over repeated half indices run in slot order, the
// reductions over lanes and over tokens in fixed trees.
#include "sdm_internal.h"

namespace sdm {
namespace {

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float softplus_b(float z) {
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}
__device__ __forceinline__ float sigmoid_b(float z) { return 1.0f / (1.0f + expf(-z)); }

// x[m] . row of W_proj, fp32 accumulation: lane l takes elements l*8 + 512 u.
template <bool BF16>
__device__ float dot_row(const void* x, const void* w, int64_t xrow, int64_t wrow, int64_t d) {
  const int lane = threadIdx.x & 63;
  float acc = 0.0f;
  if (BF16) {
    const uint16_t* xp = static_cast<const uint16_t*>(x) + xrow * d;
    const uint16_t* wp = static_cast<const uint16_t*>(w) + wrow * d;
    for (int64_t k = (int64_t)lane * 8; k < d; k += 512) {
      const uint4 xa = *reinterpret_cast<const uint4*>(xp + k);
      const uint4 wa = *reinterpret_cast<const uint4*>(wp + k);
      const uint32_t xs[4] = {xa.x, xa.y, xa.z, xa.w}, ws[4] = {wa.x, wa.y, wa.z, wa.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(__uint_as_float(xs[q] << 16), __uint_as_float(ws[q] << 16), acc);
        acc = fmaf(__uint_as_float(xs[q] & 0xffff0000u), __uint_as_float(ws[q] & 0xffff0000u),
                   acc);
      }
    }
  } else {
    const float* xp = static_cast<const float*>(x) + xrow * d;
    const float* wp = static_cast<const float*>(w) + wrow * d;
    for (int64_t k = (int64_t)lane * 8; k < d; k += 512) {
#pragma unroll
      for (int q = 0; q < 8; q += 4) {
        const float4 xa = *reinterpret_cast<const float4*>(xp + k + q);
        const float4 wa = *reinterpret_cast<const float4*>(wp + k + q);
        acc = fmaf(xa.x, wa.x, acc);
        acc = fmaf(xa.y, wa.y, acc);
        acc = fmaf(xa.z, wa.z, acc);
        acc = fmaf(xa.w, wa.w, acc);
      }
    }
  }
  return wave_sum_f(acc);
}

// One role (write or read) of one (token, head): gradients of its half-score
// columns into the LDS row.  ids ascending, cnt <= 128 (two entries per lane).
__device__ __forceinline__ void role_backward(const int32_t* __restrict__ ids, const float* __restrict__ wt,
                              const float* __restrict__ dwt, int cnt, int n, float* row,
                              int o1, int o2, int* si, int* sj, float* sds) {
  const int lane = threadIdx.x & 63;
  float w[2], dw[2];
  int id[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = lane + 64 * u;
    const bool ok = e < cnt;
    w[u] = ok ? wt[e] : 0.0f;
    dw[u] = ok ? dwt[e] : 0.0f;
    id[u] = ok ? ids[e] : 0;
  }
  const float s = wave_sum_f(w[0] * dw[0] + w[1] * dw[1]);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = lane + 64 * u;
    if (e < cnt) {
      si[e] = id[u] / n;
      sj[e] = id[u] - (id[u] / n) * n;
      sds[e] = w[u] * (dw[u] - s);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  // the last entry of each repeated i (or j) writes the sum over its group, taken in
  // slot order
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = lane + 64 * u;
    if (e < cnt) {
      const int ie = si[e], je = sj[e];
      float sum_i = 0.0f, sum_j = 0.0f;
      bool last_i = true, last_j = true;
      for (int k = 0; k < cnt; ++k) {
        const float v = sds[k];
        if (si[k] == ie) {
          sum_i += v;
          last_i = k <= e;
        }
        if (sj[k] == je) {
          sum_j += v;
          last_j = k <= e;
        }
      }
      if (last_i) row[o1 + ie] = sum_i;
      if (last_j) row[o2 + je] = sum_j;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

struct SelBackArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* alpha;
  const float* beta;
  const float* gate;
  const void* x;
  const void* w_proj;
  const float* A;
  const float* b_dt;
  const float* d_wt_w;
  const float* d_wt_r;
  const float* g_v;  // incoming gradient of the value
  const float* d_gate;
  const float* d_alpha;
  const float* d_beta;
  float* d_y;
  float* part;  // [M*H][2]: per-token terms of dA and db_dt
  int64_t M, d_model;
  int H, n, W, R, d_v, P, gate_act;
};

// One wavefront per (token, head).  LDS: the head's dY row (P floats) and the
// role's (i, j, ds) triples.
template <bool BF16>
__global__ __launch_bounds__(64) void select_backward_kernel(SelBackArgs a) {
  extern __shared__ float row[];
  __shared__ int si[SDM_MAX_COUNT], sj[SDM_MAX_COUNT];
  __shared__ float sds[SDM_MAX_COUNT];
  const int lane = threadIdx.x;
  const int64_t mh = blockIdx.x;
  const int64_t m = mh / a.H;
  const int h = (int)(mh - m * a.H);
  const int n4 = 4 * a.n;
  // the forget pre-gate, recomputed
  const int64_t arow = (int64_t)h * a.P + n4 + 2 * a.d_v;
  const float z = dot_row<BF16>(a.x, a.w_proj, m, arow, a.d_model) + a.b_dt[h];
  const float alpha = a.alpha[mh], beta = a.beta[mh];
  const float dal = a.d_alpha[mh];
  const float dz = dal * (-a.A[h] * alpha * sigmoid_b(z));
  if (lane == 0) {
    a.part[mh * 2] = dal * (-softplus_b(z) * alpha);
    a.part[mh * 2 + 1] = dz;
  }
  for (int c = lane; c < n4; c += 64) row[c] = 0.0f;
  if (a.gate_act == SDM_GATE_SILU) {
    // SiLU's derivative needs the pre-activation p: recomputed as x . W_g in fp32 and
    // parked in the gate columns of the row until the gradient replaces it
    for (int c = 0; c < a.d_v; ++c) {
      const float pre = dot_row<BF16>(a.x, a.w_proj, m, (int64_t)h * a.P + n4 + a.d_v + c,
                                      a.d_model);
      if (lane == 0) row[n4 + a.d_v + c] = pre;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }
  for (int c = lane; c < a.d_v; c += 64) {
    row[n4 + c] = a.g_v[mh * a.d_v + c];
    const float g = a.gate[mh * a.d_v + c];
    const float dg = a.d_gate[mh * a.d_v + c];
    float dgp;  // d gate / d pre-activation
    if (a.gate_act == SDM_GATE_SIGMOID) {
      dgp = g * (1.0f - g);
    } else if (a.gate_act == SDM_GATE_SILU) {
      const float p = row[n4 + a.d_v + c];
      const float sg = sigmoid_b(p);
      dgp = sg * (1.0f + p * (1.0f - sg));
    } else {
      dgp = 1.0f;
    }
    row[n4 + a.d_v + c] = dg * dgp;
  }
  if (lane == 0) {
    row[n4 + 2 * a.d_v] = dz;
    row[n4 + 2 * a.d_v + 1] = a.d_beta[mh] * beta * (1.0f - beta);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  role_backward(a.idx_w + mh * a.W, a.wt_w + mh * a.W, a.d_wt_w + mh * a.W, a.W, a.n, row, 0,
                a.n, si, sj, sds);
  role_backward(a.idx_r + mh * a.R, a.wt_r + mh * a.R, a.d_wt_r + mh * a.R, a.R, a.n, row,
                2 * a.n, 3 * a.n, si, sj, sds);
  float* dst = a.d_y + mh * a.P;
  for (int c = lane; c < a.P; c += 64) dst[c] = row[c];
}

// dA[h] and db_dt[h]: sums of the per-token terms over all tokens, in a fixed tree.
__global__ __launch_bounds__(256) void select_backward_sum_kernel(const float* __restrict__ part,
                                                                  int64_t M, int H, float* d_A,
                                                                  float* d_b_dt) {
  __shared__ float sa[256], sb[256];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  float ta = 0.0f, tb = 0.0f;
  for (int64_t m = tid; m < M; m += 256) {
    ta += part[(m * H + h) * 2];
    tb += part[(m * H + h) * 2 + 1];
  }
  sa[tid] = ta;
  sb[tid] = tb;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      sa[tid] += sa[tid + o];
      sb[tid] += sb[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    d_A[h] = sa[0];
    d_b_dt[h] = sb[0];
  }
}

}  // namespace

size_t select_backward_ws_bytes(const sdm_dims& d) {
  return (size_t)d.B * d.T * d.H * 2 * sizeof(float);
}

hipError_t launch_select_backward(const sdm_dims& d, const sdm_sel& fwd, const void* x,
                                  const void* w_proj, const float* A, const float* b_dt,
                                  const sdm_select_grads& g, float* d_y, float* d_A,
                                  float* d_b_dt, void* ws, hipStream_t s) {
  SelBackArgs a;
  a.idx_w = fwd.idx_w;
  a.wt_w = fwd.wt_w;
  a.idx_r = fwd.idx_r;
  a.wt_r = fwd.wt_r;
  a.alpha = fwd.alpha;
  a.beta = fwd.beta;
  a.gate = fwd.gate;
  a.x = x;
  a.w_proj = w_proj;
  a.A = A;
  a.b_dt = b_dt;
  a.d_wt_w = g.d_wt_w;
  a.d_wt_r = g.d_wt_r;
  a.g_v = g.d_v;
  a.d_gate = g.d_gate;
  a.d_alpha = g.d_alpha;
  a.d_beta = g.d_beta;
  a.d_y = d_y;
  a.part = static_cast<float*>(ws);
  a.M = d.B * d.T;
  a.d_model = d.d_model;
  a.H = d.H;
  a.n = d.n;
  a.W = d.W;
  a.R = d.R;
  a.d_v = d.d_v;
  a.P = 4 * d.n + 2 * d.d_v + 2;
  a.gate_act = d.gate_act;
  const dim3 grid((unsigned)(a.M * d.H));
  const size_t lds = (size_t)a.P * sizeof(float);
  {
    KernelTimer kt("select_backward", s);
    if (d.in_dtype == SDM_DTYPE_BF16)
      hipLaunchKernelGGL(select_backward_kernel<true>, grid, dim3(64), lds, s, a);
    else
      hipLaunchKernelGGL(select_backward_kernel<false>, grid, dim3(64), lds, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KernelTimer kt("select_backward_sum", s);
  hipLaunchKernelGGL(select_backward_sum_kernel, dim3((unsigned)d.H), dim3(256), 0, s,
                     static_cast<const float*>(ws), a.M, d.H, d_A, d_b_dt);
  return hipGetLastError();
}

}  // namespace sdm
