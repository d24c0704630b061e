// Recurrent sparse scan of the SDM layer (the state lives in HBM).
//
// Per (batch, head) memory M [N, d_v] and tokens t = 0..T-1 in order
// ("Sparse Delta Memory" summary on paper.rainbus.top, method paragraph, steps
// 2-4; ai-paper-analysis.pages.dev, sections "步骤 2" to "步骤 4"):
//   write: for each selected write slot i with weight k: c = beta_t k,
//          M[i] <- (1 - c) (alpha_t M[i]) + c v_t     (forget gate, then delta rule)
//   read:  y_t = sum_{i in I_r} q^(i) M[i]            (after this token's writes)
//   out:   y_t / sqrt(mean(y_t^2) + eps) * gamma_h * gate_t
// Unselected slots are never touched.  The slot ids of every token are known
// before the scan starts (selection pass), so the kernel only moves rows.
// The key-weighted variant (SDM_FLAG_DELTA_GDN) runs its direct schedule in
// scan_slices.hip.  Storage (SDM_FLAG_STATE_BF16): bf16 state rows, fp32
// arithmetic, each stored element rounded to nearest-even bf16.  SDM_FLAG_STATE_FP8:
// E4M3 codes with one power-of-two exponent per 32-column block (fp8_quantize), each
// written row's blocks requantised after the update.
#include "sdm_internal.h"

namespace sdm {
namespace {

__device__ __forceinline__ float4 f4(float a) { return make_float4(a, a, a, a); }

// One workgroup of 256 threads per (b, h).  A row of d_v floats is handled by
// LPR = d_v/4 lanes (one float4 each); the G = 256/LPR row groups split the W
// writes and R reads of a token.  Barriers order the write phase, the read phase
// and the next token's writes (all accesses stay inside one workgroup, whose
// waves share the CU's vector L1).
// LOG: the training forward's write log (a separate instantiation keeps the
// encoder's registers out of the inference kernel).  F8: fp8 state (codes plane,
// then one exponent byte per 32-column block of a row; DV >= 32).
template <int DV, bool BF, bool LOG, bool F8 = false>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  static_assert(!(F8 && (BF || LOG || DV < 32)), "fp8 state: inference, 32-column blocks");
  constexpr uint32_t ES = F8 ? 1u : StateT<BF>::ES;
  constexpr int BQ = 8;  // rows a group keeps in flight
  constexpr int LPR = DV / 4;
  constexpr int G = 256 / LPR;
  __shared__ float4 red[G][LPR];

  const int tid = threadIdx.x;
  const int li = tid % LPR;
  const int grp = tid / LPR;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.H;
  const int h = (int)(bh - b * a.H);
  // row r, this lane's 4 columns
  char* const Mb = static_cast<char*>(a.state) + bh * (int64_t)a.N * DV * ES + li * 4 * ES;
  auto row = [&](int64_t r) { return Mb + r * (DV * ES); };
  // F8: this lane's block exponent of row r at Eb + r * (DV / 32)
  uint8_t* const Eb = F8 ? static_cast<uint8_t*>(a.state) + a.B * a.H * (int64_t)a.N * DV +
                               bh * (int64_t)a.N * (DV / 32) + li / 8
                         : nullptr;
  auto load_row = [&](int64_t r) {
    if constexpr (F8)
      return fp8_decode4(*reinterpret_cast<const uint32_t*>(row(r)), Eb[r * (DV / 32)]);
    else
      return state_load<BF>(row(r));
  };
  const float4 gam = a.norm_w ? reinterpret_cast<const float4*>(a.norm_w + (int64_t)h * DV)[li]
                              : f4(1.0f);

  for (int64_t t = 0; t < a.T; ++t) {
    const int64_t tok = (b * a.T + t) * a.H + h;
    const float al = a.alpha[tok];
    const float be = a.beta[tok];
    const float4 vv = reinterpret_cast<const float4*>(a.v + tok * DV)[li];
    const int32_t* iw = a.idx_w + tok * a.W;
    const float* ww = a.wt_w + tok * a.W;
    const int32_t* ir = a.idx_r + tok * a.R;
    const float* wr = a.wt_r + tok * a.R;
    // A token's write ids are distinct, so a group's rows never alias: their loads
    // are all issued before the first store (BQ rows in flight per lane).
    for (int k0 = grp; k0 < a.W; k0 += G * BQ) {
      char* p[BQ];
      int64_t rid[BQ];
      float4 m[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        rid[j] = iw[k < a.W ? k : k0];
        p[j] = row(rid[j]);
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        if constexpr (F8)
          m[j] = fp8_decode4(*reinterpret_cast<const uint32_t*>(p[j]), Eb[rid[j] * (DV / 32)]);
        else
          m[j] = state_load<BF>(p[j]);
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        if (k >= a.W) break;
        const float c = be * ww[k];
        const float oc = 1.0f - c;
        if constexpr (LOG)  // training forward: the row as it was before this write
          log_store<LPR>(a.log, a.log_scale, a.log_fmt, tok * a.W + k, DV, m[j], li);
        float4 n;
        n.x = fmaf(c, vv.x, oc * (al * m[j].x));
        n.y = fmaf(c, vv.y, oc * (al * m[j].y));
        n.z = fmaf(c, vv.z, oc * (al * m[j].z));
        n.w = fmaf(c, vv.w, oc * (al * m[j].w));
        if constexpr (F8) {
          const Fp8Row q = fp8_quantize(n);
          *reinterpret_cast<uint32_t*>(p[j]) = q.codes;
          if ((li & 7) == 0) Eb[rid[j] * (DV / 32)] = (uint8_t)q.s;
        } else {
          state_store<BF>(reinterpret_cast<uint64_t>(p[j]), state_round<BF>(n));
        }
      }
    }
    __syncthreads();
    float4 acc = f4(0.0f);
    for (int k0 = grp; k0 < a.R; k0 += G * BQ) {  // same order of the sum, rows batched
      float4 m[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        m[j] = load_row(ir[k < a.R ? k : k0]);
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int k = k0 + j * G;
        if (k >= a.R) break;
        const float q = wr[k];
        acc.x = fmaf(q, m[j].x, acc.x);
        acc.y = fmaf(q, m[j].y, acc.y);
        acc.z = fmaf(q, m[j].z, acc.z);
        acc.w = fmaf(q, m[j].w, acc.w);
      }
    }
    red[grp][li] = acc;
    __syncthreads();
    if (grp == 0) {
      float4 y = red[0][li];
      for (int g = 1; g < G; ++g) {
        const float4 o = red[g][li];
        y.x += o.x;
        y.y += o.y;
        y.z += o.z;
        y.w += o.w;
      }
      float ss = y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
      for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LPR);
      const float rn = rsqrtf(ss / (float)DV + a.eps);
      const float4 gt = reinterpret_cast<const float4*>(a.gate + tok * DV)[li];
      float4 o;
      o.x = y.x * rn * gam.x * gt.x;
      o.y = y.y * rn * gam.y * gt.y;
      o.z = y.z * rn * gam.z * gt.z;
      o.w = y.w * rn * gam.w * gt.w;
      reinterpret_cast<float4*>(a.out + tok * DV)[li] = o;
      if (a.y_raw) reinterpret_cast<float4*>(a.y_raw + tok * DV)[li] = y;
    }
  }
}

template <int DV>
hipError_t launch_direct(dim3 grid, hipStream_t s, const ScanArgs& a) {
  if (a.log)  // training forward: fp32 state
    hipLaunchKernelGGL((scan_kernel<DV, false, true>), grid, dim3(256), 0, s, a);
  else if (a.state_fp8 && DV < 32)  // blocks of 32 columns (refused at the entry)
    return hipErrorInvalidValue;
  else if (a.state_fp8)
    hipLaunchKernelGGL((scan_kernel<DV, false, false, (DV >= 32)>), grid, dim3(256), 0, s, a);
  else if (a.state_bf16)
    hipLaunchKernelGGL((scan_kernel<DV, true, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<DV, false, false>), grid, dim3(256), 0, s, a);
  return hipSuccess;
}

}  // namespace

// The slot-owner schedules from 16 tokens, unless the walks alone fill the chip
// (kDirectWalks): then the direct walk is faster.
bool scan_uses_stream(const sdm_dims& d) {
  if (d.flags & (SDM_FLAG_SCAN_DIRECT | SDM_FLAG_DELTA_GDN | SDM_FLAG_SCAN_CHUNK)) return false;
  if (d.flags & (SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_TWO_PHASE)) return true;
  return d.T >= 16 && d.B * d.H < kDirectWalks;
}

// Workspace per token and walk of a training forward whose quantised log is staged
// in fp32 (stream schedule).
static int64_t stage_bytes(const sdm_dims& d, bool quantised_log) {
  return quantised_log ? (int64_t)d.W * d.d_v * 4 : 0;
}

size_t scan_workspace_bytes(const sdm_dims& d, bool train) {
  if (scan_uses_chunk(d)) return chunk_workspace_bytes(d);  // training: fp32 log only
  if (d.flags & SDM_FLAG_DELTA_GDN) return gdn_slice_workspace_bytes(d, train);
  if (!scan_uses_stream(d)) return 0;
  const bool q = train && (d.flags & (SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4));
  return stream_workspace_bytes(d, plan_stream(d, (int64_t)d.n * d.n, stage_bytes(d, q)));
}

hipError_t launch_scan(const sdm_dims& d, const ScanArgs& a, void* ws, size_t, hipStream_t s) {
  if (scan_uses_chunk(d)) return launch_chunk_scan(d, a, ws, s);
  if (scan_uses_stream(d))
    return launch_stream_scan(
        a, plan_stream(d, a.N, stage_bytes(d, a.log != nullptr && a.log_fmt != LOG_F32)), ws, s);
  if (d.flags & SDM_FLAG_DELTA_GDN) return launch_gdn_slices(d, a, ws, s);
  const dim3 grid((unsigned)(a.B * a.H));
  KernelTimer kt("scan_direct", s);
  hipError_t e;
  switch (a.d_v) {
    case 16: e = launch_direct<16>(grid, s, a); break;
    case 32: e = launch_direct<32>(grid, s, a); break;
    case 64: e = launch_direct<64>(grid, s, a); break;
    case 128: e = launch_direct<128>(grid, s, a); break;
    case 256: e = launch_direct<256>(grid, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace sdm
