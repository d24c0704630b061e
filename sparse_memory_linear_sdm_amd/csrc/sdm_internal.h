// Internal declarations shared by the HIP translation units of libsdm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm.h"

namespace sdm {

// Where the projection epilogue writes (see proj_gemm.hip).  Row m is the global
// token index b*T + t; the scores buffer may hold only rows [scores_row0, ...).
struct ProjDst {
  float* scores;          // [rows, H, 4n] fp32, indexed by (m - scores_row0)
  int64_t scores_row0;
  float* v;               // [M, H, d_v]
  float* gate;            // [M, H, d_v]  activated
  float* alpha;           // [M, H]
  float* beta;            // [M, H]
  const float* A;         // [H]
  const float* b_dt;      // [H]
  int H, n, d_v, P, gate_act;
};

// Projection Y = x[row0 : row0+rows] W_proj^T with the gate epilogue.
hipError_t launch_proj_gemm(const sdm_dims& d, const void* x, const void* w_proj, int64_t row0,
                            int64_t rows, const ProjDst& dst, hipStream_t s);

// Top-W / top-R selection for `rows` token rows whose half-scores start at
// `scores` ([rows, H, 4n]); results go to global rows out_row0 + r.
hipError_t launch_select(const sdm_dims& d, const float* scores, int64_t rows, int64_t out_row0,
                         int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                         hipStream_t s);

// Backward of the selection pass down to dY (select_backward.hip).
size_t select_backward_ws_bytes(const sdm_dims& d);
hipError_t launch_select_backward(const sdm_dims& d, const sdm_sel& fwd, const void* x,
                                  const void* w_proj, const float* A, const float* b_dt,
                                  const sdm_select_grads& g, float* d_y, float* d_A,
                                  float* d_b_dt, void* ws, hipStream_t s);

// Recurrent scan over all (b, h) walks.
struct ScanArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* gate;
  const float* alpha;
  const float* beta;
  const float* norm_w;  // nullable
  void* state;          // fp32, or bf16 when state_bf16
  float* out;
  float* y_raw;         // nullable
  void* log;            // nullable: rows before each write (direct schedule), see log_fmt
  float* log_scale;     // [B, T, H, W] absmax of each logged row (quantised formats)
  int32_t log_fmt;      // LOG_F32, LOG_FP8, LOG_INT4
  int64_t B, T;
  int32_t H, N, W, R, d_v;
  float eps;
  bool state_bf16;
  bool state_fp8;       // codes plane, then block exponents (see fp8_block_exp)
};
hipError_t launch_scan(const sdm_dims& d, const ScanArgs& a, void* ws, size_t ws_bytes,
                       hipStream_t s);
// train: the training forward (sdm_scan_train), whose quantised log formats stage fp32
// rows in the workspace on the stream schedule.
size_t scan_workspace_bytes(const sdm_dims& d, bool train = false);

// Slot-owner stream schedule of the scan (scan_stream.hip).
// Instrumentation (SDM_FLAG_TIMING): the C entry points switch recording on for
// the calling thread; every launch site holds a KernelTimer around its launch.
void timing_enable(bool on);
bool timing_enabled();
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

struct StreamArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* gate;
  const float* alpha;
  const float* beta;
  const float* norm_w;
  void* state;     // fp32, or bf16 when state_bf16
  float* out;
  float* y_raw;
  float* log;      // training forward: fp32 rows replaced by writes, else null; row of
                   // (b, t, h, k) at ((b * log_T + log_t0 + t) * H + h) * W + k
  int64_t log_T, log_t0;
  int* counts;     // [walks][rounds][GT]
  int* offsets;    // [walks][GT][rounds + 1]
  int* totals;     // [walks][GT] per-group totals (offsets pass over many groups x rounds)
  // owner-stream entry: {slot | token-in-round << 24, weight bits | read << 31}
  uint2* entries;  // [walks][walk_entries]
  float* y_part;   // [parts][B][Tc][H][d_v]
  float4* trash;   // one float4 per scan thread: sink of non-writing accesses' stores
  int* begins;    // two-phase: [walks][GT][rounds] start of each packed segment
  uint2* clean;   // two-phase: [B][Tc][H][R] clean reads {slot, weight bits}, grouped by part
  int* cstart;    // two-phase: [B][Tc][H][parts + 1] start of each part's clean reads
  int64_t B, T, t0, Tc, walk_entries;
  int32_t H, N, W, R, d_v;
  float eps;
  int32_t S, parts, GT, log2GT, log2GW, rounds;
};
// Tokens per round of the slot-owner stream schedules (entries keep the token's
// place in its round in 8 bits), and the most lane groups one walk's slots are
// hashed over.
constexpr int kStreamRound = 256;
constexpr int kStreamMaxGT = 4096;
// Walks (B H) from which the per-slot rule's lock-step walks, one workgroup per walk,
// fill the chip twice over and beat the slot-owner schedules by default (no bucketing
// passes, no per-part partial reads): 512 walks x 512 tokens, training forward 7.28 vs
// 7.76 ms and reverse walk 11.3 vs 13.2 ms; 1024 walks x 64 tokens, scan 1.33 vs
// 1.50 ms; but 256 walks x 512 tokens 4.76 vs 3.91 ms and 8.4 vs 6.6 ms.
constexpr int64_t kDirectWalks = 512;

// Lane `src` of a 16-lane row to the whole row (DPP row_newbcast, gfx90a and later).
template <int SRC>
__device__ __forceinline__ uint32_t row_bcast16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + SRC, 0xf, 0xf, false);
}

// Value of lane `src` of this lane's LPG-lane group (LPG = 4, 8 or 16), moved by DPP
// in the vector ALU (no LDS traffic).  quad_perm broadcasts within each quad; for
// 8-lane groups row_half_mirror brings the other quad's broadcast across; a 16-lane
// group is a DPP row.  `src` is a constant once the callers' loops are unrolled.
template <int LPG>
__device__ __forceinline__ uint32_t group_bcast(uint32_t v, int src) {
  if constexpr (LPG == 16) {
    switch (src & 15) {
      case 0: return row_bcast16<0>(v);
      case 1: return row_bcast16<1>(v);
      case 2: return row_bcast16<2>(v);
      case 3: return row_bcast16<3>(v);
      case 4: return row_bcast16<4>(v);
      case 5: return row_bcast16<5>(v);
      case 6: return row_bcast16<6>(v);
      case 7: return row_bcast16<7>(v);
      case 8: return row_bcast16<8>(v);
      case 9: return row_bcast16<9>(v);
      case 10: return row_bcast16<10>(v);
      case 11: return row_bcast16<11>(v);
      case 12: return row_bcast16<12>(v);
      case 13: return row_bcast16<13>(v);
      case 14: return row_bcast16<14>(v);
      default: return row_bcast16<15>(v);
    }
  }
  const int q = src & 3;
  const int qp = q | (q << 2) | (q << 4) | (q << 6);  // quad_perm(q,q,q,q)
  uint32_t x;
  switch (qp) {
    case 0x00: x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xf, 0xf, false); break;
    case 0x55: x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xf, 0xf, false); break;
    case 0xaa: x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xaa, 0xf, 0xf, false); break;
    default: x = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xff, 0xf, 0xf, false); break;
  }
  if (LPG == 4) return x;
  const uint32_t m = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xf, 0xf, false);  // row_half_mirror
  const bool own_quad = ((threadIdx.x >> 2) & 1) == ((src >> 2) & 1);
  return own_quad ? x : m;
}

// Bucketing pre-passes of the stream schedules (count, offsets, scatter) for one
// token chunk; train: entries carry the access's position in its token's id list
// in place of the weight.
hipError_t launch_stream_buckets(const StreamArgs& a, int64_t walks, bool train, hipStream_t st);

struct StreamPlan {
  int SW, S, NT, parts, GT, log2GT, rounds;
  bool two_phase;  // clean reads summed in registers after each round's writes
  int64_t Tc;
  int64_t stage_bytes;  // per token and walk: fp32 log rows staged for quantisation
};
// stage_bytes: workspace per token and walk for a training forward whose log is
// quantised after the walk (W * d_v * 4), else 0.
StreamPlan plan_stream(const sdm_dims& d, int64_t N, int64_t stage_bytes = 0);
size_t stream_workspace_bytes(const sdm_dims& d, const StreamPlan& pl);
hipError_t launch_stream_scan(const ScanArgs& a, const StreamPlan& pl, void* ws, hipStream_t s);
bool scan_uses_stream(const sdm_dims& d);
// y [B, T, H, d_v] (one part) through the RMSNorm and gate into a.out (and a.y_raw).
hipError_t launch_norm_gate(const ScanArgs& a, const float* y, hipStream_t st);

// Chunkwise schedule (scan_chunk.hip, SDM_FLAG_SCAN_CHUNK): fp32 state, forward only.
bool scan_uses_chunk(const sdm_dims& d);
size_t chunk_workspace_bytes(const sdm_dims& d);
hipError_t launch_chunk_scan(const sdm_dims& d, const ScanArgs& a, void* ws, hipStream_t st);

// Direct schedule of the key-weighted rule, split over column slices of the state
// (scan_slices.hip): the inference walk, the training forward (any log format) and
// its backward.
int gdn_slices(const sdm_dims& d);
size_t gdn_slice_workspace_bytes(const sdm_dims& d, bool train);
hipError_t launch_gdn_slices(const sdm_dims& d, const ScanArgs& a, void* ws, hipStream_t st);
// Encodes a token chunk's fp32 log rows, staged [B][Tc][H][W][d_v], into a.log.
hipError_t launch_log_quantize(const ScanArgs& a, const float* stage, int64_t t0, int64_t Tc,
                               hipStream_t st);

// Write-log storage (training): one row of d_v values per write, fp32, or quantised
// with one absmax per row -- fp8 (OCP E4M3, v = x * 448 / absmax) or int4 (v = x * 7 /
// absmax, codes -7..7, two per byte, low nibble first).  Codes are decided in fp32.
enum { LOG_F32 = 0, LOG_FP8 = 1, LOG_INT4 = 2 };

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (8 steps reach the smallest normal)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // a in [2^e, 2^(e+1))
    float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));   // in [8, 16], exact scaling
    if (q == 16.0f) {
      q = 8.0f;
      ++e;
    }
    const int field = e + 7;
    const uint32_t frac = (uint32_t)q - 8u;
    code = (field > 15 || (field == 15 && frac == 7)) ? 0x7Eu : ((uint32_t)field << 3) | frac;
  }
  return code | sign;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t field = (c >> 3) & 15u, frac = c & 7u;
  const float mag = field == 0 ? (float)frac * 0.001953125f  // 2^-9
                               : __builtin_ldexpf((float)(8u + frac), (int)field - 10);
  return (c & 0x80u) ? -mag : mag;
}

// Stores logged row r (rows of dv values), this lane's columns 4 li .. 4 li + 3, the
// row held by LPR lanes: fp32, or quantised with the row's absmax (a max over the
// row's lanes), the codes decided in fp32.
template <int LPR>
__device__ __forceinline__ void log_store(void* log, float* log_scale, int fmt, int64_t r, int dv,
                                          float4 m, int li) {
  if (fmt == LOG_F32) {
    reinterpret_cast<float4*>(static_cast<float*>(log) + r * dv)[li] = m;
    return;
  }
  float mx = fmaxf(fmaxf(fabsf(m.x), fabsf(m.y)), fmaxf(fabsf(m.z), fabsf(m.w)));
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, LPR));
  if (li == 0) log_scale[r] = mx;
  uint8_t* base = static_cast<uint8_t*>(log);
  if (fmt == LOG_FP8) {
    const float inv = mx > 0.0f ? 448.0f / mx : 0.0f;
    reinterpret_cast<uint32_t*>(base + r * dv)[li] =
        e4m3_encode(m.x * inv) | e4m3_encode(m.y * inv) << 8 | e4m3_encode(m.z * inv) << 16 |
        e4m3_encode(m.w * inv) << 24;
  } else {
    const float inv = mx > 0.0f ? 7.0f / mx : 0.0f;
    auto q = [&](float x) {
      const float t = fminf(fmaxf(__builtin_rintf(x * inv), -7.0f), 7.0f);
      return (uint32_t)(int)t & 15u;
    };
    reinterpret_cast<uint16_t*>(base + r * (dv / 2))[li] =
        (uint16_t)(q(m.x) | q(m.y) << 4 | q(m.z) << 8 | q(m.w) << 12);
  }
}

// Logged row r (rows of dv values), columns 4 li .. 4 li + 3: fp32, or decoded with the
// row's absmax.
__device__ __forceinline__ float4 log_load(const void* log, const float* log_scale, int fmt,
                                           int64_t r, int dv, int li) {
  if (fmt == LOG_F32)
    return reinterpret_cast<const float4*>(static_cast<const float*>(log) + r * dv)[li];
  const uint8_t* base = static_cast<const uint8_t*>(log);
  const float mx = log_scale[r];
  if (fmt == LOG_FP8) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(base + r * dv)[li];
    const float unit = mx / 448.0f;
    return make_float4(e4m3_decode(w & 0xff) * unit, e4m3_decode((w >> 8) & 0xff) * unit,
                       e4m3_decode((w >> 16) & 0xff) * unit, e4m3_decode(w >> 24) * unit);
  }
  const uint32_t w = reinterpret_cast<const uint16_t*>(base + r * (dv / 2))[li];
  const float unit = mx / 7.0f;
  auto q = [&](uint32_t s) { return (float)(((int)((w >> s) & 15u) ^ 8) - 8) * unit; };
  return make_float4(q(0), q(4), q(8), q(12));
}

// Backward of the scan and norm/gate (scan_backward.hip): reverse walk per (b, h).
struct ScanBackArgs {
  const int32_t* idx_w;
  const float* wt_w;
  const int32_t* idx_r;
  const float* wt_r;
  const float* v;
  const float* gate;
  const float* alpha;
  const float* beta;
  const float* norm_w;  // nullable (ones)
  float* state;         // IN M_T, OUT M_0
  float* d_state;       // IN dL/dM_T, OUT dL/dM_0
  const float* y_raw;
  const void* log;      // [B, T, H, W, d_v] in log_fmt
  const float* log_scale;
  int32_t log_fmt;
  const float* d_out;
  float* g_wt_w;
  float* g_wt_r;
  float* g_v;
  float* g_gate;
  float* g_alpha;
  float* g_beta;
  float* g_gamma_part;  // [B, H, d_v] per-walk partials (workspace)
  int64_t B, T;
  int32_t H, N, W, R, d_v;
  float eps;
};
hipError_t launch_scan_backward(const ScanBackArgs& a, float* d_norm_w, hipStream_t s);
size_t gdn_slice_backward_workspace_bytes(const sdm_dims& d);
hipError_t launch_gdn_slice_backward(const sdm_dims& d, const ScanBackArgs& a, float* d_norm_w,
                                     void* ws, hipStream_t st);
// Per token: the per-slice shares of the key-weighted reverse walks (pr [S][rows][R],
// pw [S][rows][W] (<G, e>, <de, m>), pa [S][rows]) summed in slice order into d_wt_r,
// d_wt_w, d_alpha and d_beta.
hipError_t launch_gdn_back_reduce(const ScanBackArgs& a, float* pr, float2* pw, float* pa, int S,
                                  hipStream_t st);
// The key-weighted reverse walk on the chunk schedule (scan_chunk.hip).
bool gdn_back_uses_chunk(const sdm_dims& d);
size_t chunk_backward_workspace_bytes(const sdm_dims& d);
hipError_t launch_chunk_backward(const sdm_dims& d, const ScanBackArgs& a, float* d_norm_w,
                                 void* ws, hipStream_t st);
// Norm/gate backward of all tokens (scan_stream_backward.hip): dy [B, T, H, d_v],
// d_gate, and d_gamma partials [B*H][norm_backward_blocks(T)][d_v]; then their sum.
int norm_backward_blocks(int64_t T);
hipError_t launch_norm_backward(const ScanBackArgs& a, float* dy, float* gpart, hipStream_t st);
hipError_t launch_gamma_blocks(const ScanBackArgs& a, const float* gpart, float* d_norm_w,
                               hipStream_t st);
// The same backward on the slot-owner stream schedule (scan_stream_backward.hip), for
// long token runs; needs stream_backward_workspace_bytes(d) of workspace.
bool backward_uses_stream(const sdm_dims& d);
size_t stream_backward_workspace_bytes(const sdm_dims& d);
hipError_t launch_stream_backward(const sdm_dims& d, const ScanBackArgs& a, float* d_norm_w,
                                  void* ws, hipStream_t s);

// Shared initial state (shared_m0.hip): set the touched bit of every id the call
// reads or writes; copy M0[h][id] into the store on the first touch.
hipError_t launch_materialize(const sdm_dims& d, int64_t N, const int32_t* idx_w,
                              const int32_t* idx_r, const void* m0, void* store,
                              uint32_t* touched, hipStream_t s);

// Slot-update histogram (monitor.hip): counts[h][id] += 1 for every write id.
hipError_t launch_slot_histogram(const sdm_dims& d, int64_t N, const int32_t* idx_w,
                                 int32_t* counts, hipStream_t s);

// State element storage of the scan kernels: fp32, or bf16 (SDM_FLAG_STATE_BF16)
// with fp32 arithmetic.  A lane moves 4 consecutive elements of a row: one 16-byte
// (fp32) or 8-byte (bf16) access.  state_round returns a value as it will be stored
// (nearest bf16, ties to even, by the hardware conversion), so that forwarded and
// re-read values agree.
template <bool BF>
struct StateT {
  static constexpr uint32_t ES = BF ? 2u : 4u;  // bytes per element
};
typedef float sdm_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 sdm_b2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  const sdm_b2 r = __builtin_convertvector((sdm_f2){a, b}, sdm_b2);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}
__device__ __forceinline__ float4 bf16_unpack4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <bool BF>
__device__ __forceinline__ float4 state_load(const char* p) {
  if constexpr (BF)
    return bf16_unpack4(*reinterpret_cast<const uint2*>(p));
  else
    return *reinterpret_cast<const float4*>(p);
}
template <bool BF>
__device__ __forceinline__ float4 state_round(float4 v) {
  if constexpr (BF)
    return bf16_unpack4(make_uint2(bf16_pack2(v.x, v.y), bf16_pack2(v.z, v.w)));
  else
    return v;
}
// Stores a value already passed through state_round (the conversion is then exact).
// The address is a plain integer so callers can pick it without a branch.
template <bool BF>
__device__ __forceinline__ void state_store(uint64_t addr, float4 v) {
  if constexpr (BF) {
    typedef uint32_t gvec2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<__attribute__((address_space(1))) gvec2*>(addr) =
        gvec2{bf16_pack2(v.x, v.y), bf16_pack2(v.z, v.w)};
  } else {
    typedef float gvec4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<__attribute__((address_space(1))) gvec4*>(addr) =
        gvec4{v.x, v.y, v.z, v.w};
  }
}

// fp8 state storage (SDM_FLAG_STATE_FP8): the state buffer holds a codes plane
// [B, H, N, d_v] of OCP E4M3 bytes (e4m3_encode above), then an exponent plane
// [B, H, N, d_v / 32] of E8M0 bytes, one per 32-column block of a row.  An element
// is value(code) * 2^(s - 127).  A block's exponent is the least e >= -127 with
// absmax <= 448 * 2^e, read off the fp32 bits of the block's absmax, so scaling by
// 2^-e is exact and never saturates.  Lanes move 4 consecutive elements; a block is
// 8 consecutive lanes of a wavefront.
__device__ __forceinline__ int fp8_block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int field = (int)((u >> 23) & 0xffu);
  if (field == 0) return -127;  // zero or below 2^-126
  const int e = field - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);  // mantissa > 1.75
  return e < -127 ? -127 : e;
}
// The element conversions are gfx950's fp8 instructions (v_cvt_f32_fp8,
// v_cvt_pk_fp8_f32), whose format is OCP E4M3 with round-to-nearest-even: on the GPU
// they give the codes and values of e4m3_encode / e4m3_decode above for every code,
// every midpoint between codes and the subnormal range.
__device__ __forceinline__ float4 fp8_decode4(uint32_t w, uint32_t s) {
  const float unit = __builtin_ldexpf(1.0f, (int)s - 127);
  return make_float4(__builtin_amdgcn_cvt_f32_fp8((int)w, 0) * unit,
                     __builtin_amdgcn_cvt_f32_fp8((int)w, 1) * unit,
                     __builtin_amdgcn_cvt_f32_fp8((int)w, 2) * unit,
                     __builtin_amdgcn_cvt_f32_fp8((int)w, 3) * unit);
}
// The largest of x over the 8 lanes of this lane's block: quad swaps by DPP, then
// the other quad of the 8 by row_half_mirror; every lane gets it.
__device__ __forceinline__ float block8_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf,
                                                          false)));
}
// This lane's 4 elements as stored: their codes, the block's exponent byte, and the
// values they decode to.  Every lane of the block must take part.
struct Fp8Row {
  float4 val;
  uint32_t codes;
  uint32_t s;
};
__device__ __forceinline__ Fp8Row fp8_quantize(float4 v) {
  const float a = block8_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const int e = fp8_block_exp(a);
  const float inv = __builtin_ldexpf(1.0f, -e);
  Fp8Row r;
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v.x * inv, v.y * inv, 0, false);
  r.codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v.z * inv, v.w * inv, lo, true);
  r.s = (uint32_t)(e + 127);
  r.val = fp8_decode4(r.codes, r.s);
  return r;
}

}  // namespace sdm
