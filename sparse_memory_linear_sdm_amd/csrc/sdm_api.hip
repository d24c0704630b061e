// C ABI of libsdm: argument validation, workspace layout and kernel dispatch.
// Every check runs before the first enqueue, so a failing call leaves all
// outputs untouched and needs no GPU to be exercised.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "sdm_internal.h"

using namespace sdm;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kScoreChunkBytes = 1ll << 30;  // bound on the scores staging buffer

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Derived {
  int64_t M;      // token rows B*T
  int64_t N;      // slots per memory
  int64_t P;      // projection columns per head
  int64_t chunk;  // GEMM rows per scores chunk when staging in the workspace
};

int32_t check_dims(const sdm_dims* d, Derived* out) {
  if (!d) return SDM_ERR_NULL;
  const int32_t sched = SDM_FLAG_SCAN_DIRECT | SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_TWO_PHASE |
                        SDM_FLAG_SCAN_CHUNK;
  if (d->flags & ~(sched | SDM_FLAG_TIMING | SDM_FLAG_DELTA_GDN | SDM_FLAG_STATE_BF16 |
                   SDM_FLAG_STATE_FP8 | SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4))
    return SDM_ERR_UNSUPPORTED;
  if ((d->flags & SDM_FLAG_LOG_FP8) && (d->flags & SDM_FLAG_LOG_INT4)) return SDM_ERR_SHAPE;
  if ((d->flags & SDM_FLAG_STATE_FP8) && (d->flags & SDM_FLAG_STATE_BF16)) return SDM_ERR_SHAPE;
  // fp8 state: the per-slot rule on the two-phase and direct schedules, d_v >= 32
  if ((d->flags & SDM_FLAG_STATE_FP8) &&
      ((d->flags & (SDM_FLAG_DELTA_GDN | SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_CHUNK)) ||
       d->d_v < 32))
    return SDM_ERR_UNSUPPORTED;
  if (__builtin_popcount((unsigned)(d->flags & sched)) > 1) return SDM_ERR_SHAPE;  // one schedule
  if ((d->flags & SDM_FLAG_DELTA_GDN) &&
      (d->flags & (SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_TWO_PHASE)))
    return SDM_ERR_UNSUPPORTED;  // the variant runs the direct or the chunk schedule
  if ((d->flags & SDM_FLAG_SCAN_CHUNK) && (d->flags & SDM_FLAG_STATE_BF16))
    return SDM_ERR_UNSUPPORTED;
  if (d->in_dtype != SDM_DTYPE_F32 && d->in_dtype != SDM_DTYPE_BF16) return SDM_ERR_DTYPE;
  if (d->gate_act < SDM_GATE_NONE || d->gate_act > SDM_GATE_SILU) return SDM_ERR_DTYPE;
  if (d->B < 0 || d->T < 0 || d->d_model < 1 || d->H < 1 || d->n < 1 || d->W < 1 || d->R < 1 ||
      d->d_v < 1)
    return SDM_ERR_SHAPE;
  if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return SDM_ERR_SHAPE;
  const int64_t N = (int64_t)d->n * d->n;
  if (d->W > N || d->R > N) return SDM_ERR_SHAPE;
  if (d->n > SDM_MAX_HALF || d->W > SDM_MAX_COUNT || d->R > SDM_MAX_COUNT)
    return SDM_ERR_UNSUPPORTED;
  if (!(d->d_v == 16 || d->d_v == 32 || d->d_v == 64 || d->d_v == 128 || d->d_v == 256))
    return SDM_ERR_UNSUPPORTED;
  if (d->d_model % 8 != 0 || d->d_model > (1ll << 30)) return SDM_ERR_UNSUPPORTED;
  const int64_t P = 4ll * d->n + 2ll * d->d_v + 2;
  if ((int64_t)d->H * P > (1ll << 30)) return SDM_ERR_UNSUPPORTED;
  if (d->B > (1ll << 40) || d->T > (1ll << 40) || (d->B > 0 && d->T > (1ll << 40) / d->B))
    return SDM_ERR_UNSUPPORTED;
  const int64_t M = d->B * d->T;
  if (M * d->H * 2 > INT32_MAX) return SDM_ERR_UNSUPPORTED;  // selection grid
  if ((int64_t)d->B * d->H > INT32_MAX) return SDM_ERR_UNSUPPORTED;
  if (out) {
    out->M = M;
    out->N = N;
    out->P = P;
    const int64_t row_bytes = (int64_t)d->H * 4 * d->n * 4;
    int64_t c = kScoreChunkBytes / row_bytes;
    c = c < 128 ? 128 : (c / 128) * 128;
    out->chunk = M < c ? M : c;
  }
  return SDM_OK;
}

// Byte sizes of the pass-(a) products of one call.
struct ProductSizes {
  size_t idx_w, wt_w, idx_r, wt_r, v, gate, alpha, beta, total;
};
ProductSizes product_sizes(const sdm_dims* d, int64_t M) {
  ProductSizes s;
  const size_t th = (size_t)M * d->H;
  s.idx_w = align_up(th * d->W * 4);
  s.wt_w = align_up(th * d->W * 4);
  s.idx_r = align_up(th * d->R * 4);
  s.wt_r = align_up(th * d->R * 4);
  s.v = align_up(th * d->d_v * 4);
  s.gate = align_up(th * d->d_v * 4);
  s.alpha = align_up(th * 4);
  s.beta = align_up(th * 4);
  s.total = s.idx_w + s.wt_w + s.idx_r + s.wt_r + s.v + s.gate + s.alpha + s.beta;
  return s;
}

size_t select_ws_bytes(const sdm_dims* d, const Derived& dv, bool have_scores) {
  if (have_scores || dv.M == 0) return 0;
  return align_up((size_t)dv.chunk * d->H * 4 * d->n * 4);
}

int32_t check_sel(const sdm_sel* s, bool need_scores) {
  if (!s) return SDM_ERR_NULL;
  const void* req[] = {s->idx_w, s->wt_w, s->idx_r, s->wt_r, s->v, s->gate, s->alpha, s->beta};
  for (const void* p : req)
    if (!p) return SDM_ERR_NULL;
  if (need_scores && !s->scores) return SDM_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return SDM_ERR_ALIGN;
  if (s->scores && !aligned16(s->scores)) return SDM_ERR_ALIGN;
  return SDM_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SDM_OK : SDM_ERR_HIP; }

// Enqueue the selection pass (validated arguments only).
int32_t run_select(const sdm_dims* d, const Derived& dv, const void* x, const void* w_proj,
                   const float* A, const float* b_dt, const sdm_sel* out, void* ws,
                   hipStream_t st) {
  ProjDst dst;
  dst.v = out->v;
  dst.gate = out->gate;
  dst.alpha = out->alpha;
  dst.beta = out->beta;
  dst.A = A;
  dst.b_dt = b_dt;
  dst.H = d->H;
  dst.n = d->n;
  dst.d_v = d->d_v;
  dst.P = (int)dv.P;
  dst.gate_act = d->gate_act;
  if (out->scores) {  // full-size scores requested: one pass over every row
    dst.scores = out->scores;
    dst.scores_row0 = 0;
    hipError_t e = launch_proj_gemm(*d, x, w_proj, 0, dv.M, dst, st);
    if (e != hipSuccess) return SDM_ERR_HIP;
    e = launch_select(*d, out->scores, dv.M, 0, out->idx_w, out->wt_w, out->idx_r, out->wt_r, st);
    return hip_status(e);
  }
  dst.scores = static_cast<float*>(ws);
  for (int64_t r0 = 0; r0 < dv.M; r0 += dv.chunk) {
    const int64_t rows = dv.M - r0 < dv.chunk ? dv.M - r0 : dv.chunk;
    dst.scores_row0 = r0;
    hipError_t e = launch_proj_gemm(*d, x, w_proj, r0, rows, dst, st);
    if (e != hipSuccess) return SDM_ERR_HIP;
    e = launch_select(*d, static_cast<const float*>(ws), rows, r0, out->idx_w, out->wt_w,
                      out->idx_r, out->wt_r, st);
    if (e != hipSuccess) return SDM_ERR_HIP;
  }
  return SDM_OK;
}

ScanArgs scan_args(const sdm_dims* d, const Derived& dv, const sdm_sel* in,
                   const float* norm_w, void* state, float* out, float* y_raw) {
  ScanArgs a;
  a.idx_w = in->idx_w;
  a.wt_w = in->wt_w;
  a.idx_r = in->idx_r;
  a.wt_r = in->wt_r;
  a.v = in->v;
  a.gate = in->gate;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.norm_w = norm_w;
  a.state = state;
  a.out = out;
  a.y_raw = y_raw;
  a.log = nullptr;
  a.log_scale = nullptr;
  a.log_fmt = LOG_F32;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.N = (int32_t)dv.N;
  a.W = d->W;
  a.R = d->R;
  a.d_v = d->d_v;
  a.eps = d->eps;
  a.state_bf16 = (d->flags & SDM_FLAG_STATE_BF16) != 0;
  a.state_fp8 = (d->flags & SDM_FLAG_STATE_FP8) != 0;
  return a;
}

int32_t run_scan(const sdm_dims* d, const Derived& dv, const sdm_sel* in, const float* norm_w,
                 void* state, float* out, float* y_raw, void* ws, size_t ws_bytes,
                 hipStream_t st) {
  const ScanArgs a = scan_args(d, dv, in, norm_w, state, out, y_raw);
  return hip_status(launch_scan(*d, a, ws, ws_bytes, st));
}

// Switches kernel timing on for this thread while an entry point runs.
struct TimingScope {
  bool prev;
  explicit TimingScope(const sdm_dims* d) : prev(timing_enabled()) {
    timing_enable((d->flags & SDM_FLAG_TIMING) != 0);
  }
  ~TimingScope() { timing_enable(prev); }
};

// sdm_scan, and with m0 / touched the shared-initial-state form.
int32_t scan_entry(const sdm_dims* d, const sdm_sel* in, const float* norm_w, const void* m0,
                   void* state, uint32_t* touched, float* out, float* y_raw, void* ws,
                   size_t ws_bytes, void* stream, bool shared) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (shared && (d->flags & SDM_FLAG_STATE_FP8)) return SDM_ERR_UNSUPPORTED;
  if (dv.M == 0) return SDM_OK;
  if ((st = check_sel(in, false)) != SDM_OK) return st;
  if (!state || !out || (shared && (!m0 || !touched))) return SDM_ERR_NULL;
  if (!aligned16(state) || !aligned16(out) || (y_raw && !aligned16(y_raw)) ||
      (norm_w && !aligned16(norm_w)) || (m0 && !aligned16(m0)) ||
      (touched && !aligned16(touched)))
    return SDM_ERR_ALIGN;
  const size_t need = align_up(scan_workspace_bytes(*d));
  if (need && (!ws || ws_bytes < need)) return SDM_ERR_WORKSPACE;
  TimingScope timing(d);
  (void)hipGetLastError();
  if (m0 && launch_materialize(*d, dv.N, in->idx_w, in->idx_r, m0, state, touched,
                               (hipStream_t)stream) != hipSuccess)
    return SDM_ERR_HIP;
  return run_scan(d, dv, in, norm_w, state, out, y_raw, ws, ws_bytes, (hipStream_t)stream);
}

// sdm_forward, and with m0 / touched the shared-initial-state form.
int32_t forward_entry(const sdm_dims* d, const void* x, const void* w_proj, const float* A,
                      const float* b_dt, const float* norm_w, const void* m0, void* state,
                      uint32_t* touched, float* out, const sdm_sel* debug, void* ws,
                      size_t ws_bytes, void* stream, bool shared) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (shared && (d->flags & SDM_FLAG_STATE_FP8)) return SDM_ERR_UNSUPPORTED;
  if (dv.M == 0) return SDM_OK;
  if (!x || !w_proj || !A || !b_dt || !state || !out || (shared && (!m0 || !touched)))
    return SDM_ERR_NULL;
  if (debug && (st = check_sel(debug, false)) != SDM_OK) return st;
  if (!aligned16(x) || !aligned16(w_proj) || !aligned16(A) || !aligned16(b_dt) ||
      !aligned16(state) || !aligned16(out) || (norm_w && !aligned16(norm_w)) ||
      (m0 && !aligned16(m0)) || (touched && !aligned16(touched)))
    return SDM_ERR_ALIGN;
  const ProductSizes ps = product_sizes(d, dv.M);
  const size_t sel_ws = select_ws_bytes(d, dv, false);
  const size_t scan_ws = align_up(scan_workspace_bytes(*d));
  const size_t need = ps.total + sel_ws + scan_ws;
  if (!ws || ws_bytes < need) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_ALIGN;

  char* base = static_cast<char*>(ws);
  sdm_sel prod;
  if (debug) {
    prod = *debug;
  } else {
    char* p = base;
    prod.idx_w = reinterpret_cast<int32_t*>(p); p += ps.idx_w;
    prod.wt_w = reinterpret_cast<float*>(p); p += ps.wt_w;
    prod.idx_r = reinterpret_cast<int32_t*>(p); p += ps.idx_r;
    prod.wt_r = reinterpret_cast<float*>(p); p += ps.wt_r;
    prod.v = reinterpret_cast<float*>(p); p += ps.v;
    prod.gate = reinterpret_cast<float*>(p); p += ps.gate;
    prod.alpha = reinterpret_cast<float*>(p); p += ps.alpha;
    prod.beta = reinterpret_cast<float*>(p); p += ps.beta;
    prod.scores = nullptr;
  }
  void* sel_space = base + ps.total;
  void* scan_space = base + ps.total + sel_ws;
  hipStream_t s = (hipStream_t)stream;
  TimingScope timing(d);
  (void)hipGetLastError();
  st = run_select(d, dv, x, w_proj, A, b_dt, &prod, sel_space, s);
  if (st != SDM_OK) return st;
  if (m0 && launch_materialize(*d, dv.N, prod.idx_w, prod.idx_r, m0, state, touched, s) !=
                hipSuccess)
    return SDM_ERR_HIP;
  return run_scan(d, dv, &prod, norm_w, state, out, nullptr, scan_space, scan_ws, s);
}

// ---------------------------------------------------------------------------
// Workspace of sdm_forward_noalloc: one fixed array per GPU in the code object's
// device memory, so that the entry point needs no allocation.  Host code must not
// pass the array's name to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, taken once per device with
// that device current and kept in `g_scratch_ptr`.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[SDM_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's array (resolved on the first call there),
// or nullptr if the device cannot be queried.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int32_t sdm_abi_version(void) { return SDM_ABI_VERSION; }

const char* sdm_status_string(int32_t status) {
  switch (status) {
    case SDM_OK: return "ok";
    case SDM_ERR_NULL: return "a required pointer is NULL";
    case SDM_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case SDM_ERR_DTYPE: return "unknown element type or gate activation";
    case SDM_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case SDM_ERR_WORKSPACE: return "workspace missing or too small";
    case SDM_ERR_UNSUPPORTED: return "sizes outside this build's limits";
    case SDM_ERR_HIP: return "the HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

static int32_t log_format(const sdm_dims* d) {
  return (d->flags & SDM_FLAG_LOG_FP8) ? LOG_FP8 : (d->flags & SDM_FLAG_LOG_INT4) ? LOG_INT4
                                                                                   : LOG_F32;
}

// The training entries take fp32 state: the per-slot rule on the direct, slot-owner and
// chunk schedules, the key-weighted rule on the direct and chunk ones; the chunk
// schedule logs fp32 rows only.
static int32_t check_train_flags(const sdm_dims* d) {
  if (d->flags & (SDM_FLAG_STATE_BF16 | SDM_FLAG_STATE_FP8)) return SDM_ERR_UNSUPPORTED;
  if ((d->flags & SDM_FLAG_SCAN_CHUNK) && (d->flags & (SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4)))
    return SDM_ERR_UNSUPPORTED;
  return SDM_OK;
}

// Schedule of the training forward as scan flags: a schedule asked for; else for the
// per-slot rule the two-phase one from 256 tokens and the direct one below that or from
// kDirectWalks walks; for the key-weighted rule the inference scan's choice with an
// fp32 log (the chunk one from 64 tokens while the walks are few enough) and the
// direct one with a quantised log.
static sdm_dims train_dims(const sdm_dims* d) {
  const int32_t sched = SDM_FLAG_SCAN_DIRECT | SDM_FLAG_SCAN_STREAM | SDM_FLAG_SCAN_TWO_PHASE |
                        SDM_FLAG_SCAN_CHUNK;
  sdm_dims dd = *d;
  if (!(d->flags & sched)) {
    const bool gdn = (d->flags & SDM_FLAG_DELTA_GDN) != 0;
    const bool qlog = (d->flags & (SDM_FLAG_LOG_FP8 | SDM_FLAG_LOG_INT4)) != 0;
    if (gdn)
      dd.flags |= !qlog && scan_uses_chunk(*d) ? SDM_FLAG_SCAN_CHUNK : SDM_FLAG_SCAN_DIRECT;
    else
      dd.flags |= d->T < kStreamRound || d->B * d->H >= kDirectWalks ? SDM_FLAG_SCAN_DIRECT
                                                                      : SDM_FLAG_SCAN_TWO_PHASE;
  }
  return dd;
}

// Backward workspace: per-walk d_gamma partials (direct schedule), or the stream
// schedule's buckets, dy, per-slice partial dots and per-part d_v.
static size_t backward_ws_bytes(const sdm_dims* d) {
  if (d->flags & SDM_FLAG_DELTA_GDN)
    return align_up(gdn_back_uses_chunk(*d) ? chunk_backward_workspace_bytes(*d)
                                            : gdn_slice_backward_workspace_bytes(*d));
  if (backward_uses_stream(*d))
    return align_up(stream_backward_workspace_bytes(*d));
  return align_up((size_t)d->B * d->H * d->d_v * 4);
}

size_t sdm_workspace_bytes(const sdm_dims* d, int32_t entry) {
  Derived dv;
  if (check_dims(d, &dv) != SDM_OK || dv.M == 0) return 0;
  switch (entry) {
    case SDM_ENTRY_SELECT: return select_ws_bytes(d, dv, false);
    case SDM_ENTRY_SCAN: return align_up(scan_workspace_bytes(*d));
    case SDM_ENTRY_FORWARD:
      return product_sizes(d, dv.M).total + select_ws_bytes(d, dv, false) +
             align_up(scan_workspace_bytes(*d));
    case SDM_ENTRY_SCAN_BACKWARD: return backward_ws_bytes(d);
    case SDM_ENTRY_SELECT_FROM_SCORES: return 0;
    case SDM_ENTRY_SELECT_BACKWARD: return align_up(select_backward_ws_bytes(*d));
    case SDM_ENTRY_SCAN_TRAIN: {
      const sdm_dims dd = train_dims(d);
      return align_up(scan_workspace_bytes(dd, true));
    }
    default: return 0;
  }
}

int32_t sdm_select(const sdm_dims* d, const void* x, const void* w_proj, const float* A,
                   const float* b_dt, const sdm_sel* out, void* ws, size_t ws_bytes,
                   void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if (!x || !w_proj || !A || !b_dt) return SDM_ERR_NULL;
  if ((st = check_sel(out, false)) != SDM_OK) return st;
  if (!aligned16(x) || !aligned16(w_proj) || !aligned16(A) || !aligned16(b_dt))
    return SDM_ERR_ALIGN;
  const size_t need = select_ws_bytes(d, dv, out->scores != nullptr);
  if (need && (!ws || ws_bytes < need)) return SDM_ERR_WORKSPACE;
  if (need && !aligned16(ws)) return SDM_ERR_ALIGN;
  TimingScope timing(d);
  (void)hipGetLastError();
  return run_select(d, dv, x, w_proj, A, b_dt, out, ws, (hipStream_t)stream);
}

int32_t sdm_select_from_scores(const sdm_dims* d, const float* scores, int32_t* idx_w,
                               float* wt_w, int32_t* idx_r, float* wt_r, void* ws,
                               size_t ws_bytes, void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if (!scores || !idx_w || !wt_w || !idx_r || !wt_r) return SDM_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx_w) || !aligned16(wt_w) || !aligned16(idx_r) ||
      !aligned16(wt_r) || (ws && !aligned16(ws)))
    return SDM_ERR_ALIGN;
  (void)ws_bytes;  // the ranking needs no workspace (sdm_workspace_bytes returns 0)
  TimingScope timing(d);
  (void)hipGetLastError();
  return hip_status(
      launch_select(*d, scores, dv.M, 0, idx_w, wt_w, idx_r, wt_r, (hipStream_t)stream));
}

int32_t sdm_scan(const sdm_dims* d, const sdm_sel* in, const float* norm_w, void* state,
                 float* out, float* y_raw, void* ws, size_t ws_bytes, void* stream) {
  return scan_entry(d, in, norm_w, nullptr, state, nullptr, out, y_raw, ws, ws_bytes, stream,
                    false);
}

int32_t sdm_scan_train(const sdm_dims* d, const sdm_sel* in, const float* norm_w, float* state,
                       float* out, float* y_raw, void* log, float* log_scale, void* ws,
                       size_t ws_bytes, void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if ((st = check_train_flags(d)) != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if ((st = check_sel(in, false)) != SDM_OK) return st;
  const int32_t fmt = log_format(d);
  if (!state || !out || !y_raw || !log || (fmt != LOG_F32 && !log_scale)) return SDM_ERR_NULL;
  if (!aligned16(state) || !aligned16(out) || !aligned16(y_raw) || !aligned16(log) ||
      (norm_w && !aligned16(norm_w)) || (log_scale && !aligned16(log_scale)))
    return SDM_ERR_ALIGN;
  const sdm_dims dd = train_dims(d);
  const size_t need = align_up(scan_workspace_bytes(dd, true));
  if (need && (!ws || ws_bytes < need)) return SDM_ERR_WORKSPACE;
  if (need && !aligned16(ws)) return SDM_ERR_ALIGN;
  ScanArgs a = scan_args(&dd, dv, in, norm_w, state, out, y_raw);
  a.log = log;
  a.log_scale = log_scale;
  a.log_fmt = fmt;
  TimingScope timing(d);
  (void)hipGetLastError();
  return hip_status(launch_scan(dd, a, ws, ws_bytes, (hipStream_t)stream));
}

int32_t sdm_scan_backward(const sdm_dims* d, const sdm_sel* in, const float* norm_w,
                          float* state, float* d_state, const float* y_raw, const void* log,
                          const float* log_scale, const float* d_out, const sdm_scan_grads* g,
                          void* ws, size_t ws_bytes, void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if ((st = check_train_flags(d)) != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if ((st = check_sel(in, false)) != SDM_OK) return st;
  const int32_t fmt = log_format(d);
  if (!state || !d_state || !y_raw || !log || !d_out || !g || (fmt != LOG_F32 && !log_scale))
    return SDM_ERR_NULL;
  if (!g->d_wt_w || !g->d_wt_r || !g->d_v || !g->d_gate || !g->d_alpha || !g->d_beta)
    return SDM_ERR_NULL;
  const void* ptrs[] = {state, d_state, y_raw, log, d_out, g->d_wt_w, g->d_wt_r, g->d_v,
                        g->d_gate, g->d_alpha, g->d_beta};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDM_ERR_ALIGN;
  if ((norm_w && !aligned16(norm_w)) || (g->d_norm_w && !aligned16(g->d_norm_w)) ||
      (log_scale && !aligned16(log_scale)))
    return SDM_ERR_ALIGN;
  const size_t need = backward_ws_bytes(d);
  if (!ws || ws_bytes < need) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_ALIGN;
  ScanBackArgs a;
  a.idx_w = in->idx_w;
  a.wt_w = in->wt_w;
  a.idx_r = in->idx_r;
  a.wt_r = in->wt_r;
  a.v = in->v;
  a.gate = in->gate;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.norm_w = norm_w;
  a.state = state;
  a.d_state = d_state;
  a.y_raw = y_raw;
  a.log = log;
  a.log_scale = log_scale;
  a.log_fmt = fmt;
  a.d_out = d_out;
  a.g_wt_w = g->d_wt_w;
  a.g_wt_r = g->d_wt_r;
  a.g_v = g->d_v;
  a.g_gate = g->d_gate;
  a.g_alpha = g->d_alpha;
  a.g_beta = g->d_beta;
  a.g_gamma_part = static_cast<float*>(ws);
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.N = (int32_t)dv.N;
  a.W = d->W;
  a.R = d->R;
  a.d_v = d->d_v;
  a.eps = d->eps;
  TimingScope timing(d);
  (void)hipGetLastError();
  if (d->flags & SDM_FLAG_DELTA_GDN)
    return hip_status(gdn_back_uses_chunk(*d)
                          ? launch_chunk_backward(*d, a, g->d_norm_w, ws, (hipStream_t)stream)
                          : launch_gdn_slice_backward(*d, a, g->d_norm_w, ws, (hipStream_t)stream));
  if (backward_uses_stream(*d))
    return hip_status(launch_stream_backward(*d, a, g->d_norm_w, ws, (hipStream_t)stream));
  return hip_status(launch_scan_backward(a, g->d_norm_w, (hipStream_t)stream));
}

int32_t sdm_select_backward(const sdm_dims* d, const sdm_sel* fwd, const void* x,
                            const void* w_proj, const float* A, const float* b_dt,
                            const sdm_select_grads* g, float* d_y, float* d_A, float* d_b_dt,
                            void* ws, size_t ws_bytes, void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if (!fwd || !g) return SDM_ERR_NULL;
  const void* req[] = {fwd->idx_w, fwd->wt_w, fwd->idx_r, fwd->wt_r, fwd->alpha, fwd->beta,
                       fwd->gate, x, w_proj, A, b_dt, g->d_wt_w, g->d_wt_r, g->d_v,
                       g->d_gate, g->d_alpha, g->d_beta, d_y, d_A, d_b_dt};
  for (const void* p : req)
    if (!p) return SDM_ERR_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return SDM_ERR_ALIGN;
  const size_t need = align_up(select_backward_ws_bytes(*d));
  if (!ws || ws_bytes < need) return SDM_ERR_WORKSPACE;
  if (!aligned16(ws)) return SDM_ERR_ALIGN;
  // one (token, head) per workgroup; its dY row is staged in LDS
  if ((int64_t)dv.M * d->H > INT32_MAX || dv.P * 4 > 60 * 1024) return SDM_ERR_UNSUPPORTED;
  TimingScope timing(d);
  (void)hipGetLastError();
  return hip_status(launch_select_backward(*d, *fwd, x, w_proj, A, b_dt, *g, d_y, d_A, d_b_dt,
                                           ws, (hipStream_t)stream));
}

int32_t sdm_scan_shared_m0(const sdm_dims* d, const sdm_sel* in, const float* norm_w,
                           const void* m0, void* state, uint32_t* touched, float* out,
                           float* y_raw, void* ws, size_t ws_bytes, void* stream) {
  return scan_entry(d, in, norm_w, m0, state, touched, out, y_raw, ws, ws_bytes, stream, true);
}

int32_t sdm_slot_histogram(const sdm_dims* d, const int32_t* idx_w, int32_t* counts,
                           void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  if (dv.M == 0) return SDM_OK;
  if (!idx_w || !counts) return SDM_ERR_NULL;
  if (!aligned16(idx_w) || !aligned16(counts)) return SDM_ERR_ALIGN;
  TimingScope timing(d);
  (void)hipGetLastError();
  return hip_status(launch_slot_histogram(*d, dv.N, idx_w, counts, (hipStream_t)stream));
}

int32_t sdm_forward(const sdm_dims* d, const void* x, const void* w_proj, const float* A,
                    const float* b_dt, const float* norm_w, void* state, float* out,
                    const sdm_sel* debug, void* ws, size_t ws_bytes, void* stream) {
  return forward_entry(d, x, w_proj, A, b_dt, norm_w, nullptr, state, nullptr, out, debug, ws,
                       ws_bytes, stream, false);
}

int32_t sdm_forward_shared_m0(const sdm_dims* d, const void* x, const void* w_proj,
                              const float* A, const float* b_dt, const float* norm_w,
                              const void* m0, void* state, uint32_t* touched, float* out,
                              void* ws, size_t ws_bytes, void* stream) {
  return forward_entry(d, x, w_proj, A, b_dt, norm_w, m0, state, touched, out, nullptr, ws,
                       ws_bytes, stream, true);
}

int32_t sdm_forward_noalloc(const sdm_dims* d, const void* x, const void* w_proj,
                            const float* A, const float* b_dt, const float* norm_w, void* state,
                            float* out, void* stream) {
  Derived dv;
  int32_t st = check_dims(d, &dv);
  if (st != SDM_OK) return st;
  // the timing record creates HIP events on first use: not part of this entry
  if (d->flags & SDM_FLAG_TIMING) return SDM_ERR_UNSUPPORTED;
  if (dv.M == 0) return SDM_OK;
  if (!x || !w_proj || !A || !b_dt || !state || !out) return SDM_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_proj) || !aligned16(A) || !aligned16(b_dt) ||
      !aligned16(state) || !aligned16(out) || (norm_w && !aligned16(norm_w)))
    return SDM_ERR_ALIGN;
  const size_t need = sdm_workspace_bytes(d, SDM_ENTRY_FORWARD);
  if (need > (size_t)SDM_NOALLOC_SCRATCH_BYTES) return SDM_ERR_WORKSPACE;
  void* ws = scratch_address();  // validated arguments only: the first call resolves it
  if (!ws) return SDM_ERR_HIP;
  return forward_entry(d, x, w_proj, A, b_dt, norm_w, nullptr, state, nullptr, out, nullptr, ws,
                       (size_t)SDM_NOALLOC_SCRATCH_BYTES, stream, false);
}

}  // extern "C"
