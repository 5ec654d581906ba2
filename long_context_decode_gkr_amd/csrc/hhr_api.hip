// C ABI of the HHR decode library: argument validation, workspace planning, launch order.
// Declarations and the full contract are in include/hhr.h.
#include <math.h>
#include <stdarg.h>
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hhr.h"
#include "hhr_launch.h"

using namespace hhr;

namespace hhr {

bool trace_on() {
  static const bool on = [] {
    const char* v = getenv("HHR_TRACE");
    return v && *v && strcmp(v, "0") != 0;
  }();
  return on;
}

void trace_printf(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  fputs("[hhr] ", stderr);
  vfprintf(stderr, fmt, ap);
  fputc('\n', stderr);
  va_end(ap);
}

// Scratch memory of the allocation-free decode entry point: one copy per device, at that
// device's own address (resolved once per device with hipGetSymbolAddress; the array's name in
// host code is only a handle, never a device address).
__device__ __align__(256) unsigned char scratch[HHR_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The current device's scratch address, resolved on the first call on that device.
static hhr_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HHR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HHR_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HHR_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return HHR_OK;
}

}  // namespace hhr

namespace {

constexpr int kHeadDim = 128;

bool dtype_ok(int32_t t) { return t == HHR_F32 || t == HHR_BF16; }

// Checks the shape fields and fills `s`. Returns HHR_OK or the first problem found.
hhr_status check_dims(const hhr_dims* d, Shape* s) {
  if (!d) return HHR_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->page_size <= 0 || d->hash_bits <= 0 || d->max_seq_len <= 0)
    return HHR_ERR_INVALID_ARG;
  if (!dtype_ok(d->kv_dtype) || !dtype_ok(d->q_dtype) || !dtype_ok(d->summary_dtype))
    return HHR_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return HHR_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HHR_ERR_UNSUPPORTED;
  if (d->head_dim != kHeadDim) return HHR_ERR_UNSUPPORTED;
  if (d->page_size != 16 && d->page_size != 32) return HHR_ERR_UNSUPPORTED;
  if (d->hash_bits != 128 && d->hash_bits != 256) return HHR_ERR_UNSUPPORTED;
  if (d->max_seq_len % (4 * d->page_size) != 0) return HHR_ERR_UNSUPPORTED;
  if (d->max_seq_len / d->page_size > HHR_MAX_PAGES) return HHR_ERR_CAPACITY;
  if (int64_t(d->batch) * d->num_q_heads > 65535 * 16 || d->batch > 65535 ||
      d->num_q_heads > 65535)
    return HHR_ERR_CAPACITY;
  s->B = d->batch;
  s->Hq = d->num_q_heads;
  s->Hkv = d->num_kv_heads;
  s->G = G;
  s->S = d->page_size;
  s->NB = d->hash_bits;
  s->NW = d->hash_bits / 32;
  s->Lmax = d->max_seq_len;
  s->Pmax = d->max_seq_len / d->page_size;
  s->kv_bf16 = d->kv_dtype == HHR_BF16;
  s->q_bf16 = d->q_dtype == HHR_BF16;
  s->sum_bf16 = d->summary_dtype == HHR_BF16;
  return HHR_OK;
}

hhr_status check_cache(const hhr_cache* c, bool need_ticket, CacheView* v) {
  if (!c) return HHR_ERR_INVALID_ARG;
  if (!c->K || !c->V || !c->page_min || !c->page_max || !c->codes || !c->seq_lens)
    return HHR_ERR_INVALID_ARG;
  if (need_ticket && !c->append_ticket) return HHR_ERR_INVALID_ARG;
  *v = CacheView{c->K, c->V, c->page_min, c->page_max, c->codes, c->seq_lens, c->append_ticket};
  return HHR_OK;
}

float softmax_scale(float given) {
  return given > 0.f ? given : float(1.0 / sqrt(double(kHeadDim)));
}

hhr_status check_params(const hhr_params* p, const Shape& s, DecodePlan* plan) {
  if (!p) return HHR_ERR_INVALID_ARG;
  const double rho = p->page_keep_ratio;
  if (!(rho > 0.0 && rho <= 1.0)) return HHR_ERR_INVALID_ARG;
  if (p->token_budget < 1) return HHR_ERR_INVALID_ARG;
  if (!isfinite(p->softmax_scale)) return HHR_ERR_INVALID_ARG;
  if (p->stages != HHR_STAGES_BOTH && p->stages != HHR_STAGES_PAGES_ONLY &&
      p->stages != HHR_STAGES_CODES_ONLY)
    return HHR_ERR_INVALID_ARG;
  if (p->group_shared != 0 && p->group_shared != 1) return HHR_ERR_INVALID_ARG;
  *plan = plan_decode(s, rho, p->token_budget, softmax_scale(p->softmax_scale),
                      static_cast<Stages>(p->stages), p->group_shared);
  return HHR_OK;
}

hhr_status hip_status(hipError_t e) { return e == hipSuccess ? HHR_OK : HHR_ERR_HIP; }

DebugView debug_view(const hhr_debug* dbg) {
  DebugView dv{};
  if (dbg) dv = DebugView{dbg->q_rot, dbg->q_code, dbg->bounds, dbg->page_ids,
                          dbg->page_count, dbg->dist, dbg->token_idx, dbg->token_count,
                          reinterpret_cast<hipEvent_t*>(dbg->kernel_events)};
  return dv;
}

}  // namespace

extern "C" {

hhr_status hhr_build_pages(const hhr_dims* dims, const hhr_cache* cache, const float* R,
                           const float* W, hhr_stream_t stream) {
  Shape s;
  CacheView c;
  hhr_status st = check_dims(dims, &s);
  if (st != HHR_OK) return st;
  if ((st = check_cache(cache, false, &c)) != HHR_OK) return st;
  if (!R || !W) return HHR_ERR_INVALID_ARG;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (s.kv_bf16) return hip_status(launch_build_mfma(s, c, R, W, hs));
  return hip_status(launch_build_fp64(s, c, R, W, hs));
}

hhr_status hhr_build_pages_fp64(const hhr_dims* dims, const hhr_cache* cache, const float* R,
                                const float* W, hhr_stream_t stream) {
  Shape s;
  CacheView c;
  hhr_status st = check_dims(dims, &s);
  if (st != HHR_OK) return st;
  if ((st = check_cache(cache, false, &c)) != HHR_OK) return st;
  if (!R || !W) return HHR_ERR_INVALID_ARG;
  return hip_status(launch_build_fp64(s, c, R, W, reinterpret_cast<hipStream_t>(stream)));
}

hhr_status hhr_append(const hhr_dims* dims, const hhr_cache* cache, const void* k_new,
                      const void* v_new, const float* R, const float* W, hhr_stream_t stream) {
  Shape s;
  CacheView c;
  hhr_status st = check_dims(dims, &s);
  if (st != HHR_OK) return st;
  if ((st = check_cache(cache, true, &c)) != HHR_OK) return st;
  if (!k_new || !v_new || !R || !W) return HHR_ERR_INVALID_ARG;
  return hip_status(launch_prep(s, c, k_new, v_new, nullptr, R, W, nullptr, nullptr, nullptr,
                                nullptr, PrepMode::kAppend, KernelTimer{nullptr, nullptr},
                                reinterpret_cast<hipStream_t>(stream)));
}

size_t hhr_decode_workspace_bytes(const hhr_dims* dims, const hhr_params* params) {
  Shape s;
  DecodePlan p;
  if (check_dims(dims, &s) != HHR_OK) return 0;
  if (check_params(params, s, &p) != HHR_OK) return 0;
  return p.total;
}

// Validation of a decode call (everything but the workspace) and its plan.
static hhr_status check_decode_call(const hhr_dims* dims, const hhr_params* params,
                                    const hhr_cache* cache, const void* k_new, const void* v_new,
                                    bool append, const void* q, const float* R, const float* W,
                                    const float* out, Shape* s, CacheView* c, DecodePlan* p) {
  hhr_status st = check_dims(dims, s);
  if (st != HHR_OK) return st;
  if ((st = check_cache(cache, append, c)) != HHR_OK) return st;
  if ((st = check_params(params, *s, p)) != HHR_OK) return st;
  if (!q || !R || !W || !out) return HHR_ERR_INVALID_ARG;
  if (append && (!k_new || !v_new)) return HHR_ERR_INVALID_ARG;
  return HHR_OK;
}

static hhr_status decode_common(const hhr_dims* dims, const hhr_params* params,
                                const hhr_cache* cache, const void* k_new, const void* v_new,
                                bool append, const void* q, const float* R, const float* W,
                                void* ws, size_t ws_bytes, float* out, const hhr_debug* dbg,
                                hhr_stream_t stream) {
  Shape s;
  CacheView c;
  DecodePlan p;
  hhr_status st = check_decode_call(dims, params, cache, k_new, v_new, append, q, R, W, out, &s,
                                    &c, &p);
  if (st != HHR_OK) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < p.total)
    return HHR_ERR_WORKSPACE;
  return hip_status(launch_decode(s, p, c, append ? k_new : nullptr, append ? v_new : nullptr, q,
                                  R, W, ws, out, debug_view(dbg),
                                  reinterpret_cast<hipStream_t>(stream)));
}

hhr_status hhr_decode(const hhr_dims* dims, const hhr_params* params, const hhr_cache* cache,
                      const void* q, const float* R, const float* W, void* ws, size_t ws_bytes,
                      float* out, const hhr_debug* dbg, hhr_stream_t stream) {
  return decode_common(dims, params, cache, nullptr, nullptr, false, q, R, W, ws, ws_bytes, out,
                       dbg, stream);
}

hhr_status hhr_append_decode(const hhr_dims* dims, const hhr_params* params,
                             const hhr_cache* cache, const void* k_new, const void* v_new,
                             const void* q, const float* R, const float* W, void* ws,
                             size_t ws_bytes, float* out, const hhr_debug* dbg,
                             hhr_stream_t stream) {
  return decode_common(dims, params, cache, k_new, v_new, true, q, R, W, ws, ws_bytes, out, dbg,
                       stream);
}

hhr_status hhr_decode_scratch(const hhr_dims* dims, const hhr_params* params,
                              const hhr_cache* cache, const void* q, const float* R,
                              const float* W, float* out, const hhr_debug* dbg,
                              hhr_stream_t stream) {
  Shape s;
  CacheView c;
  DecodePlan p;
  hhr_status st = check_decode_call(dims, params, cache, nullptr, nullptr, false, q, R, W, out,
                                    &s, &c, &p);
  if (st != HHR_OK) return st;
  if (p.total > HHR_SCRATCH_BYTES) {
    if (trace_on())
      trace_printf("hhr_decode_scratch: these shapes need %zu B of workspace, more than the "
                   "%zu B of scratch", p.total, size_t(HHR_SCRATCH_BYTES));
    return HHR_ERR_CAPACITY;
  }
  void* ws = nullptr;
  if ((st = current_scratch(&ws)) != HHR_OK) return st;
  return hip_status(launch_decode(s, p, c, nullptr, nullptr, q, R, W, ws, out, debug_view(dbg),
                                  reinterpret_cast<hipStream_t>(stream)));
}

size_t hhr_dense_workspace_bytes(const hhr_dims* dims) {
  Shape s;
  if (check_dims(dims, &s) != HHR_OK) return 0;
  return dense_workspace_bytes(s);
}

hhr_status hhr_dense_decode(const hhr_dims* dims, const hhr_cache* cache, const void* q,
                            float softmax_scale_in, void* ws, size_t ws_bytes, float* out,
                            const hhr_debug* dbg, hhr_stream_t stream) {
  Shape s;
  hhr_status st = check_dims(dims, &s);
  if (st != HHR_OK) return st;
  if (!cache || !cache->K || !cache->V || !cache->seq_lens) return HHR_ERR_INVALID_ARG;
  if (!q || !out || !isfinite(softmax_scale_in)) return HHR_ERR_INVALID_ARG;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < dense_workspace_bytes(s))
    return HHR_ERR_WORKSPACE;
  const CacheView c{cache->K, cache->V, nullptr, nullptr, nullptr, cache->seq_lens, nullptr};
  DebugView dv{};
  if (dbg) dv.events = reinterpret_cast<hipEvent_t*>(dbg->kernel_events);
  return hip_status(launch_dense(s, c, q, softmax_scale(softmax_scale_in), ws, out, dv,
                                 reinterpret_cast<hipStream_t>(stream)));
}

const char* hhr_status_string(hhr_status status) {
  switch (status) {
    case HHR_OK: return "ok";
    case HHR_ERR_INVALID_ARG: return "invalid argument";
    case HHR_ERR_UNSUPPORTED: return "unsupported shape or type";
    case HHR_ERR_CAPACITY: return "size exceeds a documented maximum";
    case HHR_ERR_WORKSPACE: return "workspace too small or misaligned";
    case HHR_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

}  // extern "C"
