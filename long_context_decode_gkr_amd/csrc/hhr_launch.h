// Internal launch interface between the C-ABI host layer and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hhr {

struct Shape {
  int B, Hq, Hkv, G, S, NB, NW, Lmax, Pmax;
  int kv_bf16, q_bf16;
  int sum_bf16;       // page extrema stored as bf16 rounded outward (else fp32)
};

struct CacheView {
  void* K;
  void* V;
  void* pmin;         // fp32 or (sum_bf16) bf16 bits, [B][Hkv][128][Pmax]
  void* pmax;
  uint32_t* codes;
  int32_t* seq_lens;
  int32_t* ticket;
};

struct DebugView {
  float* q_rot;
  uint32_t* q_code;
  float* bounds;
  int32_t* page_ids;
  int32_t* page_count;
  uint16_t* dist;
  int32_t* token_idx;
  int32_t* token_count;
  hipEvent_t* events;  // NULL or 10 events: start and stop of each of the five kernels
};

// Start and stop events of one kernel's execution; both NULL for a plain launch.
struct KernelTimer {
  hipEvent_t start, stop;
};
inline KernelTimer kernel_timer(const DebugView& d, int k) {
  return d.events ? KernelTimer{d.events[2 * k], d.events[2 * k + 1]} : KernelTimer{nullptr, nullptr};
}
// Launch on stream st; with a timer the runtime records its events around the kernel itself.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t st, KernelTimer tm,
                          Args... args) {
  if (tm.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, tm.start, tm.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// Which stages choose the attended tokens (the stage-wise ablation of the method).
enum class Stages { kBoth = 0, kPagesOnly = 1, kCodesOnly = 2 };

// Workspace carve-up of one decode call (byte offsets from the workspace base).
struct DecodePlan {
  Stages stages;
  int shared;      // one page and token selection per KV head for its G query heads
  int kcap;        // most tokens attended per (b, h): the token budget clamped to max_seq_len,
                   // or (pages only) every token of the largest kept page set
  int istride;     // per-(b, h) stride of the index list: kcap entries + one trash entry per lane
  int chunk;       // tokens per attention workgroup
  int nsplit;      // attention workgroups per (b, h)
  double rho;
  float scale;
  size_t off_qrot, off_qcode, off_U, off_idx, off_cnt, off_part, off_dist, off_hist, total;
};

DecodePlan plan_decode(const Shape& s, double rho, int k, float scale, Stages stages,
                       int shared);

hipError_t launch_build_fp64(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st);
hipError_t launch_build_mfma(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st);
// Preparation kernel.
//   kAppend (hhr_append): appends k_new / v_new: K/V rows, page extrema, key code, then
//     advances seq_lens.
//   kDecode (first kernel of a decode step): q~ of every query head into qrot [B][Hq][128],
//     the query codes into qcode [B][Hq][NW] and, when k_new != NULL, the appended token's K/V
//     rows, page extrema and code (seq_lens is advanced by the step's last kernel).
enum class PrepMode { kAppend, kDecode };
hipError_t launch_prep(const Shape& s, const CacheView& c, const void* k_new, const void* v_new,
                       const void* q, const float* R, const float* W, float* qrot,
                       uint32_t* qcode, float* dbg_qrot, uint32_t* dbg_qcode, PrepMode mode,
                       KernelTimer tm, hipStream_t st);
// Fine stage over every token (fine-stage-only variant): distances and per-slice histograms,
// then the threshold and the ordered emission of the selected tokens, kScanTok tokens per
// workgroup in both kernels.
constexpr int kScanTok = 4096;
struct ScanArgs {
  const uint32_t* qcode;  // [B][Hq][NW]
  void* dist;             // [units][Lmax]: one byte per distance (two for 256-bit codes)
  int32_t* hist;          // [units][nsl][NB + 1]
  int32_t* idx;           // [units][istride]
  int32_t* cnt;           // [units]
  int kcap, istride, nsl, appended, shared;
};
int scan_slices(const Shape& s);
hipError_t launch_scan_select(const Shape& s, const CacheView& c, const ScanArgs& a,
                              const DebugView& dbg, hipStream_t st);
// Merge of split-K attention partials [B][Hq][nsplit][128 + 2] (o, m, l) into out
// [B][Hq][128]; with `appended` it also advances seq_lens (the sparse step's last kernel).
hipError_t launch_combine(const Shape& s, const float* part, int nsplit, float* out,
                          int32_t* seq_lens, int appended, KernelTimer tm, hipStream_t st);
// Attention of the G query heads of every KV head over that KV head's list of selected tokens
// (group-shared selection), each gathered row read once: kGatherChunk list positions per
// workgroup, partials [B][Hq][nsplit][128 + 2] for launch_combine.
constexpr int kGatherChunk = 128;
hipError_t launch_attn_gather(const Shape& s, const CacheView& c, const void* q, float scale,
                              const int32_t* idx, const int32_t* cnt, int istride, float* part,
                              int nsplit, KernelTimer tm, hipStream_t st);
// Dense attention over every token (split-K, grouped-query sharing) and its merge; ws holds
// dense_workspace_bytes(s) bytes of partials. Timers: events 0-1 (attention), 2-3 (merge).
size_t dense_workspace_bytes(const Shape& s);
hipError_t launch_dense(const Shape& s, const CacheView& c, const void* q, float scale,
                        void* ws, float* out, const DebugView& dbg, hipStream_t st);
// The decode step, with the append of k_new / v_new folded into its kernels when given.
hipError_t launch_decode(const Shape& s, const DecodePlan& p, const CacheView& c,
                         const void* k_new, const void* v_new, const void* q, const float* R,
                         const float* W, void* ws, float* out, const DebugView& dbg,
                         hipStream_t st);

}  // namespace hhr
