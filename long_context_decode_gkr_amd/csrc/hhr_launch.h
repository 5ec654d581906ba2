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
  hipEvent_t* events;  // NULL or 2 kStepKernels events: start and stop of each kernel
};

// Start and stop events of one kernel's execution; both NULL for a plain launch.
struct KernelTimer {
  hipEvent_t start, stop;
};
// Event slots of a decode step: 0 preparation, 1 page bound, 2 selection scan, 3 selection
// emission, 4 attention, 5 merge (12 events: start and stop of each).
constexpr int kStepKernels = 6;
inline KernelTimer kernel_timer(const DebugView& d, int k) {
  return d.events ? KernelTimer{d.events[2 * k], d.events[2 * k + 1]} : KernelTimer{nullptr, nullptr};
}
// HHR_TRACE: when the environment variable is set to anything but "0" (read once per process),
// every launch and every decode step's plan and byte counts are logged to stderr.
bool trace_on();
void trace_printf(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Launch on stream st and return this launch's own status (not a sticky error left by an earlier
// call); with a timer the runtime records its events around the kernel itself.
template <typename... KArgs>
inline hipError_t launch_args(const void* f, dim3 grid, dim3 block, hipStream_t st,
                              KernelTimer tm, KArgs... v) {
  void* argv[] = {static_cast<void*>(&v)...};
  if (tm.start) return hipExtLaunchKernel(f, grid, block, argv, 0, st, tm.start, tm.stop, 0);
  return hipLaunchKernel(f, grid, block, argv, 0, st);
}
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                                hipStream_t st, KernelTimer tm, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  // each argument converted to the kernel's parameter type before its address is taken
  const hipError_t e = launch_args<KArgs...>(reinterpret_cast<const void*>(kernel), grid, block,
                                             st, tm, args...);
  if (trace_on())
    trace_printf("launch %s grid (%u, %u, %u) block %u stream %p timed %d: %s", name, grid.x,
                 grid.y, grid.z, block.x, static_cast<void*>(st), tm.start ? 1 : 0,
                 hipGetErrorString(e));
  return e;
}

// Which stages choose the attended tokens (the stage-wise ablation of the method).
enum class Stages { kBoth = 0, kPagesOnly = 1, kCodesOnly = 2 };

// Page capacity (HHR_MAX_PAGES) and the page counts of one selection slice.
constexpr int kMaxPages = 16384;
constexpr int kSlicePages = 512;      // most kept pages per selection slice
constexpr int kMinSlicePages = 8;     // fewest, when the step would not fill the GPU otherwise
constexpr int kUnitSlots = 32768;     // most candidates of a one-workgroup-per-unit selection

// Workspace carve-up of one decode call (byte offsets from the workspace base).
struct DecodePlan {
  Stages stages;
  int shared;      // one page and token selection per KV head for its G query heads
  int kcap;        // most tokens attended per (b, h): the token budget clamped to max_seq_len,
                   // or (pages only) every token of the largest kept page set
  int istride;     // per-unit stride of the index list: kcap entries + one trash entry per lane
  int chunk;       // tokens per attention workgroup
  int nsplit;      // attention workgroups per (b, h)
  int kpages;      // most kept pages per selection unit, min(Pmax, max(1, ceil(rho Pmax)))
  int unit_select; // one workgroup per unit selects (else the sliced form)
  int unit_threads;  // its workgroup size: 256, 512 or 1024
  int nsl;         // selection slices per unit (sliced form)
  int dstride;     // per-unit stride of the candidate distances (elements, a multiple of 16)
  double rho;
  float scale;
  size_t off_qrot, off_qcode, off_U, off_idx, off_cnt, off_part, off_pages, off_dist, off_hist,
      total;
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
// Selection of the attended tokens (select_scan_kernel, select_emit_kernel), grid
// (nsl, units, B): the exact page cut, the Hamming distances of the kept pages' keys and one
// histogram per slice, then the token threshold and the ordered emission.
struct SelectArgs {
  const uint32_t* qcode;  // [B][Hq][NW]
  const float* U;         // [units][Pmax] page bounds; NULL when every page is kept
  int32_t* pages;         // [units][kpages] kept pages, ascending
  void* dist;             // [units][dstride] distance per candidate slot (u8, or u16 for 256 bits)
  int32_t* hist;          // [units][nsl][NB + 1]
  int32_t* idx;           // [units][istride]
  int32_t* cnt;           // [units]
  double rho;
  int kcap, istride, nsl, kpages, dstride;
  int appended;           // a token is appended in this step (seq_lens is advanced at its end)
  int fine;               // 0: no Hamming ranking, every candidate is taken (coarse stage only)
  int shared;             // units are KV heads (group-shared selection)
};
// Slices per unit for kpages kept pages at most over `units` selection units.
int select_slices(int kpages, int units, bool all_kept);
// unit_threads: the workgroup size of the one-workgroup-per-unit form (1024, or 256 / 512 where
// the pages fit 16 per thread), or 0 for the sliced form.
hipError_t launch_select(const Shape& s, const CacheView& c, const SelectArgs& a,
                         const DebugView& dbg, int unit_threads, hipStream_t st);
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
