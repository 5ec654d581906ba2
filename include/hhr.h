/*
 * hhr.h -- C ABI of the HHR (Hierarchical Hash Retrieval) sparse-attention decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation"
 * (arXiv 2610.01230). One decode step, for every sequence b and query head h, runs
 *   coarse stage (GKR, §3.3.1): rotate the query, q~ = q R (Eq. 4); bound every page p of the
 *     head's rotated keys by U = sum_j max(q~_j l_j, q~_j u_j) (Eq. 3), where l, u are the
 *     page's per-dimension minimum and maximum of the rotated keys; keep the best pages;
 *   fine stage (LHP, §3.3.2): hash the query, c = sign(q W) (Eq. 1, Eq. 10), take the Hamming
 *     distance (Eq. 2) to the stored code of every key in the kept pages and keep the closest
 *     keys;
 *   attention: exact softmax attention of q over the kept keys (§1).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller. The library allocates no
 *     memory, keeps no state between calls, never synchronises the host, and enqueues all work
 *     on `stream` (a hipStream_t; NULL means the null stream). Calls on different streams that
 *     touch disjoint caches and workspaces may run concurrently.
 *   - Arguments are validated on the host before anything is enqueued; an invalid call
 *     returns an error status and enqueues nothing. Values that live in device memory
 *     (seq_lens) cannot be checked on the host: kernels clamp them to [0, max_seq_len].
 *   - A failed kernel launch returns HHR_ERR_HIP (each launch's own status is checked, so an
 *     error left by an earlier, unrelated call is not reported). The launches before the failed
 *     one stay enqueued: after HHR_ERR_HIP from hhr_append_decode the new token's K/V rows,
 *     page extrema and code may already be written while seq_lens was not advanced, and after
 *     HHR_ERR_HIP from hhr_append the same holds when the sequence's last workgroup did not
 *     run; rebuild the index (hhr_build_pages) before the next append or decode. Faults inside
 *     a kernel surface at the caller's next synchronisation.
 *   - Head dimension d is 128. Query head h reads KV head g = h / (Hq / Hkv) (grouped-query
 *     attention); the rotation R_g and projection W_g belong to the KV head.
 *   - Rows are row vectors: q~ = q R_g, z = x W_g.
 *   - Inputs must be finite.
 *
 * Layouts (row-major, innermost last; Pmax = max_seq_len / page_size, nw = hash_bits / 32)
 *   K, V       [B][Hkv][max_seq_len][128]   kv_dtype
 *   page_min   [B][Hkv][128][Pmax]          summary_dtype, channel-major ("SoA"): entry
 *   page_max   [B][Hkv][128][Pmax]          [b][g][j][p] is the min / max over the page's
 *                                            valid tokens of dimension j of the rotated key
 *                                            k~ = k R_g (fp32 values of the fp32-rounded k~; as
 *                                            bf16, the min rounded toward -inf and the max
 *                                            toward +inf, so Eq. 3 stays an upper bound)
 *   codes      [B][Hkv][max_seq_len][nw]    uint32; bit c of a key's code sits in word c / 32
 *                                            at bit position c % 32; bit c = 1 iff the exact
 *                                            real value of (k W_g)_c is > 0
 *   seq_lens   [B]                          int32, number of valid tokens per sequence
 *   R          [Hkv][128][128]              fp32, orthogonal (caller-supplied)
 *   W          [Hkv][128][hash_bits]        fp32 (caller-supplied)
 *   q          [B][Hq][128]                 q_dtype
 *   out        [B][Hq][128]                 fp32
 */
#ifndef HHR_H
#define HHR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hhr_stream_t; /* the same type as hipStream_t */
typedef struct ihipEvent_t* hhr_event_t;   /* the same type as hipEvent_t */

typedef enum {
  HHR_OK = 0,
  HHR_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, malformed value          */
  HHR_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the kernels implement         */
  HHR_ERR_CAPACITY = 3,     /* a size exceeds a documented maximum                        */
  HHR_ERR_WORKSPACE = 4,    /* workspace too small or misaligned                          */
  HHR_ERR_HIP = 5           /* a HIP launch or runtime call failed                        */
} hhr_status;

typedef enum { HHR_F32 = 0, HHR_BF16 = 1 } hhr_dtype;

/* Shapes. Supported: head_dim = 128; num_q_heads = G * num_kv_heads with G in {1, 2, 4, 8};
 * page_size in {16, 32}; hash_bits in {128, 256}; max_seq_len a multiple of 4 * page_size with
 * max_seq_len / page_size <= HHR_MAX_PAGES; kv_dtype, q_dtype and summary_dtype in {HHR_F32,
 * HHR_BF16}. */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t hash_bits;
  int32_t max_seq_len;
  int32_t kv_dtype;     /* hhr_dtype of K and V (and k_new, v_new) */
  int32_t q_dtype;      /* hhr_dtype of q */
  int32_t summary_dtype;  /* hhr_dtype of page_min / page_max: HHR_F32, or HHR_BF16 rounded
                             outward (half the bytes the page-bound kernel streams) */
} hhr_dims;

#define HHR_MAX_PAGES 16384

/* Budgets of one decode step.
 * page_keep_ratio rho in (0, 1]: a sequence with L tokens has P = ceil(L / page_size) pages and
 *   keeps n_keep = min(P, max(1, ceil(rho * P))) of them, rho * P being one IEEE double multiply
 *   (the threshold c_h of §3.3.1, read as "keep the n_keep largest bounds"; the paper's default
 *   candidate budget is 30 %, Appendix A). Ties in U go to the lower page index.
 * token_budget k >= 1: the min(k, #candidates) candidates of smallest (Hamming distance,
 *   token position) are attended to (§3.3.2; the paper's default is 1.5 % of the context).
 * softmax_scale: logits are scale * q.k; a value <= 0 selects 1/sqrt(128) rounded to fp32.
 * stages: which stages choose the attended keys (hhr_stages; the stage-wise ablation of
 *   Appendix C, Table 8). The rotation R is an input, so the "no rotation" variant of the coarse stage is
 *   R = I (the plain per-channel min/max bound). */
typedef enum {
  HHR_STAGES_BOTH = 0,        /* coarse then fine: the method                                  */
  HHR_STAGES_PAGES_ONLY = 1,  /* coarse only: every token of the kept pages is attended;
                                 token_budget is not used                                     */
  HHR_STAGES_CODES_ONLY = 2   /* fine only: every page is a candidate (page_keep_ratio is not
                                 used, no page bound is computed, dbg->bounds stays untouched) */
} hhr_stages;

typedef struct {
  double page_keep_ratio;
  int32_t token_budget;
  float softmax_scale;
  int32_t stages;       /* hhr_stages */
  int32_t group_shared; /* 0: each query head selects its own pages and tokens (the method as
                           read); 1: one selection per KV head for its G query heads: a page's
                           bound is the largest of the heads' bounds, a token's distance the
                           smallest of their distances (a quarter of the K/V rows gathered
                           at G = 4) */
} hhr_params;

/* The KV cache and its derived index (page extrema and key codes). All device pointers.
 * append_ticket is a [B] int32 array that must be zero when the cache is created; every call
 * leaves it zero again. */
typedef struct {
  void* K;
  void* V;
  float* page_min;
  float* page_max;
  uint32_t* codes;
  int32_t* seq_lens;
  int32_t* append_ticket;
} hhr_cache;

/* Optional intermediate outputs of hhr_decode, for testing. Every pointer may be NULL.
 *   q_rot       [B][Hq][128]        fp32  q~ = q R_g (Eq. 4)
 *   q_code      [B][Hq][nw]         query code (Eq. 1 / Eq. 10)
 *   bounds      [B][Hq][Pmax]       U of every page p < P_b (Eq. 3); other entries untouched
 *   page_ids    [B][Hq][Pmax]       the kept pages, ascending, in the first n_keep entries
 *   page_count  [B][Hq]             n_keep
 *   dist        [B][Hq][max_seq_len] Hamming distance of candidate slot i, i.e. of token
 *                                   page_ids[i / S] * S + i % S, for i < n_keep * S; 0xFFFF
 *                                   for a slot past the end of the sequence
 *   token_idx   [B][Hq][kcap]       the selected token positions, ascending; kcap =
 *                                   min(token_budget, max_seq_len), or with
 *                                   HHR_STAGES_PAGES_ONLY min(max(1, ceil(rho Pmax)) *
 *                                   page_size, max_seq_len)
 *   token_count [B][Hq]             how many were selected
 *   With group_shared, page_ids, page_count, dist, token_idx and token_count hold one row per
 *   (b, KV head) instead, at row b * Hkv + g; bounds stays per query head.
 *   kernel_events  NULL or 12 caller-created events: the start and stop of each of the six
 *                  kernel slots of a decode step, in launch order, recorded by the runtime around
 *                  the kernel's own execution (hipExtLaunchKernel), so that their elapsed times
 *                  are the kernels' durations: (0) the preparation kernel (query rotations and
 *                  codes; in hhr_append_decode also the new token's K/V rows, page extrema and
 *                  code),
 *                  (1) the page-bound kernel, (2) the selection (page cut, Hamming distances of
 *                  the kept pages' keys and, when it is one kernel, the token threshold and the
 *                  selected positions), (3) the second selection kernel of the sliced form
 *                  (token threshold, selected positions), (4) the attention kernel, and (5) the
 *                  kernel that merges the attention partials (and commits the append). A slot
 *                  whose kernel does not run in this configuration (the page bound with
 *                  HHR_STAGES_CODES_ONLY, slot 3 when the selection is one kernel) gets its two
 *                  events recorded back to back.
 *   The selection runs as one workgroup per selection unit when the largest kept page set's
 *   tokens fit its cache (at most 32768 candidates) and the stages include the coarse one, and
 *   otherwise in slices of the kept pages over two kernels; both give identical results. For
 *   testing, the environment variable HHR_SELECT=sliced forces the sliced form,
 *   HHR_SELECT_SLICES=n (1..1024) its slice count, and HHR_SELECT_THREADS=256, 512 or 1024
 *   the first form's workgroup size (by default 512 up to 2048 pages of max_seq_len, else
 *   1024; a smaller size is used only up to 16 pages per thread). The page-bound kernel's
 *   workgroups cover 64, 128 or 256 pages (the largest that still gives every compute unit a
 *   workgroup); HHR_BOUND_PAGES=64, 128 or 256 forces one, with identical results. */
typedef struct {
  float* q_rot;
  uint32_t* q_code;
  float* bounds;
  int32_t* page_ids;
  int32_t* page_count;
  uint16_t* dist;
  int32_t* token_idx;
  int32_t* token_count;
  hhr_event_t* kernel_events;
} hhr_debug;

/* Index build (prefill; §3.3.1 paging and page extrema, §3.3.2 key codes).
 * For every sequence b and KV head g, over tokens t < seq_lens[b] of K: computes k~ = k R_g,
 * writes page_min / page_max of every page p < ceil(seq_lens[b] / page_size) (a partial last
 * page covers only its valid tokens) and the code of every token t < seq_lens[b]. Entries past
 * the end are left untouched, and so are V, seq_lens and append_ticket.
 * bf16 keys go through matrix-core (MFMA) GEMMs of K against [R_g | W_g]; fp32 keys through
 * the fp64 vector path of hhr_build_pages_fp64. Codes are exact in both (see `codes` above);
 * page extrema are within a few fp32 ulps of the correctly rounded rotated keys. */
hhr_status hhr_build_pages(const hhr_dims* dims, const hhr_cache* cache, const float* R,
                           const float* W, hhr_stream_t stream);

/* The same index build on the fp64 vector units for any kv_dtype: rotated keys are the fp64
 * dot products rounded once to fp32; codes are certified from fp64 sums of exact products and
 * recomputed exactly where the fp64 sum is too close to zero. */
hhr_status hhr_build_pages_fp64(const hhr_dims* dims, const hhr_cache* cache, const float* R,
                                const float* W, hhr_stream_t stream);

/* Append one token per (sequence, KV head). k_new, v_new: [B][Hkv][128] in kv_dtype.
 * For each b with t = seq_lens[b] < max_seq_len: writes K[b][g][t] and V[b][g][t]; folds
 * k~ = k R_g into page t / page_size (a new page when t % page_size == 0: min = max = k~);
 * writes the code of k; then sets seq_lens[b] = t + 1. A sequence already at max_seq_len is
 * left unchanged. The index maintenance an appended token needs is implied by the paper (every
 * key has a page summary and a code), which does not describe it. */
hhr_status hhr_append(const hhr_dims* dims, const hhr_cache* cache, const void* k_new,
                      const void* v_new, const float* R, const float* W, hhr_stream_t stream);

/* Bytes of workspace hhr_decode needs for these shapes and budgets (0 if they are invalid). */
size_t hhr_decode_workspace_bytes(const hhr_dims* dims, const hhr_params* params);

/* One decode step (both stages and the attention) for every (b, h), over the seq_lens[b]
 * tokens of the cache. ws: device workspace of at least hhr_decode_workspace_bytes bytes,
 * 256-byte aligned, caller-owned, needing no initialisation; it must not be shared by calls
 * that may run concurrently. out: [B][Hq][128] fp32. dbg: NULL or optional side outputs.
 * A sequence with no tokens gets a zero output. */
hhr_status hhr_decode(const hhr_dims* dims, const hhr_params* params, const hhr_cache* cache,
                      const void* q, const float* R, const float* W, void* ws, size_t ws_bytes,
                      float* out, const hhr_debug* dbg, hhr_stream_t stream);

/* hhr_append followed by hhr_decode in one call (the query attends over the new token too),
 * with the same results. The append is folded into the decode's kernels (the preparation
 * kernel stores the K/V rows, updates the page and stores the key's code; the last kernel
 * advances seq_lens), so a generation step costs no launch beyond the decode. Same arguments
 * and rules as the two calls; append_ticket is required. */
hhr_status hhr_append_decode(const hhr_dims* dims, const hhr_params* params,
                             const hhr_cache* cache, const void* k_new, const void* v_new,
                             const void* q, const float* R, const float* W, void* ws,
                             size_t ws_bytes, float* out, const hhr_debug* dbg,
                             hhr_stream_t stream);

/* hhr_decode for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same step and results, with the workspace
 * taken from scratch memory the library holds in a static device array of HHR_SCRATCH_BYTES per
 * GPU (each GPU the library runs on keeps its copy until the process ends). It allocates and
 * frees nothing. Arguments as for hhr_decode, without ws / ws_bytes.
 *   - Shapes and budgets whose hhr_decode_workspace_bytes exceeds HHR_SCRATCH_BYTES return
 *     HHR_ERR_CAPACITY before anything is enqueued (HHR_TRACE also logs the sizes).
 *   - Every call on a GPU uses that GPU's one scratch array: calls that may overlap on one GPU
 *     (concurrent streams, threads) race and must be serialised by the caller. The array keeps
 *     the last call's contents; the step needs none of them (its workspace needs no
 *     initialisation).
 *   - On the first call on a device (that device current) the library looks up the array's
 *     address there; a failure returns HHR_ERR_HIP. */
#define HHR_SCRATCH_BYTES (16u * 1024u * 1024u)
hhr_status hhr_decode_scratch(const hhr_dims* dims, const hhr_params* params,
                              const hhr_cache* cache, const void* q, const float* R,
                              const float* W, float* out, const hhr_debug* dbg,
                              hhr_stream_t stream);

/* Dense decode attention, the baseline of §4.3 / Fig. 7 (HHR against full attention): for
 * every (b, h), o = softmax(scale q K^T) V over ALL seq_lens[b] tokens of the cache, fp32
 * accumulation; no index is read (page_min, page_max, codes may be anything). Split-K over the
 * context with the G query heads of a KV head served by one read of its K/V rows, then a merge
 * of the partials. softmax_scale as in hhr_params. ws: at least hhr_dense_workspace_bytes
 * bytes, 256-byte aligned, caller-owned, needing no initialisation. dbg: NULL, or its
 * kernel_events used alone (4 events: start and stop of the attention and of the merge kernel).
 * A sequence with no tokens gets a zero output. */
size_t hhr_dense_workspace_bytes(const hhr_dims* dims);
hhr_status hhr_dense_decode(const hhr_dims* dims, const hhr_cache* cache, const void* q,
                            float softmax_scale, void* ws, size_t ws_bytes, float* out,
                            const hhr_debug* dbg, hhr_stream_t stream);

/* Measurement aid, no step of the method: the practical one-pass read rate of device memory,
 * against which the HBM-bound kernels above are compared (a single launch pays its ramp-up and
 * drain, so it cannot reach the HBM peak). Reads the `bytes` bytes at src once with the page-
 * bound kernel's load width and cache policy (16-byte non-temporal loads) and writes, for each
 * block of 32 KiB (the last one partial), the fp32 sum of the floats it read to partial[i],
 * i < hhr_read_probe_blocks(bytes). src: device, 16-byte aligned; bytes: a nonzero multiple of
 * 16 (else HHR_ERR_INVALID_ARG); partial: device, caller-owned. Nothing else is written. */
size_t hhr_read_probe_blocks(size_t bytes);
hhr_status hhr_read_probe(const void* src, size_t bytes, float* partial, hhr_stream_t stream);

/* Static text for a status code. */
const char* hhr_status_string(hhr_status status);

#ifdef __cplusplus
}
#endif

#endif /* HHR_H */
