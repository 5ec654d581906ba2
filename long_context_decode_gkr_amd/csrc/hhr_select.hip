// Selection of the tokens a decode step attends to, for every selection unit (a query head, or a
// KV head whose query heads share one selection).
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation" (arXiv 2610.01230):
//   §3.3.1 (after Eq. 3)  the pages whose bound passes the threshold survive; the threshold is
//                         read as "the n_keep largest bounds", ties to the lower page index;
//   §3.1 Eq. 2            Hamming distance of a key code to the query code by XOR + popcount;
//   §3.3.2                the closest keys among the surviving pages' keys are kept (ties to
//                         the lower position).
//
// Two forms, with identical results:
//   select_unit_kernel  grid (units, B), 1024 threads: one workgroup per unit does the whole
//                       selection (page cut, Hamming distances of the kept pages' keys cached
//                       in LDS, token threshold, ordered emission). The selection is a chain of
//                       dependent steps (bounds, cut, code loads, histogram, threshold,
//                       emission) whose latency, not its instruction count, sets its time, so
//                       one launch per unit is the fastest form whenever the candidates fit in
//                       LDS (at most kUnitSlots).
//   select_scan_kernel  grid (nsl slices, units, B), then select_emit_kernel over the same
//                       grid: for the fine-stage-only variant (every token a candidate) and
//                       other candidate sets beyond kUnitSlots, and whenever it is asked for.
//     select_scan_kernel: every workgroup of a unit finds the same exact page cut from the
//                       unit's bounds, takes the kept pages of rank [r0, r1) (the slice's even
//                       share), computes the Hamming distance of each of their keys, and writes
//                       the distances (one byte, two for 256-bit codes, per candidate slot,
//                       slots in ascending token order), the slice's kept page ids and its
//                       histogram of distances;
//     select_emit_kernel: every workgroup sums the unit's histograms, finds the token threshold
//                       D* (smallest with #(D <= D*) >= k_eff) and the counts of the slices
//                       before its own, and writes its slice's selected tokens at their final,
//                       ascending positions.
//   No workgroup waits for another inside a launch. With every page kept (the fine-stage-only
//   variant, or ceil(rho P) >= P) the cut is skipped.
#include <type_traits>

#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

constexpr int kScanThreads = 1024;   // select_scan_kernel workgroup
constexpr int kEmitThreads = 256;    // select_emit_kernel workgroup
constexpr int kEmitPer = 16;         // candidate slots per thread per emission round
constexpr int kRadixBits = 12;
constexpr int kRadixBins = 1 << kRadixBits;

// Order-preserving map of a bound to uint32 in which SMALLER means LARGER U (the kept pages are
// the smallest keys); -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t desc_key(float u) {
  const uint32_t x = __float_as_uint(u + 0.0f);   // -0 + 0 = +0
  const uint32_t asc = (x & 0x80000000u) ? ~x : (x | 0x80000000u);
  return ~asc;
}

// n_keep = min(P, max(1, ceil(rho P))), 0 for an empty sequence; rho P is one double multiply.
__device__ __forceinline__ int keep_count(int P, double rho) {
  return P == 0 ? 0 : min(P, max(1, int(ceil(rho * double(P)))));
}
// First kept-page rank of slice i of n: the n_keep kept pages are shared out evenly.
__device__ __forceinline__ int slice_begin(int i, int n_keep, int n) {
  return int((int64_t(i) * n_keep) / n);
}

// ---------------------------------------------------------------------------------------------
// Page cut: the kept flags of a thread's EPT pages [tid EPT, tid EPT + EPT) (the n_keep pages of
// largest bound, ties to the lower page). A radix select over rel = key - min(key), 12 bits at a
// time from the top set bit of the range. As soon as the threshold bin holds at most 64 keys,
// one wave ranks them by (key, page) and the kept set is the lexicographic cut; if the whole bin
// is taken, the cut is its upper edge; only more than 64 exactly equal keys at the threshold fall
// back to taking the equal keys in page order (one scan). Called by every thread of the
// workgroup (it holds barriers); `hist` must be zero and `ncand` 0 on entry, and hist is zero
// again on return. Its first barrier also publishes what the caller wrote to LDS before.
// ---------------------------------------------------------------------------------------------
template <int NWV>
struct CutLds {
  uint32_t hist[kRadixBins + kWave];   // radix bins, then one dummy per lane
  uint32_t mm[2][NWV];
  int pick[3];
  uint32_t ckey[kWave];   // keys of the threshold bin (when it holds <= 64)
  int cidx[kWave];
  int ncand;
};

template <int EPT, int NT>
__device__ __forceinline__ void page_cut(const uint32_t (&key)[EPT], const bool (&valid)[EPT],
                                         int n_keep, CutLds<NT / kWave>& cl,
                                         BlockScan<NT / kWave>& scan, bool (&tk)[EPT]) {
  constexpr int NWV = NT / kWave;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  // ---- key range (one barrier for both reductions)
  uint32_t kmin, kmax;
  {
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      lmin = min(lmin, key[e]);                 // an invalid key is the largest value
      lmax = max(lmax, valid[e] ? key[e] : 0u);
    }
    lmin = wave_min_u32(lmin);
    lmax = wave_max_u32(lmax);
    if (lane == 0) {
      cl.mm[0][w] = lmin;
      cl.mm[1][w] = lmax;
    }
    __syncthreads();
    kmin = wave_min_u32(cl.mm[0][lane % NWV]);
    kmax = wave_max_u32(cl.mm[1][lane % NWV]);
  }
  // ---- radix passes. The kept set is described by a cut (ck, ci): page i is kept iff
  // (key_i, i) <= (ck, ci); or, with more than 64 equal keys at the threshold, by the final
  // prefix and the number `need` of its elements to take in page order.
  int need = n_keep;        // still to take among elements matching `prefix`
  uint32_t prefix = 0;      // high bits of rel fixed so far
  int res_lo = 0;           // elements compare on rel >> res_lo
  bool cut = false;
  uint32_t ck = 0xFFFFFFFFu;
  int ci = 0x7FFFFFFF;
  int cur_hi = (kmax == kmin) ? -1 : 31 - __clz(int(kmax - kmin));
  bool first = true;
  while (cur_hi >= 0) {
    const int cur_lo = max(cur_hi - (kRadixBits - 1), 0);
    const int width = cur_hi - cur_lo + 1;
    const uint32_t dmask = (1u << width) - 1u;
    if (first) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t rel = key[e] - kmin;
        atomicAdd(&cl.hist[valid[e] ? (rel >> cur_lo) & dmask : kRadixBins + lane], 1u);
      }
    } else {
      // few keys match a longer prefix: waves without a match skip the atomic
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t rel = key[e] - kmin;
        if (valid[e] && uint32_t(uint64_t(rel) >> (cur_hi + 1)) == prefix)
          atomicAdd(&cl.hist[(rel >> cur_lo) & dmask], 1u);
      }
    }
    first = false;
    __syncthreads();
    // thread i owns bins [BPT i, BPT i + BPT): read them and clear them for the next pass
    constexpr int BPT = kRadixBins / NT;
    uint32_t hb[BPT];
    int loc = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      hb[j] = cl.hist[tid * BPT + j];
      cl.hist[tid * BPT + j] = 0;
      loc += int(hb[j]);
    }
    int tot;
    int run = scan.excl(loc, &tot);
    int fbin = -1, fbefore = 0, fcnt = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int cnt = int(hb[j]);
      const bool hit = cnt > 0 && run < need && need <= run + cnt;
      fbin = hit ? tid * BPT + j : fbin;
      fbefore = hit ? run : fbefore;
      fcnt = hit ? cnt : fcnt;
      run += cnt;
    }
    if (fbin >= 0) {   // exactly one thread
      cl.pick[0] = fbin;
      cl.pick[1] = fbefore;
      cl.pick[2] = fcnt;
    }
    __syncthreads();
    const int d = cl.pick[0], before = cl.pick[1], in_bin = cl.pick[2];
    prefix = (prefix << width) | uint32_t(d);
    need -= before;
    res_lo = cur_lo;
    cur_hi = cur_lo - 1;
    if (in_bin == need) {
      // the whole bin is taken: keep every key with rel >> res_lo <= prefix
      const uint64_t top = uint64_t(kmin) + ((uint64_t(prefix) + 1) << res_lo) - 1;
      ck = top > 0xFFFFFFFFull ? 0xFFFFFFFFu : uint32_t(top);
      ci = 0x7FFFFFFF;
      cut = true;
      break;
    }
    if (in_bin <= kWave) {
      // few keys share the threshold bin: wave 0 ranks them by (key, page) and the need-th
      // smallest becomes the cut
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        if (valid[e] && ((key[e] - kmin) >> res_lo) == prefix) {
          const int j = atomicAdd(&cl.ncand, 1);
          cl.ckey[j] = key[e];
          cl.cidx[j] = tid * EPT + e;
        }
      }
      __syncthreads();
      if (w == 0) {
        // (key, index) of every lane compared with the in_bin entries through register reads
        // (in_bin is uniform and usually a handful)
        const uint32_t kl = lane < in_bin ? cl.ckey[lane] : 0xFFFFFFFFu;
        const uint32_t il = lane < in_bin ? uint32_t(cl.cidx[lane]) : 0x7FFFFFFFu;
        const uint64_t vl = (uint64_t(kl) << 32) | il;
        int rank = 0;
        for (int j = 0; j < in_bin; ++j) {
          const uint64_t vj = (uint64_t(__builtin_amdgcn_readlane(kl, j)) << 32) |
                              uint32_t(__builtin_amdgcn_readlane(il, j));
          rank += vj < vl ? 1 : 0;
        }
        if (lane < in_bin && rank == need - 1) {
          cl.pick[0] = int(kl);
          cl.pick[1] = il;
        }
      }
      __syncthreads();
      ck = uint32_t(cl.pick[0]);
      ci = cl.pick[1];
      cut = true;
      break;
    }
  }
  if (cut) {
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      tk[e] = valid[e] && (key[e] < ck || (key[e] == ck && tid * EPT + e <= ci));
  } else {
    // rel >> res_lo below prefix: kept; equal: kept in page order up to `need`
    bool eq[EPT];
    int neq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t v = (key[e] - kmin) >> res_lo;
      tk[e] = valid[e] && v < prefix;
      eq[e] = valid[e] && v == prefix;
      neq += eq[e] ? 1 : 0;
    }
    int tot;
    int eq_seen = scan.excl(neq, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      tk[e] = tk[e] || (eq[e] && eq_seen < need);
      eq_seen += eq[e] ? 1 : 0;
    }
  }
}

// A unit's bound row, from whole float4 loads at clamped addresses (rows are Pmax long, Pmax a
// multiple of 4), in two steps: issue_bounds issues every load, and pin_bounds, called after
// the caller has issued its other early loads, pins each value (materialize) so that the
// compiler cannot sink a load into the code that needs the sequence length. (Pinning a value
// right after its load would wait for it before the next load is issued: one memory round trip
// per load.)
template <int EPT>
__device__ __forceinline__ void issue_bounds(const float* Urow, int Pmax, float4 (&x)[EPT / 4]) {
  const float4* U4 = reinterpret_cast<const float4*>(Urow);
  const int last4 = Pmax / 4 - 1;
#pragma unroll
  for (int e = 0; e < EPT; e += 4) x[e / 4] = U4[min(int(threadIdx.x) * (EPT / 4) + e / 4, last4)];
}
template <int EPT>
__device__ __forceinline__ void pin_bounds(const float4 (&x)[EPT / 4], float (&uv)[EPT]) {
#pragma unroll
  for (int e = 0; e < EPT; e += 4) {
    uv[e] = materialize(x[e / 4].x); uv[e + 1] = materialize(x[e / 4].y);
    uv[e + 2] = materialize(x[e / 4].z); uv[e + 3] = materialize(x[e / 4].w);
  }
}

// Distance of a code to the query code qw (in registers) or, with a shared selection, the
// smallest over the ncodes codes of the group (the others read from LDS as broadcasts).
template <int NW, int SHARED>
__device__ __forceinline__ uint32_t code_dist(const uint4 (&x)[NW / 4], const uint32_t (&qw)[NW],
                                              const uint32_t (*sqw)[NW], int ncodes) {
  uint32_t dd = 0;
#pragma unroll
  for (int v = 0; v < NW / 4; ++v)
    dd += __popc(x[v].x ^ qw[4 * v]) + __popc(x[v].y ^ qw[4 * v + 1]) +
          __popc(x[v].z ^ qw[4 * v + 2]) + __popc(x[v].w ^ qw[4 * v + 3]);
  if constexpr (SHARED) {
    for (int i = 1; i < ncodes; ++i) {   // uniform
      uint32_t di = 0;
#pragma unroll
      for (int v = 0; v < NW / 4; ++v)
        di += __popc(x[v].x ^ sqw[i][4 * v]) + __popc(x[v].y ^ sqw[i][4 * v + 1]) +
              __popc(x[v].z ^ sqw[i][4 * v + 2]) + __popc(x[v].w ^ sqw[i][4 * v + 3]);
      dd = min(dd, di);
    }
  }
  return dd;
}

// ---------------------------------------------------------------------------------------------
// Whole selection of one unit in one workgroup of NT threads (256, 512 or 1024; pages per
// thread EPT):
//   the bounds and the query code(s) are loaded before the sequence length is known;
//   page cut; kept pages in ascending order in LDS;
//   Hamming distance of every candidate slot (ascending token order), cached in LDS as one byte
//   (two for 256-bit codes), and their histogram over D in [0, NB];
//   the smallest D* with #(D <= D*) >= k_eff (wave 0);
//   one scan of per-thread (#lt, #eq) counts per round places every slot with D < D* and the
//   first k_eff - #(D < D*) slots with D == D*; the list is assembled in LDS (the histograms are
//   done with) and copied out with 16-byte stores when it fits, else written directly.
// Per-element steps are branch-free: a lane with nothing to record writes a dummy LDS entry or a
// trash slot of its own past the live data.
// ---------------------------------------------------------------------------------------------
constexpr int kEmitSPT = 8;         // cached distances per thread per emission round
static_assert(16 % kEmitSPT == 0, "an emission round must not cross a page (sizes 16, 32)");

// FINE: the instantiation for a.fine = 1 (the Hamming ranking runs) or 0 (the coarse stage
// alone: every live candidate is taken, and the histogram counts them once per wave)
template <int NB, int EPT, int SHARED, int NT, int FINE>
__global__ void __launch_bounds__(NT)
select_unit_kernel(Shape s, CacheView c, SelectArgs a, DebugView dbg) {
  constexpr int NWV = NT / kWave;
  constexpr int NW = NB / 32;
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  constexpr uint32_t kNone = NB == 128 ? 0xFFu : 0xFFFFu;   // distance of a slot past the end
  const int u = blockIdx.x, b = blockIdx.y;
  const int g = SHARED ? u : u / s.G;
  const int bu = b * (SHARED ? s.Hkv : s.Hq) + u;
  const int ncodes = SHARED ? s.G : 1;
  const int tid = threadIdx.x, lane = lane_id();

  __shared__ int32_t s_pages[kMaxPages + kWave];
  __shared__ __align__(16) DT s_dist[kUnitSlots + kWave];
  __shared__ __align__(16) CutLds<NWV> cl;
  __shared__ uint32_t s_qw[SHARED ? 8 : 1][NW];
  __shared__ int s_wt[2][NWV];
  __shared__ int s_pick[3];
  BlockScan<NWV> scan{s_wt, 0};

  // bounds, query code(s) and sequence length loaded together (the first two do not depend on
  // the length); every lane loads a code word (clamped), so that no branch holds a load back
  float4 ux[EPT / 4];
  issue_bounds<EPT>(a.U + size_t(bu) * s.Pmax, s.Pmax, ux);
  const uint32_t qraw =
      a.qcode[(size_t(b) * s.Hq + (SHARED ? g * s.G : u)) * NW + min(tid, ncodes * NW - 1)];
  const int t = c.seq_lens[b];                   // position of the appended token, if any
  float uv[EPT];
  pin_bounds<EPT>(ux, uv);
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  int32_t* out_idx = a.idx + size_t(bu) * a.istride;
  if (L == 0) {
    if (tid == 0) {
      a.cnt[bu] = 0;
      if (dbg.page_count) dbg.page_count[bu] = 0;
      if (dbg.token_count) dbg.token_count[bu] = 0;
    }
    return;
  }
  const int n_keep = keep_count(P, a.rho);
  if (tid < ncodes * NW) s_qw[tid / NW][tid % NW] = qraw;
  if (tid == 0) cl.ncand = 0;
  for (int i = tid; i < kRadixBins; i += NT) cl.hist[i] = 0;

  // ---- coarse stage: kept pages, ascending, into s_pages
  {
    uint32_t key[EPT];
    bool valid[EPT], tk[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      valid[e] = tid * EPT + e < P;
      key[e] = valid[e] ? desc_key(uv[e]) : 0xFFFFFFFFu;
    }
    if (n_keep < P) {   // uniform
      page_cut<EPT, NT>(key, valid, n_keep, cl, scan, tk);
    } else {
      __syncthreads();   // publishes s_qw and the cleared bins
#pragma unroll
      for (int e = 0; e < EPT; ++e) tk[e] = valid[e];
    }
    int n = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) n += tk[e] ? 1 : 0;
    int tot;
    int pos = scan.excl(n, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      s_pages[tk[e] ? pos : kMaxPages + lane] = tid * EPT + e;
      pos += tk[e] ? 1 : 0;
    }
  }
  __syncthreads();
  if (dbg.page_ids)
    for (int i = tid; i < n_keep; i += NT) dbg.page_ids[size_t(bu) * s.Pmax + i] = s_pages[i];
  if (tid == 0 && dbg.page_count) dbg.page_count[bu] = n_keep;

  // ---- fine stage: Hamming distance of every candidate slot (§3.1 Eq. 2)
  uint32_t qw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) qw[i] = s_qw[0][i];
  const int lgS = (s.S == 16) ? 4 : 5;
  const int nslots = n_keep << lgS;              // at most kUnitSlots (the host's rule)
  const uint32_t* cbase = c.codes + (size_t(b) * s.Hkv + g) * s.Lmax * NW;
  auto slot_token = [&](int slot) { return (s_pages[slot >> lgS] << lgS) + (slot & (s.S - 1)); };
  uint32_t* whist = cl.hist;   // bins 0..NB (cleared by the cut's last pass or above)
  // batches of BAT slots per thread: all code loads of a batch are issued before any is used.
  // The first batch is a copy of its own (outside the loop), so that its loads are not held
  // back by waits that a loop's reuse of its load registers would require
  constexpr int BAT = 8 / (NW / 4);
  auto batch = [&](int base) {
    int tt[BAT];
    uint4 cw[BAT][NW / 4];
#pragma unroll
    for (int k = 0; k < BAT; ++k) {
      const int slot = base + k * NT + tid;
      const int tk = materialize(slot_token(min(slot, nslots - 1)));   // every lane
      tt[k] = (slot < nslots) ? tk : L;
    }
    if (a.fine) {   // uniform
#pragma unroll
      for (int k = 0; k < BAT; ++k) {
        const uint4* cp = reinterpret_cast<const uint4*>(cbase + size_t(min(tt[k], L - 1)) * NW);
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) cw[k][v] = cp[v];
      }
    }
#pragma unroll
    for (int k = 0; k < BAT; ++k) {
      const int slot = base + k * NT + tid;
      // (without the fine stage every live candidate has distance 0: all are taken)
      const uint32_t dd = a.fine ? code_dist<NW, SHARED>(cw[k], qw, s_qw, ncodes) : 0u;
      const bool live = tt[k] < L;               // implies slot < nslots
      if constexpr (FINE) {
        atomicAdd(live ? &whist[dd] : &whist[kRadixBins + lane], 1u);
      } else {
        // one count per wave: per-lane atomics on the one bin would queue behind each other
        const uint32_t nl = uint32_t(__popcll(__ballot(live)));
        if (lane == 0) atomicAdd(&whist[0], nl);
      }
      s_dist[slot < nslots ? slot : kUnitSlots + lane] = DT(live ? dd : kNone);
    }
  };
  batch(0);
  for (int base = BAT * NT; base < nslots; base += BAT * NT) batch(base);
  __syncthreads();
  if (dbg.dist) {
    for (int i = tid; i < nslots; i += NT) {
      const uint32_t dd = s_dist[i];
      dbg.dist[size_t(bu) * s.Lmax + i] = uint16_t(dd == kNone ? 0xFFFFu : dd);
    }
  }

  // ---- token threshold: smallest D* with #(D <= D*) >= k_eff, found by wave 0 alone
  if (wave_id() == 0) {
    constexpr int BPL = (NB + 1 + kWave - 1) / kWave;   // distance bins per lane
    int cnt[BPL];
    int tot_d = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      const int v = int(whist[min(bin, NB)]);
      cnt[j] = bin <= NB ? v : 0;
      tot_d += cnt[j];
    }
    const int incl = wave_incl_sum(tot_d);
    const int C = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int k_eff = min(a.kcap, C);
    int run = incl - tot_d;
    int fbin = -1, fbefore = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const bool hit = cnt[j] > 0 && run < k_eff && k_eff <= run + cnt[j];
      fbin = hit ? lane * BPL + j : fbin;
      fbefore = hit ? run : fbefore;
      run += cnt[j];
    }
    if (fbin >= 0) {   // exactly one lane
      s_pick[0] = fbin;
      s_pick[1] = fbefore;
      s_pick[2] = k_eff;
    }
  }
  __syncthreads();
  const uint32_t dstar = uint32_t(s_pick[0]);
  const int k_eff = s_pick[2];
  const int need_eq = k_eff - s_pick[1];

  // ---- emission in ascending position (slots are in ascending t)
  int32_t* trash = out_idx + a.kcap + lane;
  int32_t* dbg_idx = dbg.token_idx ? dbg.token_idx + size_t(bu) * a.kcap : nullptr;
  int32_t* stage = reinterpret_cast<int32_t*>(cl.hist);
  constexpr int HB = kRadixBins;
  const bool staged = k_eff <= HB;
  int run_lt = 0, run_eq = 0;
  constexpr int kPer = 4 / int(sizeof(DT));            // distances per 32-bit word
  constexpr int kWords = kEmitSPT / kPer;
  const int nrounds = (nslots + NT * kEmitSPT - 1) / (NT * kEmitSPT);
  for (int ch = 0; ch < nrounds; ++ch) {
    const int s0 = (ch * NT + tid) * kEmitSPT;
    const bool any = s0 < nslots;
    const int sc = any ? s0 : 0;                 // read position (in bounds)
    uint32_t wv[kWords];
    if constexpr (kWords == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(&s_dist[sc]);
      wv[0] = x.x; wv[1] = x.y;
    } else {
#pragma unroll
      for (int i = 0; i < kWords; i += 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(&s_dist[sc + i * kPer]);
        wv[i] = x.x; wv[i + 1] = x.y; wv[i + 2] = x.z; wv[i + 3] = x.w;
      }
    }
    uint32_t dv[kEmitSPT];
#pragma unroll
    for (int k = 0; k < kEmitSPT; ++k) {
      const uint32_t d = (wv[k / kPer] >> (8 * sizeof(DT) * (k % kPer))) & kNone;
      dv[k] = (any && s0 + k < nslots) ? d : kNone;
    }
    int nlt = 0, neq = 0;
#pragma unroll
    for (int k = 0; k < kEmitSPT; ++k) {
      nlt += dv[k] < dstar ? 1 : 0;
      neq += dv[k] == dstar ? 1 : 0;
    }
    const int t0 = slot_token(sc);               // the round's slots lie in one page
    int tot;
    const int ex = scan.excl((nlt << 16) | neq, &tot);
    int eq_seen = run_eq + (ex & 0xFFFF);
    int pos = run_lt + (ex >> 16) + min(eq_seen, need_eq);
#pragma unroll
    for (int k = 0; k < kEmitSPT; ++k) {
      const bool is_eq = dv[k] == dstar;
      const bool take = dv[k] < dstar || (is_eq && eq_seen < need_eq);
      eq_seen += is_eq ? 1 : 0;
      if (staged) stage[take ? pos : HB + lane] = t0 + k;
      else *(take ? out_idx + pos : trash) = t0 + k;
      if (dbg_idx && !staged && take) dbg_idx[pos] = t0 + k;
      pos += take ? 1 : 0;
    }
    run_lt += tot >> 16;
    run_eq += tot & 0xFFFF;
  }
  if (staged) {
    __syncthreads();
    const int n4 = k_eff >> 2;   // rows of idx start 16-byte aligned
    for (int i = tid; i < n4; i += NT)
      reinterpret_cast<int4*>(out_idx)[i] = reinterpret_cast<const int4*>(stage)[i];
    for (int i = 4 * n4 + tid; i < k_eff; i += NT) out_idx[i] = stage[i];
    if (dbg_idx)
      for (int i = tid; i < k_eff; i += NT) dbg_idx[i] = stage[i];
  }
  if (tid == 0) {
    a.cnt[bu] = k_eff;
    if (dbg.token_count) dbg.token_count[bu] = k_eff;
  }
}

// ---------------------------------------------------------------------------------------------
// Sliced form, first kernel: page cut (repeated by every slice of a unit), Hamming distances of
// the slice's candidate slots and its histogram. 1024 threads; 4 consecutive candidate slots
// (one page) per thread and unit of work, the code loads of up to 16 slots issued before any
// use.
// ---------------------------------------------------------------------------------------------
template <int NB, int EPT, int SHARED, int FINE>
__global__ void __launch_bounds__(kScanThreads)
select_scan_kernel(Shape s, CacheView c, SelectArgs a, DebugView dbg) {
  constexpr int NT = kScanThreads;
  constexpr int NWV = NT / kWave;
  constexpr int NW = NB / 32;
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  constexpr uint32_t kNone = NB == 128 ? 0xFFu : 0xFFFFu;
  const int sl = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int Hs = SHARED ? s.Hkv : s.Hq;
  const int g = SHARED ? u : u / s.G;
  const int bu = b * Hs + u;
  const int ncodes = SHARED ? s.G : 1;
  const int tid = threadIdx.x, lane = lane_id();

  __shared__ __align__(16) CutLds<NWV> cl;          // its bins then hold distances 0..NB
  __shared__ int32_t s_pages[kSlicePages + kWave];  // the slice's kept pages, then dummies
  __shared__ uint32_t s_qw[SHARED ? 8 : 1][NW];
  __shared__ int s_wt[2][NWV];
  BlockScan<NWV> scan{s_wt, 0};

  const bool cutting = a.U != nullptr;           // else every page is kept (no bounds)
  float4 ux[EPT / 4];
  if (cutting) issue_bounds<EPT>(a.U + size_t(bu) * s.Pmax, s.Pmax, ux);
  const uint32_t qraw =
      a.qcode[(size_t(b) * s.Hq + (SHARED ? g * s.G : u)) * NW + min(tid, ncodes * NW - 1)];
  const int t = c.seq_lens[b];
  float uv[EPT];
  if (cutting) pin_bounds<EPT>(ux, uv);
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  const int n_keep = keep_count(P, a.rho);
  const int r0 = slice_begin(sl, n_keep, a.nsl), r1 = slice_begin(sl + 1, n_keep, a.nsl);

  int32_t* hg = a.hist + (size_t(bu) * a.nsl + sl) * (NB + 1);
  if (sl == 0 && tid == 0 && dbg.page_count) dbg.page_count[bu] = n_keep;
  if (r1 == r0) {   // nothing in this slice (also an empty sequence): a zero histogram
    for (int i = tid; i <= NB; i += NT) hg[i] = 0;
    return;
  }
  if (tid < ncodes * NW) s_qw[tid / NW][tid % NW] = qraw;
  if (tid == 0) cl.ncand = 0;
  for (int i = tid; i < kRadixBins; i += NT) cl.hist[i] = 0;
  int32_t* prow = a.pages + size_t(bu) * a.kpages;

  if (cutting && n_keep < P) {   // uniform
    uint32_t key[EPT];
    bool valid[EPT], tk[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      valid[e] = tid * EPT + e < P;
      key[e] = valid[e] ? desc_key(uv[e]) : 0xFFFFFFFFu;
    }
    page_cut<EPT, NT>(key, valid, n_keep, cl, scan, tk);
    int n = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) n += tk[e] ? 1 : 0;
    int tot;
    int rank = scan.excl(n, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool mine = tk[e] && rank >= r0 && rank < r1;
      s_pages[mine ? rank - r0 : kSlicePages + lane] = tid * EPT + e;
      rank += tk[e] ? 1 : 0;
    }
  } else {
    // every page is kept: the slice is pages [r0, r1)
    for (int j = tid; j < r1 - r0; j += NT) s_pages[j] = r0 + j;
  }
  __syncthreads();

  // ---- fine stage: Hamming distances of the slice's candidate slots (§3.1 Eq. 2)
  uint32_t qw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) qw[i] = s_qw[0][i];
  const int lgS = (s.S == 16) ? 4 : 5;
  const int nunits = ((r1 - r0) << lgS) / 4;     // groups of 4 slots (one page each)
  const int slot0 = r0 << lgS;
  const uint32_t* cbase = c.codes + (size_t(b) * s.Hkv + g) * s.Lmax * NW;
  DT* drow = static_cast<DT*>(a.dist) + size_t(bu) * a.dstride + slot0;
  uint16_t* dbg_dist = dbg.dist ? dbg.dist + size_t(bu) * s.Lmax + slot0 : nullptr;
  constexpr int UB = NB == 128 ? 4 : 2;          // units per thread per batch (16 code loads)
  for (int ub = 0; ub < nunits; ub += UB * NT) {
    // batch of up to UB units per thread; units past the end are not loaded (uniform per k
    // within a wave when the whole wave is past it)
    int tok0[UB];
    uint4 cw[UB][4][NW / 4];
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int slot = min(ub + k * NT + tid, nunits - 1) * 4;
      tok0[k] = (s_pages[slot >> lgS] << lgS) + (slot & (s.S - 1));
    }
    if (a.fine) {   // uniform
#pragma unroll
      for (int k = 0; k < UB; ++k) {
        if (ub + k * NT >= nunits) break;        // uniform: no thread of the batch has unit k
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4* cp =
              reinterpret_cast<const uint4*>(cbase + size_t(min(tok0[k] + i, L - 1)) * NW);
#pragma unroll
          for (int v = 0; v < NW / 4; ++v) cw[k][i][v] = cp[v];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      if (ub + k * NT >= nunits) break;          // uniform
      const int unit = ub + k * NT + tid;
      const bool in = unit < nunits;
      uint32_t dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (without the fine stage every live candidate has distance 0: all are taken)
        const uint32_t d = a.fine ? code_dist<NW, SHARED>(cw[k][i], qw, s_qw, ncodes) : 0u;
        const bool live = in && tok0[k] + i < L;
        if constexpr (FINE) {
          atomicAdd(live ? &cl.hist[d] : &cl.hist[kRadixBins + lane], 1u);
        } else {   // one count per wave (per-lane atomics on the one bin would queue)
          const uint32_t nl = uint32_t(__popcll(__ballot(live)));
          if (lane == 0) atomicAdd(&cl.hist[0], nl);
        }
        dd[i] = live ? d : kNone;
      }
      if (in) {
        if constexpr (NB == 128) {
          *reinterpret_cast<uint32_t*>(drow + unit * 4) =
              dd[0] | (dd[1] << 8) | (dd[2] << 16) | (dd[3] << 24);
        } else {
          *reinterpret_cast<uint2*>(drow + unit * 4) =
              make_uint2(dd[0] | (dd[1] << 16), dd[2] | (dd[3] << 16));
        }
        if (dbg_dist) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dbg_dist[unit * 4 + i] = uint16_t(dd[i] == kNone ? 0xFFFFu : dd[i]);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i <= NB; i += NT) hg[i] = int32_t(cl.hist[i]);
  // the slice's kept pages, for the emission kernel and the debug output
  int32_t* dbg_pages = dbg.page_ids ? dbg.page_ids + size_t(bu) * s.Pmax : nullptr;
  for (int j = tid; j < r1 - r0; j += NT) {
    prow[r0 + j] = s_pages[j];
    if (dbg_pages) dbg_pages[r0 + j] = s_pages[j];
  }
}

// ---------------------------------------------------------------------------------------------
// Token threshold and ordered emission. 256 threads; in each round thread i owns the 16 slots
// [16 i, 16 i + 16) of the round's 4096 (one page, or half of one: S is 16 or 32).
// ---------------------------------------------------------------------------------------------
template <int NB>
__global__ void __launch_bounds__(kEmitThreads)
select_emit_kernel(Shape s, CacheView c, SelectArgs a, DebugView dbg) {
  constexpr int NT = kEmitThreads;
  constexpr int NWV = NT / kWave;
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  constexpr int kWords = kEmitPer * int(sizeof(DT)) / 4;   // 32-bit words of 16 distances
  constexpr int kPer = 4 / int(sizeof(DT));                // distances per word
  const int sl = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int Hs = a.shared ? s.Hkv : s.Hq;
  const int bu = b * Hs + u;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int t = c.seq_lens[b];
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  const int n_keep = keep_count(P, a.rho);
  const int r0 = slice_begin(sl, n_keep, a.nsl), r1 = slice_begin(sl + 1, n_keep, a.nsl);
  const int lgS = (s.S == 16) ? 4 : 5;
  const int nslots = (r1 - r0) << lgS;           // a multiple of 16

  __shared__ int s_tot[NB + 1], s_pre[NB + 1];
  __shared__ int s_pick[4];
  __shared__ int s_wt[2][NWV];
  BlockScan<NWV> scan{s_wt, 0};

  if (L == 0) {
    if (sl == 0 && tid == 0) {
      a.cnt[bu] = 0;
      if (dbg.token_count) dbg.token_count[bu] = 0;
    }
    return;
  }

  // The first round's distances and page id: their addresses do not depend on the histograms,
  // so these loads are issued before them.
  const DT* drow = static_cast<const DT*>(a.dist) + size_t(bu) * a.dstride + (r0 << lgS);
  const int32_t* prow = a.pages + size_t(bu) * a.kpages + r0;
  auto load_round = [&](int base, uint32_t (&wv)[kWords], int& page) {
    const int s0 = min(base + kEmitPer * tid, max(nslots - kEmitPer, 0));
    const uint4* dp = reinterpret_cast<const uint4*>(drow + s0);
#pragma unroll
    for (int i = 0; i < kWords; i += 4) {
      const uint4 x = dp[i / 4];
      wv[i] = x.x; wv[i + 1] = x.y; wv[i + 2] = x.z; wv[i + 3] = x.w;
    }
    page = prow[s0 >> lgS];
  };
  uint32_t wv[kWords];
  int page = 0;
  if (nslots > 0) load_round(0, wv, page);

  // totals over the unit's slices and over the slices before this one, bin by bin
  for (int bin = tid; bin <= NB; bin += NT) {
    const int32_t* hb = a.hist + size_t(bu) * a.nsl * (NB + 1) + bin;
    int tot = 0, pre = 0;
    for (int s0 = 0; s0 < a.nsl; s0 += 16) {
      int v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = hb[size_t(min(s0 + r, a.nsl - 1)) * (NB + 1)];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int x = s0 + r < a.nsl ? v[r] : 0;
        tot += x;
        pre += s0 + r < sl ? x : 0;
      }
    }
    s_tot[bin] = tot;
    s_pre[bin] = pre;
  }
  __syncthreads();

  // threshold D* (wave 0): the smallest distance with #(D <= D*) >= k_eff; then how many of the
  // slices before this one select
  if (w == 0) {
    constexpr int BPL = (NB + 1 + kWave - 1) / kWave;   // bins per lane
    int cnt[BPL];
    int tot_d = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      cnt[j] = bin <= NB ? s_tot[min(bin, NB)] : 0;
      tot_d += cnt[j];
    }
    const int incl = wave_incl_sum(tot_d);
    const int C = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int k_eff = min(a.kcap, C);
    int run = incl - tot_d, fbin = -1, fbefore = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const bool hit = cnt[j] > 0 && run < k_eff && k_eff <= run + cnt[j];
      fbin = hit ? lane * BPL + j : fbin;
      fbefore = hit ? run : fbefore;
      run += cnt[j];
    }
    const uint64_t hm = __ballot(fbin >= 0);   // exactly one lane, none when k_eff = 0
    const int src = hm ? int(__builtin_ctzll(hm)) : 0;
    const int dstar = hm ? __builtin_amdgcn_readlane(fbin, src) : 0;
    const int before = hm ? __builtin_amdgcn_readlane(fbefore, src) : 0;
    int lt = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      lt += bin < dstar ? s_pre[min(bin, NB)] : 0;
    }
    lt = __builtin_amdgcn_readlane(wave_incl_sum(lt), kWave - 1);
    if (lane == 0) {
      s_pick[0] = dstar;
      s_pick[1] = k_eff;
      s_pick[2] = k_eff - before;   // how many of the D* ties are taken
      s_pick[3] = lt;
    }
  }
  __syncthreads();
  const uint32_t dstar = uint32_t(s_pick[0]);
  const int k_eff = s_pick[1], need_eq = s_pick[2];
  int run_lt = s_pick[3];
  int run_eq = s_pre[min(int(dstar), NB)];
  if (sl == 0 && tid == 0) {
    a.cnt[bu] = k_eff;
    if (dbg.token_count) dbg.token_count[bu] = k_eff;
  }
  if (k_eff == 0 || nslots == 0) return;

  int32_t* out = a.idx + size_t(bu) * a.istride;
  int32_t* trash = out + a.kcap + lane;
  int32_t* dbg_idx = dbg.token_idx ? dbg.token_idx + size_t(bu) * a.kcap : nullptr;
  for (int base = 0; base < nslots; base += NT * kEmitPer) {
    if (base > 0) load_round(base, wv, page);
    const int s0 = base + kEmitPer * tid;
    const bool any = s0 < nslots;
    uint32_t dv[kEmitPer];
#pragma unroll
    for (int e = 0; e < kEmitPer; ++e) {
      const uint32_t d = (wv[e / kPer] >> (8 * sizeof(DT) * (e % kPer))) & (NB == 128 ? 0xFFu : 0xFFFFu);
      dv[e] = any ? d : 0xFFFFFFFFu;   // a slot past the end holds kNone > NB
    }
    int nlt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < kEmitPer; ++e) {
      nlt += dv[e] < dstar ? 1 : 0;
      neq += dv[e] == dstar ? 1 : 0;
    }
    int tot;
    const int ex = scan.excl((nlt << 16) | neq, &tot);
    int eq_seen = run_eq + (ex & 0xFFFF);
    int pos = run_lt + (ex >> 16) + min(eq_seen, need_eq);
    const int tok0 = (page << lgS) + (s0 & (s.S - 1));
#pragma unroll
    for (int e = 0; e < kEmitPer; ++e) {
      const bool is_eq = dv[e] == dstar;
      const bool take = dv[e] < dstar || (is_eq && eq_seen < need_eq);
      eq_seen += is_eq ? 1 : 0;
      *(take ? out + pos : trash) = tok0 + e;
      if (dbg_idx && take) dbg_idx[pos] = tok0 + e;
      pos += take ? 1 : 0;
    }
    run_lt += tot >> 16;
    run_eq += tot & 0xFFFF;
  }
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
int select_slices(int kpages, int units, bool all_kept) {
  // enough workgroups to spread a batch-1 step over the GPU, but no more than are resident at
  // once (two 1024-thread workgroups per CU: a second round of workgroups repeats the whole
  // latency chain; 1024 workgroups measured 18.2 us for the fine stage alone at 128K); fewer per
  // unit when a page cut is computed (every workgroup repeats it); at most kSlicePages pages
  // per slice
  const int target = all_kept ? 512 : 256;
  const int want = (target + units - 1) / units;
  const int lo = (kpages + kSlicePages - 1) / kSlicePages;
  const int hi = max(lo, (kpages + kMinSlicePages - 1) / kMinSlicePages);
  return max(1, min(max(want, lo), hi));
}

// Both events of an unlaunched kernel's slot, back to back (its duration reads as ~0).
static hipError_t record_empty(KernelTimer tm, hipStream_t st) {
  if (!tm.start) return hipSuccess;
  hipError_t e = hipEventRecord(tm.start, st);
  return e != hipSuccess ? e : hipEventRecord(tm.stop, st);
}

template <int NB, int EPT, int NT>
static hipError_t launch_unit(const Shape& s, const CacheView& c, const SelectArgs& a,
                              const DebugView& dbg, hipStream_t st) {
  const dim3 grid(a.shared ? s.Hkv : s.Hq, s.B);
  const KernelTimer tm = kernel_timer(dbg, 2);
  const char* nm = "select_unit_kernel";
  const hipError_t e =
      a.fine ? (a.shared ? launch_kernel(nm, select_unit_kernel<NB, EPT, 1, NT, 1>, grid, dim3(NT),
                                         st, tm, s, c, a, dbg)
                         : launch_kernel(nm, select_unit_kernel<NB, EPT, 0, NT, 1>, grid, dim3(NT),
                                         st, tm, s, c, a, dbg))
             : (a.shared ? launch_kernel(nm, select_unit_kernel<NB, EPT, 1, NT, 0>, grid, dim3(NT),
                                         st, tm, s, c, a, dbg)
                         : launch_kernel(nm, select_unit_kernel<NB, EPT, 0, NT, 0>, grid, dim3(NT),
                                         st, tm, s, c, a, dbg));
  return e != hipSuccess ? e : record_empty(kernel_timer(dbg, 3), st);
}

template <int NB, int EPT>
static hipError_t launch_sliced(const Shape& s, const CacheView& c, const SelectArgs& a,
                                const DebugView& dbg, hipStream_t st) {
  const int units = a.shared ? s.Hkv : s.Hq;
  const dim3 grid(a.nsl, units, s.B);
  const KernelTimer tm = kernel_timer(dbg, 2);
  const dim3 blk(kScanThreads);
  const char* nm = "select_scan_kernel";
  const hipError_t e =
      a.fine ? (a.shared ? launch_kernel(nm, select_scan_kernel<NB, EPT, 1, 1>, grid, blk, st, tm,
                                         s, c, a, dbg)
                         : launch_kernel(nm, select_scan_kernel<NB, EPT, 0, 1>, grid, blk, st, tm,
                                         s, c, a, dbg))
             : (a.shared ? launch_kernel(nm, select_scan_kernel<NB, EPT, 1, 0>, grid, blk, st, tm,
                                         s, c, a, dbg)
                         : launch_kernel(nm, select_scan_kernel<NB, EPT, 0, 0>, grid, blk, st, tm,
                                         s, c, a, dbg));
  if (e != hipSuccess) return e;
  return launch_kernel("select_emit_kernel",
                       select_emit_kernel<NB>, grid, dim3(kEmitThreads), st, kernel_timer(dbg, 3),
                       s, c, a, dbg);
}

template <int NB>
static hipError_t launch_select_nb(const Shape& s, const CacheView& c, const SelectArgs& a,
                                   const DebugView& dbg, int unit_threads, hipStream_t st) {
  static_assert(kMaxPages <= 16 * kScanThreads, "16 pages per thread cover the page capacity");
  if (unit_threads == 256 && s.Pmax <= 16 * 256) {
    if (s.Pmax <= 4 * 256) return launch_unit<NB, 4, 256>(s, c, a, dbg, st);
    if (s.Pmax <= 8 * 256) return launch_unit<NB, 8, 256>(s, c, a, dbg, st);
    return launch_unit<NB, 16, 256>(s, c, a, dbg, st);
  }
  if (unit_threads == 512 && s.Pmax <= 16 * 512) {
    if (s.Pmax <= 4 * 512) return launch_unit<NB, 4, 512>(s, c, a, dbg, st);
    if (s.Pmax <= 8 * 512) return launch_unit<NB, 8, 512>(s, c, a, dbg, st);
    return launch_unit<NB, 16, 512>(s, c, a, dbg, st);
  }
  const int ept = (s.Pmax + kScanThreads - 1) / kScanThreads;
  if (unit_threads > 0) {
    if (ept <= 4) return launch_unit<NB, 4, kScanThreads>(s, c, a, dbg, st);
    if (ept <= 8) return launch_unit<NB, 8, kScanThreads>(s, c, a, dbg, st);
    return launch_unit<NB, 16, kScanThreads>(s, c, a, dbg, st);
  }
  if (ept <= 4) return launch_sliced<NB, 4>(s, c, a, dbg, st);
  if (ept <= 8) return launch_sliced<NB, 8>(s, c, a, dbg, st);
  return launch_sliced<NB, 16>(s, c, a, dbg, st);
}

hipError_t launch_select(const Shape& s, const CacheView& c, const SelectArgs& a,
                         const DebugView& dbg, int unit_threads, hipStream_t st) {
  if (s.NB == 128) return launch_select_nb<128>(s, c, a, dbg, unit_threads, st);
  return launch_select_nb<256>(s, c, a, dbg, unit_threads, st);
}

}  // namespace hhr
