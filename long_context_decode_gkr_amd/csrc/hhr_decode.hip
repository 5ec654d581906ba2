// HHR decode step: coarse stage, fine stage and sparse attention.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation" (arXiv 2610.01230):
//   §3.3.1 Eq. 4  q~ = q R (row vector), the rotation of the query;
//   §3.3.1 Eq. 3  page bound U = sum_j max(q~_j l_j, q~_j u_j); pages above the threshold stay;
//   §3.1 Eq. 1, §3.3.2 Eq. 10  query code = sign(q W);
//   §3.1 Eq. 2    Hamming distance by XOR + popcount;
//   §3.3.2, §1    the closest candidates are kept and attended to exactly.
//
// Kernels of a step, all on the caller's stream (after the preparation kernel, which appends
// the new token and writes q~ and the query codes):
//   page_bound_kernel  grid (ceil(Pmax/256), Hkv, B): streams the page extrema once for the G
//                      query heads of a KV head (HBM-bound).
//   select_kernel      grid (Hq, B), 1024 threads: query code, exact top-n_keep pages by a
//                      range-adapted radix select, Hamming distances of the kept pages' keys,
//                      exact top-k tokens by a histogram select; writes ascending indices.
//   attn_kernel        grid (nsplit, Hq, B): split-K softmax attention over gathered K/V rows,
//                      one partial (m, l, o) per workgroup;
//   combine_kernel     grid (B * Hq): merges the partials of each (b, h) into the output and
//                      advances seq_lens when the step appended a token.
// The merge is a kernel of its own: an in-kernel "last workgroup merges" scheme needs a
// device-scope release and acquire in every workgroup, which on gfx950 write back and
// invalidate the whole L2 of an XCD, and costs far more than one small launch.
#include <type_traits>

#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

constexpr int kMaxPages = 16384;       // = HHR_MAX_PAGES
constexpr int kBoundPages = 256;       // pages per bound workgroup (4 per lane)
constexpr int kBoundThreads = 512;     // 8 waves x 16 channels
constexpr int kDistCache = 32768;      // candidate slots whose distance stays in LDS

// ---------------------------------------------------------------------------------------------
// Coarse stage: page bounds (Eq. 3) for the G query heads of one KV head from ONE read of the
// page extrema. Lane l of wave w covers pages p0 + 4l .. p0 + 4l + 3 and channels
// 16w .. 16w + 15: 32 float4 loads per lane are issued at once, q~ (prepared by the preparation
// kernel) is read with wave-uniform loads, and the 8 waves' partial sums meet in LDS.
// Nothing else happens here: while the extrema stream in, any other load waits behind them, so
// work that depends on one would sit on the kernel's tail.
// ---------------------------------------------------------------------------------------------
struct BoundArgs {
  const float* qrot;      // [B][Hq][128] q~ from the preparation kernel
  float* U;               // [B][Hq][Pmax], or (shared) [B][Hkv][Pmax]: max over the group
  int appended;           // a token is appended in this step (seq_lens is advanced at its end)
  int shared;             // one selection per KV head: U of a page = max over its G heads
};

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int G, int SB>   // SB: extrema stored as bf16
__global__ void __launch_bounds__(kBoundThreads)
page_bound_kernel(Shape s, CacheView c, BoundArgs a, float* __restrict__ dbg_U) {
  const int b = blockIdx.z, g = blockIdx.y, p0 = blockIdx.x * kBoundPages;
  const int t = c.seq_lens[b];
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  if (p0 >= P) return;
  const int w = wave_id(), lane = lane_id();
  const int j0 = w * 16;
  const int pl = p0 + lane * 4;
  const int plc = min(pl, s.Pmax - 4);             // in bounds for every lane
  const size_t srow = (size_t(b) * s.Hkv + g) * kD + j0;

  float4 lo[16], hi[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    // non-temporal loads: the extrema are read once per step (measured 14.6 -> 13.8 us at 128K)
    if constexpr (SB) {
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
          static_cast<const uint16_t*>(c.pmin) + (srow + jj) * s.Pmax + plc));
      const u32x2 y = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
          static_cast<const uint16_t*>(c.pmax) + (srow + jj) * s.Pmax + plc));
      lo[jj] = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
      hi[jj] = make_float4(__uint_as_float(y.x << 16), __uint_as_float(y.x & 0xFFFF0000u),
                           __uint_as_float(y.y << 16), __uint_as_float(y.y & 0xFFFF0000u));
    } else {
      const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(
          static_cast<const float*>(c.pmin) + (srow + jj) * s.Pmax + plc));
      const f32x4v y = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(
          static_cast<const float*>(c.pmax) + (srow + jj) * s.Pmax + plc));
      lo[jj] = make_float4(x.x, x.y, x.z, x.w);
      hi[jj] = make_float4(y.x, y.y, y.z, y.w);
    }
  }
  const float* qb = a.qrot + (size_t(b) * s.Hq + size_t(g) * G) * kD + j0;

  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) acc[hh][0] = acc[hh][1] = acc[hh][2] = acc[hh][3] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // max(q l, q u) = q * (q >= 0 ? u : l) since l <= u; q is wave-uniform.
      const float qv = qb[hh * kD + jj];
      const float4 e = (qv >= 0.f) ? hi[jj] : lo[jj];
      acc[hh][0] = fmaf(qv, e.x, acc[hh][0]);
      acc[hh][1] = fmaf(qv, e.y, acc[hh][1]);
      acc[hh][2] = fmaf(qv, e.z, acc[hh][2]);
      acc[hh][3] = fmaf(qv, e.w, acc[hh][3]);
    }
  }

  __shared__ float4 red[kBoundThreads / kWave][G][kBoundPages / 4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    red[w][hh][lane] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
  __syncthreads();
  if (a.shared) {
    // one bound per page for the whole group: the largest of its heads' bounds (the group's
    // pages are chosen once; each head's own bound goes to the debug output only)
    for (int pp = threadIdx.x; pp < kBoundPages; pp += kBoundThreads) {
      const int p = p0 + pp;
      if (p < P) {
        float um = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float sum = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kBoundThreads / kWave; ++w2)
            sum += reinterpret_cast<const float*>(&red[w2][hh][0])[pp];
          um = fmaxf(um, sum);
          if (dbg_U) dbg_U[(size_t(b) * s.Hq + g * G + hh) * s.Pmax + p] = sum;
        }
        a.U[(size_t(b) * s.Hkv + g) * s.Pmax + p] = um;
      }
    }
    return;
  }
  for (int o = threadIdx.x; o < G * kBoundPages; o += kBoundThreads) {
    const int hh = o / kBoundPages, pp = o % kBoundPages;
    const int p = p0 + pp;
    if (p < P) {
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kBoundThreads / kWave; ++w2)
        sum += reinterpret_cast<const float*>(&red[w2][hh][0])[pp];
      const size_t oi = (size_t(b) * s.Hq + g * G + hh) * s.Pmax + p;
      a.U[oi] = sum;
      if (dbg_U) dbg_U[oi] = sum;
    }
  }
}

// Order-preserving map of a bound to uint32 where SMALLER means LARGER U (so the kept pages are
// the smallest keys); -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t desc_key(float u) {
  if (u == 0.f) u = 0.f;
  const uint32_t x = __float_as_uint(u);
  const uint32_t asc = (x & 0x80000000u) ? ~x : (x | 0x80000000u);
  return ~asc;
}

struct SelectArgs {
  const uint32_t* qcode;  // [B][Hq][NW]
  const float* U;
  int32_t* idx;       // [B][Hq][kcap]
  int32_t* cnt;       // [B][Hq]
  double rho;
  int kcap;
  int istride;        // row stride of idx: kcap live entries, then one trash entry per lane
  int appended;       // a token is appended in this step (seq_lens is advanced at its end)
  int fine;           // 0: no Hamming ranking, every candidate is taken (pages-only stages)
};

// ---------------------------------------------------------------------------------------------
// Selection, one workgroup per (b, h).
//   Coarse: the n_keep pages of largest U, ties to the lower index. Keys are ranked by a radix
//   select over rel = key - min(key), 12 bits at a time from the top set bit of the range; as
//   soon as the threshold bin holds at most 64 keys, one wave ranks them by (key, page) and the
//   kept set is a lexicographic cut; only more than 64 exactly equal keys at the threshold
//   fall back to breaking ties in page order by one scan. EPT pages per thread (contiguous:
//   thread i owns pages [i EPT, i EPT + EPT)).
//   Fine: Hamming distance of every key of the kept pages (slots in ascending token order),
//   histogram over D in [0, NB], the smallest D* with #(D <= D*) >= k_eff, and one scan that
//   places every slot with D < D* and the first k_eff - #(D < D*) slots with D == D*.
// The kernel runs on one CU per (b, h) and is bound by instruction issue, so every per-element
// step is branch-free: a lane with nothing to record still executes the LDS or global write,
// aimed at a dummy entry of its own past the live data (no divergent branch, no bank conflict).
// ---------------------------------------------------------------------------------------------
constexpr int kRadixBins = 1 << 12;
constexpr int kRadixBits = 12;
constexpr int kEmitSPT = 8;    // cached distances per thread per emit chunk
static_assert(16 % kEmitSPT == 0 && kEmitSPT >= 8, "an emit chunk must not cross a page (page sizes 16, 32)");

template <int NB, int EPT, int NT, int SHARED>
__global__ void __launch_bounds__(NT)
select_kernel(Shape s, CacheView c, SelectArgs a, DebugView dbg) {
  constexpr int kSelThreads = NT;
  constexpr int kSelWaves = NT / kWave;
  constexpr int NW = NB / 32;
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  constexpr uint32_t kNone = NB == 128 ? 0xFFu : 0xFFFFu;   // distance of a slot past the end
  constexpr int HB = kRadixBins > NB + 1 ? kRadixBins : NB + 1;
  // selection unit: a query head, or (SHARED) a KV head whose G query heads share the choice
  const int h = blockIdx.x, b = blockIdx.y, g = SHARED ? h : h / s.G;
  const int bh = b * (SHARED ? s.Hkv : s.Hq) + h;
  const int ncodes = SHARED ? s.G : 1;            // query codes whose nearest distance counts
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int t = c.seq_lens[b];                   // position of the appended token, if any
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;

  // Live entries, then one dummy entry per lane.
  __shared__ int32_t s_pages[kMaxPages + kWave];
  __shared__ __align__(16) DT s_dist[kDistCache + kWave];
  __shared__ __align__(16) uint32_t s_hist[HB + kWave];
  __shared__ uint32_t s_qw[SHARED ? 8 : 1][NW];   // query code(s)
  __shared__ int s_wt[2][kSelWaves];
  __shared__ uint32_t s_mm[2][kSelWaves];
  __shared__ int s_pick[3];
  __shared__ uint32_t s_ckey[kWave];   // keys of the threshold bin (when it holds <= 64)
  __shared__ int s_cidx[kWave];
  __shared__ int s_ncand;
  BlockScan<kSelWaves> scan{s_wt, 0};

  int32_t* out_idx = a.idx + size_t(bh) * a.istride;
  if (L == 0) {
    if (tid == 0) {
      a.cnt[bh] = 0;
      if (dbg.page_count) dbg.page_count[bh] = 0;
      if (dbg.token_count) dbg.token_count[bh] = 0;
    }
    return;
  }
  const int n_keep = min(P, max(1, int(ceil(a.rho * double(P)))));

  // ---- query code (from the code workgroups of the bound kernel), page keys to registers,
  // histograms cleared
  if (tid < ncodes * NW)
    s_qw[tid / NW][tid % NW] = a.qcode[(size_t(b) * s.Hq + (SHARED ? g * s.G : h)) * NW + tid];
  if (tid == 0) s_ncand = 0;
  for (int i = tid; i < HB; i += kSelThreads) s_hist[i] = 0;
  uint32_t key[EPT];
  bool valid[EPT];
  {
    // whole float4 loads at clamped addresses (rows are Pmax long, Pmax a multiple of 4)
    const float4* U4 = reinterpret_cast<const float4*>(a.U + size_t(bh) * s.Pmax);
    const int last4 = s.Pmax / 4 - 1;
    float u[EPT];
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      const float4 x = U4[min(tid * (EPT / 4) + e / 4, last4)];
      u[e] = x.x; u[e + 1] = x.y; u[e + 2] = x.z; u[e + 3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      valid[e] = tid * EPT + e < P;
      const uint32_t k = materialize(desc_key(u[e]));   // computed by every lane
      key[e] = valid[e] ? k : 0xFFFFFFFFu;
    }
  }

  // ---- key range (one barrier for both reductions)
  uint32_t kmin, kmax;
  {
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      lmin = min(lmin, key[e]);                  // an invalid key is the largest value
      lmax = max(lmax, valid[e] ? key[e] : 0u);
    }
    lmin = wave_min_u32(lmin);
    lmax = wave_max_u32(lmax);
    if (lane == 0) {
      s_mm[0][w] = lmin;
      s_mm[1][w] = lmax;
    }
    __syncthreads();   // also publishes s_qw and the cleared histograms
    kmin = wave_min_u32(s_mm[0][lane % kSelWaves]);
    kmax = wave_max_u32(s_mm[1][lane % kSelWaves]);
  }


  // ---- coarse selection. The kept set is described, where possible, by a cut (ck, ci): page
  // i is kept iff (key_i, i) <= (ck, ci) lexicographically (smaller key = larger U, ties to the
  // lower index). Otherwise (more than 64 exactly equal keys straddle the cut) by the final
  // radix prefix plus the number `need` of its elements to take in page order.
  int need = n_keep;        // still to take among elements matching `prefix`
  uint32_t prefix = 0;      // high bits of rel fixed so far
  int res_lo = 0;           // elements compare on rel >> res_lo
  bool cut = true;
  uint32_t ck = 0xFFFFFFFFu;
  int ci = 0x7FFFFFFF;
  if (n_keep < P) {
    cut = false;
    int cur_hi = (kmax == kmin) ? -1 : 31 - __clz(int(kmax - kmin));
    bool first = true;
    while (cur_hi >= 0) {
      const int cur_lo = max(cur_hi - (kRadixBits - 1), 0);
      const int width = cur_hi - cur_lo + 1;
      const uint32_t dmask = (1u << width) - 1u;
      if (first) {
        // every valid key matches the empty prefix
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          const uint32_t rel = key[e] - kmin;
          atomicAdd(&s_hist[valid[e] ? (rel >> cur_lo) & dmask : HB + lane], 1u);
        }
      } else {
        // few keys match a longer prefix: waves without a match skip the atomic
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          const uint32_t rel = key[e] - kmin;
          if (valid[e] && uint32_t(uint64_t(rel) >> (cur_hi + 1)) == prefix)
            atomicAdd(&s_hist[(rel >> cur_lo) & dmask], 1u);
        }
      }
      first = false;
      __syncthreads();
      // thread i owns bins [BPT i, BPT i + BPT): read them, clear them for the next pass
      constexpr int BPT = kRadixBins / kSelThreads;
      uint32_t hb[BPT];
      int loc = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        hb[j] = s_hist[tid * BPT + j];
        s_hist[tid * BPT + j] = 0;
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
        s_pick[0] = fbin;
        s_pick[1] = fbefore;
        s_pick[2] = fcnt;
      }
      __syncthreads();
      const int d = s_pick[0], before = s_pick[1], in_bin = s_pick[2];
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
        // few keys share the threshold bin: wave 0 ranks them by (key, index) and the
        // need-th smallest becomes the cut
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          if (valid[e] && ((key[e] - kmin) >> res_lo) == prefix) {
            const int j = atomicAdd(&s_ncand, 1);
            s_ckey[j] = key[e];
            s_cidx[j] = tid * EPT + e;
          }
        }
        __syncthreads();
        if (w == 0) {
          // (key, index) of every lane compared with the in_bin entries through register
          // reads (in_bin is uniform and usually a handful)
          const uint32_t kl = lane < in_bin ? s_ckey[lane] : 0xFFFFFFFFu;
          const uint32_t il = lane < in_bin ? uint32_t(s_cidx[lane]) : 0x7FFFFFFFu;
          const uint64_t vl = (uint64_t(kl) << 32) | il;
          int rank = 0;
          for (int j = 0; j < in_bin; ++j) {
            const uint64_t vj = (uint64_t(__builtin_amdgcn_readlane(kl, j)) << 32) |
                                uint32_t(__builtin_amdgcn_readlane(il, j));
            rank += vj < vl ? 1 : 0;
          }
          if (lane < in_bin && rank == need - 1) {
            s_pick[0] = int(kl);
            s_pick[1] = il;
          }
        }
        __syncthreads();
        ck = uint32_t(s_pick[0]);
        ci = s_pick[1];
        cut = true;
        break;
      }
    }
  }
  if (cut) {
    bool tk[EPT];
    int n = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      tk[e] = valid[e] && (key[e] < ck || (key[e] == ck && tid * EPT + e <= ci));
      n += tk[e] ? 1 : 0;
    }
    int tot;
    int pos = scan.excl(n, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      s_pages[tk[e] ? pos : kMaxPages + lane] = tid * EPT + e;
      pos += tk[e] ? 1 : 0;
    }
  } else {
    // rel >> res_lo below prefix: taken; equal: taken in page order up to `need`
    bool lt[EPT], eq[EPT];
    int nlt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t v = (key[e] - kmin) >> res_lo;
      lt[e] = valid[e] && v < prefix;
      eq[e] = valid[e] && v == prefix;
      nlt += lt[e] ? 1 : 0;
      neq += eq[e] ? 1 : 0;
    }
    int tot;
    const int ex = scan.excl((nlt << 16) | neq, &tot);
    int eq_seen = ex & 0xFFFF;
    int pos = (ex >> 16) + min(eq_seen, need);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool take = lt[e] || (eq[e] && eq_seen < need);
      eq_seen += eq[e] ? 1 : 0;
      s_pages[take ? pos : kMaxPages + lane] = tid * EPT + e;
      pos += take ? 1 : 0;
    }
  }
  __syncthreads();
  if (dbg.page_ids) {
    for (int i = tid; i < n_keep; i += kSelThreads)
      dbg.page_ids[size_t(bh) * s.Pmax + i] = s_pages[i];
    if (tid == 0 && dbg.page_count) dbg.page_count[bh] = n_keep;
  } else if (tid == 0 && dbg.page_count) {
    dbg.page_count[bh] = n_keep;
  }

  // ---- fine stage: Hamming distance of every candidate slot (§3.1 Eq. 2)
  uint32_t qw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) qw[i] = s_qw[0][i];
  // distance of a code: to the query code, or (SHARED) the smallest over the group's codes
  auto code_dist = [&](const uint4 (&x)[NW / 4]) -> uint32_t {
    uint32_t dd = 0;
#pragma unroll
    for (int v = 0; v < NW / 4; ++v)
      dd += __popc(x[v].x ^ qw[4 * v]) + __popc(x[v].y ^ qw[4 * v + 1]) +
            __popc(x[v].z ^ qw[4 * v + 2]) + __popc(x[v].w ^ qw[4 * v + 3]);
    if constexpr (SHARED) {
      for (int i = 1; i < ncodes; ++i) {   // uniform; the other codes are LDS broadcasts
        uint32_t di = 0;
#pragma unroll
        for (int v = 0; v < NW / 4; ++v)
          di += __popc(x[v].x ^ s_qw[i][4 * v]) + __popc(x[v].y ^ s_qw[i][4 * v + 1]) +
                __popc(x[v].z ^ s_qw[i][4 * v + 2]) + __popc(x[v].w ^ s_qw[i][4 * v + 3]);
        dd = min(dd, di);
      }
    }
    return dd;
  };
  const int lgS = (s.S == 16) ? 4 : 5;
  const int nslots = n_keep << lgS;
  const bool cache_d = nslots <= kDistCache;
  const uint32_t* cbase = c.codes + (size_t(b) * s.Hkv + g) * s.Lmax * NW;
  auto slot_token = [&](int slot) { return (s_pages[slot >> lgS] << lgS) + (slot & (s.S - 1)); };
  auto distance = [&](int tk) -> uint32_t {
    if (tk >= L) return kNone;
    if (!a.fine) return 0u;
    const uint4* cp = reinterpret_cast<const uint4*>(cbase + size_t(tk) * NW);
    uint4 x[NW / 4];
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) x[v] = cp[v];
    return code_dist(x);
  };
  uint32_t* whist = s_hist;   // bins 0..NB (cleared by the coarse stage's last pass)
  // Batches of 8 x (1024 / NT) slots per thread: all code loads of a batch are issued before
  // any is used.
  constexpr int BAT = 8 * (1024 / NT) / (NW / 4);
  for (int base = 0; base < nslots; base += BAT * kSelThreads) {
    int tt[BAT];
    uint4 cw[BAT][NW / 4];
#pragma unroll
    for (int u = 0; u < BAT; ++u) {
      const int slot = base + u * kSelThreads + tid;
      const int tk = materialize(slot_token(min(slot, nslots - 1)));   // every lane
      tt[u] = (slot < nslots) ? tk : L;
    }
    if (a.fine) {   // uniform
#pragma unroll
      for (int u = 0; u < BAT; ++u) {
        const uint4* cp = reinterpret_cast<const uint4*>(cbase + size_t(min(tt[u], L - 1)) * NW);
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) cw[u][v] = cp[v];
      }
    } else {
      // no fine stage: every live candidate gets distance 0 (the query code itself)
#pragma unroll
      for (int u = 0; u < BAT; ++u)
#pragma unroll
        for (int v = 0; v < NW / 4; ++v)
          cw[u][v] = make_uint4(qw[4 * v], qw[4 * v + 1], qw[4 * v + 2], qw[4 * v + 3]);
    }
#pragma unroll
    for (int u = 0; u < BAT; ++u) {
      const int slot = base + u * kSelThreads + tid;
      // (without the fine stage every code equals the first query code: distance 0)
      const uint32_t dd = a.fine ? code_dist(cw[u]) : 0u;
      const bool live = tt[u] < L;                // implies slot < nslots
      atomicAdd(live ? &whist[dd] : &s_hist[HB + lane], 1u);
      // (without the LDS cache every lane writes its dummy entry; the emit recomputes)
      s_dist[cache_d && slot < nslots ? slot : kDistCache + lane] = DT(live ? dd : kNone);
    }
  }
  __syncthreads();
  if (cache_d && dbg.dist) {
    for (int i = tid; i < nslots; i += kSelThreads) {
      const uint32_t dd = s_dist[i];
      dbg.dist[size_t(bh) * s.Lmax + i] = uint16_t(dd == kNone ? 0xFFFFu : dd);
    }
  }

  // ---- token threshold: smallest D* with #(D <= D*) >= k_eff, found by wave 0 alone
  if (w == 0) {
    constexpr int BPL = (NB + 1 + kWave - 1) / kWave;   // distance bins per lane
    int cnt[BPL];
    int tot_d = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      const int v = int(s_hist[min(bin, NB)]);
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
  const int dstar = s_pick[0];
  const int k_eff = s_pick[2];
  const int need_eq = k_eff - s_pick[1];

  // ---- emit the selected tokens in ascending position (slots are in ascending t): one scan
  // of the per-thread (#lt, #eq) counts places every slot. The list is assembled in LDS (the
  // histograms are done with) and copied out coalesced when it fits; otherwise it is written
  // straight to global memory. A slot not taken goes to the lane's trash entry.
  int32_t* trash = out_idx + a.kcap + lane;
  int32_t* dbg_idx = dbg.token_idx ? dbg.token_idx + size_t(bh) * a.kcap : nullptr;
  int32_t* stage = reinterpret_cast<int32_t*>(s_hist);
  const bool staged = k_eff <= HB;
  int run_lt = 0, run_eq = 0;
  if (cache_d) {
    const int nchunks = (nslots + kSelThreads * kEmitSPT - 1) / (kSelThreads * kEmitSPT);
    for (int ch = 0; ch < nchunks; ++ch) {
      const int s0 = (ch * kSelThreads + tid) * kEmitSPT;
      const bool any = s0 < nslots;
      const int sc = any ? s0 : 0;                // read position (in bounds)
      // the chunk's distances as 32-bit words (sc is a multiple of kEmitSPT: aligned)
      constexpr int kPer = 4 / int(sizeof(DT));            // distances per word
      constexpr int kWords = kEmitSPT / kPer;
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
      for (int u = 0; u < kEmitSPT; ++u)
        dv[u] = (wv[u / kPer] >> (8 * sizeof(DT) * (u % kPer))) & kNone;
#pragma unroll
      for (int u = 0; u < kEmitSPT; ++u) dv[u] = (any && s0 + u < nslots) ? dv[u] : kNone;
      int nlt = 0, neq = 0;
#pragma unroll
      for (int u = 0; u < kEmitSPT; ++u) {
        nlt += dv[u] < uint32_t(dstar) ? 1 : 0;
        neq += dv[u] == uint32_t(dstar) ? 1 : 0;
      }
      // the chunk's slots lie in one page (kEmitSPT divides the page size)
      const int t0 = slot_token(sc);
      int tot;
      const int ex = scan.excl((nlt << 16) | neq, &tot);
      const int eq0 = run_eq + (ex & 0xFFFF);
      const int pos0 = run_lt + (ex >> 16) + min(eq0, need_eq);
      int eq_seen = eq0, pos = pos0;
      if (staged) {
#pragma unroll
        for (int u = 0; u < kEmitSPT; ++u) {
          const bool is_eq = dv[u] == uint32_t(dstar);
          const bool take = dv[u] < uint32_t(dstar) || (is_eq && eq_seen < need_eq);
          eq_seen += is_eq ? 1 : 0;
          stage[take ? pos : HB + lane] = t0 + u;
          pos += take ? 1 : 0;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kEmitSPT; ++u) {
          const bool is_eq = dv[u] == uint32_t(dstar);
          const bool take = dv[u] < uint32_t(dstar) || (is_eq && eq_seen < need_eq);
          eq_seen += is_eq ? 1 : 0;
          *(take ? out_idx + pos : trash) = t0 + u;
          pos += take ? 1 : 0;
        }
      }
      if (dbg_idx && !staged) {
        eq_seen = eq0;
        pos = pos0;
        for (int u = 0; u < kEmitSPT; ++u) {
          const bool is_eq = dv[u] == uint32_t(dstar);
          const bool take = dv[u] < uint32_t(dstar) || (is_eq && eq_seen < need_eq);
          eq_seen += is_eq ? 1 : 0;
          if (take) dbg_idx[pos++] = t0 + u;
        }
      }
      run_lt += tot >> 16;
      run_eq += tot & 0xFFFF;
    }
    if (staged) {
      __syncthreads();
      const int n4 = k_eff >> 2;   // rows of idx start 16-byte aligned
      for (int i = tid; i < n4; i += kSelThreads)
        reinterpret_cast<int4*>(out_idx)[i] = reinterpret_cast<const int4*>(stage)[i];
      for (int i = 4 * n4 + tid; i < k_eff; i += kSelThreads) out_idx[i] = stage[i];
      if (dbg_idx)
        for (int i = tid; i < k_eff; i += kSelThreads) dbg_idx[i] = stage[i];
    }
  } else {
    for (int base = 0; base < nslots; base += kSelThreads) {
      const int slot = base + tid;
      int tk = 0;
      uint32_t dd = kNone;
      if (slot < nslots) {
        tk = slot_token(slot);
        dd = distance(tk);
        if (dbg.dist) dbg.dist[size_t(bh) * s.Lmax + slot] = uint16_t(dd == kNone ? 0xFFFFu : dd);
      }
      const bool is_lt = dd < uint32_t(dstar), is_eq = dd == uint32_t(dstar);
      int tot;
      const int ex = scan.excl((int(is_lt) << 16) | int(is_eq), &tot);
      const int eq_seen = run_eq + (ex & 0xFFFF);
      const int pos = run_lt + (ex >> 16) + min(eq_seen, need_eq);
      if (is_lt || (is_eq && eq_seen < need_eq)) {
        out_idx[pos] = tk;
        if (dbg_idx) dbg_idx[pos] = tk;
      }
      run_lt += tot >> 16;
      run_eq += tot & 0xFFFF;
    }
  }
  if (tid == 0) {
    a.cnt[bh] = k_eff;
    if (dbg.token_count) dbg.token_count[bh] = k_eff;
  }
}

// ---------------------------------------------------------------------------------------------
// Sparse attention over the selected rows, split-K: one chunk of rows per workgroup.
// A row of d = 128 is read as 16-byte pieces: 16 lanes per row for bf16, 32 for fp32. Every
// wave issues all its K and V loads up front, then computes logits, the workgroup maximum, the
// exponentials and the weighted V sum. The workgroup writes (o, m, l) for its chunk; the
// combine kernel merges the chunks of each (b, h).
// ---------------------------------------------------------------------------------------------
template <int BF16>
struct AttnShape {
  static constexpr int EPL = BF16 ? 8 : 4;        // elements per lane per row
  static constexpr int LPR = kD / EPL;            // lanes per row
  static constexpr int RPI = kWave / LPR;         // rows per wave-wide load
  static constexpr int ITER = 8;                  // loads per lane for K (and for V)
  static constexpr int RPW = RPI * ITER;          // rows per wave
  static constexpr int CHUNK = 4 * RPW;           // rows per workgroup (4 waves)
};

__device__ __forceinline__ void unpack(const uint4& x, float (&f)[8]) {
  f[0] = __uint_as_float(x.x << 16); f[1] = __uint_as_float(x.x & 0xFFFF0000u);
  f[2] = __uint_as_float(x.y << 16); f[3] = __uint_as_float(x.y & 0xFFFF0000u);
  f[4] = __uint_as_float(x.z << 16); f[5] = __uint_as_float(x.z & 0xFFFF0000u);
  f[6] = __uint_as_float(x.w << 16); f[7] = __uint_as_float(x.w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack(const uint4& x, float (&f)[4]) {
  f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
  f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
}

struct AttnArgs {
  const int32_t* idx;   // rows of selected tokens: per (b, h), or (shared) per (b, KV head)
  const int32_t* cnt;
  float* part;        // [B][Hq][nsplit][kD + 2]: o[0..127], m, l
  int kcap, istride, nsplit;
  int shared;
  float scale_log2e;
};

template <int BF16>
__global__ void __launch_bounds__(256)
attn_kernel(Shape s, const void* __restrict__ K, const void* __restrict__ V,
            const void* __restrict__ q, AttnArgs a) {
  using A = AttnShape<BF16>;
  constexpr int EPL = A::EPL, LPR = A::LPR, RPI = A::RPI, ITER = A::ITER;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / s.G;
  const int bh = b * s.Hq + h;
  const int bu = a.shared ? b * s.Hkv + g : bh;   // selection unit whose tokens are attended
  const int count = a.cnt[bu];
  const int w = wave_id(), lane = lane_id();
  const int rg = lane / LPR, sub = lane % LPR;
  const int row0 = split * A::CHUNK + w * A::RPW;
  const size_t esz = BF16 ? 2 : 4;
  const bool live = split * A::CHUNK < count;   // uniform over the workgroup

  __shared__ float s_m[4], s_l[4];
  __shared__ float s_o[4][kD];

  float M = -INFINITY;
  float l = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  if (live) {
    // query slice (scaled into the log2 domain)
    float qv[EPL];
    const size_t qo = size_t(bh) * kD + sub * EPL;
    if (s.q_bf16) {
      if constexpr (EPL == 8) {
        float f[8];
        unpack(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + qo), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = f[e];
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + qo);
        qv[0] = __uint_as_float(x.x << 16); qv[1] = __uint_as_float(x.x & 0xFFFF0000u);
        qv[2] = __uint_as_float(x.y << 16); qv[3] = __uint_as_float(x.y & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(q) + qo + e);
        qv[e] = x.x; qv[e + 1] = x.y; qv[e + 2] = x.z; qv[e + 3] = x.w;
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= a.scale_log2e;

    // selected rows: indices first (no branches, so all loads stay in flight together)
    const size_t kvrow0 = (size_t(b) * s.Hkv + g) * s.Lmax;
    const int32_t* ib = a.idx + size_t(bu) * a.istride;
    int tok[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) tok[it] = ib[min(row0 + it * RPI + rg, count - 1)];
    uint4 kr[ITER], vr[ITER];
    const char* Kc = static_cast<const char*>(K);
    const char* Vc = static_cast<const char*>(V);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      // indices come from select_kernel and are < seq_len; the clamp only keeps any reader in
      // bounds of the cache
      const int t = min(max(tok[it], 0), s.Lmax - 1);
      const size_t off = ((kvrow0 + size_t(t)) * kD + sub * EPL) * esz;
      kr[it] = *reinterpret_cast<const uint4*>(Kc + off);
      vr[it] = *reinterpret_cast<const uint4*>(Vc + off);
    }
    // keep all 2 x ITER row loads in flight before the first use
    __builtin_amdgcn_sched_barrier(0);

    // logits (log2 domain)
    float sc[ITER];
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      float f[EPL];
      unpack(kr[it], f);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qv[e], f[e], d);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      sc[it] = (row0 + it * RPI + rg < count) ? d : -INFINITY;
      mx = fmaxf(mx, sc[it]);
    }
    mx = wave_max(mx);
    if (lane == 0) s_m[w] = mx;
    __syncthreads();
    M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const float p = (sc[it] == -INFINITY) ? 0.f : exp2f(sc[it] - M);
      l += p;
      float f[EPL];
      unpack(vr[it], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, f[e], o[e]);
    }
    // reduce across the row groups of the wave (lanes that share `sub`)
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
      l += __shfl_xor(l, off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], off);
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[w][sub * EPL + e] = o[e];
      if (sub == 0) s_l[w] = l;
    }
    __syncthreads();
  } else {
    for (int i = threadIdx.x; i < 4 * kD; i += blockDim.x) s_o[i / kD][i % kD] = 0.f;
    if (threadIdx.x < 4) s_l[threadIdx.x] = 0.f;
    __syncthreads();
  }
  float* pp = a.part + (size_t(bh) * a.nsplit + split) * (kD + 2);
  if (threadIdx.x < kD) {
    const int d = threadIdx.x;
    pp[d] = s_o[0][d] + s_o[1][d] + s_o[2][d] + s_o[3][d];
  }
  if (threadIdx.x == 0) {
    pp[kD] = M;
    pp[kD + 1] = s_l[0] + s_l[1] + s_l[2] + s_l[3];
  }
}

// Merge of the split partials of one (b, h): o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// NG groups of 128 threads (thread = output dimension) take every NG-th partial; each group
// reads its partials in batches of 16, all loads of a batch issued before any use, merged
// without branches (an empty partial has m = -inf, l = 0 and gets weight 0); the groups then
// meet in LDS. The sparse step's last kernel also commits an append: every earlier kernel of
// the step read seq_lens[b] = t and worked on t + 1 tokens; the workgroup of head 0 now stores
// t + 1.
template <int NG>
__global__ void __launch_bounds__(kD * NG)
combine_kernel(const float* __restrict__ part, int nsplit, float* __restrict__ out,
               int32_t* __restrict__ seq_lens, int Hq, int Lmax, int appended) {
  constexpr int CB = 16;
  const int bh = blockIdx.x, d = threadIdx.x % kD, grp = threadIdx.x / kD;
  if (appended && threadIdx.x == 0 && bh % Hq == 0) {
    const int b = bh / Hq;
    const int t = seq_lens[b];
    if (t >= 0 && t < Lmax) seq_lens[b] = t + 1;
  }
  const float* pb = part + size_t(bh) * nsplit * (kD + 2);
  float Mx = -INFINITY, Ls = 0.f, Os = 0.f;
  for (int i0 = grp * CB; i0 < nsplit; i0 += NG * CB) {
    float m[CB], l[CB], o[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float* pi = pb + size_t(min(i0 + u, nsplit - 1)) * (kD + 2);
      m[u] = pi[kD];
      l[u] = pi[kD + 1];
      o[u] = pi[d];
    }
    __builtin_amdgcn_sched_barrier(0);
    float bm = Mx;
#pragma unroll
    for (int u = 0; u < CB; ++u) bm = (i0 + u < nsplit) ? fmaxf(bm, m[u]) : bm;
    // rescale what has been summed so far to the new maximum, then add this batch
    const float f0 = (bm == -INFINITY || Mx == -INFINITY) ? 0.f : exp2f(Mx - bm);
    Ls *= f0;
    Os *= f0;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const bool ok = i0 + u < nsplit && l[u] > 0.f;
      const float f = ok ? exp2f(m[u] - bm) : 0.f;
      Ls = fmaf(ok ? l[u] : 0.f, f, Ls);
      Os = fmaf(ok ? o[u] : 0.f, f, Os);
    }
    Mx = bm;
  }
  if constexpr (NG > 1) {
    __shared__ float s_m[NG], s_l[NG], s_o[NG][kD];
    s_o[grp][d] = Os;
    if (d == 0) {
      s_m[grp] = Mx;
      s_l[grp] = Ls;
    }
    __syncthreads();
    if (grp != 0) return;
    float M = s_m[0];
#pragma unroll
    for (int i = 1; i < NG; ++i) M = fmaxf(M, s_m[i]);
    Ls = 0.f;
    Os = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float f = s_m[i] == -INFINITY ? 0.f : exp2f(s_m[i] - M);
      Ls = fmaf(s_l[i], f, Ls);
      Os = fmaf(s_o[i][d], f, Os);
    }
  }
  out[size_t(bh) * kD + d] = (Ls > 0.f) ? Os / Ls : 0.f;
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

DecodePlan plan_decode(const Shape& s, double rho, int k, float scale, Stages stages,
                       int shared) {
  DecodePlan p{};
  p.stages = stages;
  p.shared = shared;
  if (stages == Stages::kPagesOnly) {
    // every token of the kept pages: at most max(1, ceil(rho Pmax)) pages of S tokens
    const long long keep = (long long)ceil(rho * double(s.Pmax));
    const long long toks = (keep < 1 ? 1 : keep) * s.S;
    p.kcap = toks < s.Lmax ? int(toks) : s.Lmax;
  } else {
    p.kcap = k < s.Lmax ? k : s.Lmax;
  }
  if (stages == Stages::kCodesOnly) rho = 1.0;   // every page is a candidate
  // (group-shared bf16: the gathered matrix-core attention, kGatherChunk positions per
  // workgroup; otherwise the per-head kernel)
  p.chunk = shared && s.kv_bf16 ? kGatherChunk
                                : (s.kv_bf16 ? AttnShape<1>::CHUNK : AttnShape<0>::CHUNK);
  p.nsplit = (p.kcap + p.chunk - 1) / p.chunk;
  p.rho = rho;
  p.scale = scale;
  const size_t BH = size_t(s.B) * s.Hq;
  const size_t NU = size_t(s.B) * (shared ? s.Hkv : s.Hq);   // selection units
  size_t off = 0;
  p.off_qrot = off;   off = align256(off + BH * kD * sizeof(float));
  p.off_qcode = off;  off = align256(off + BH * s.NW * sizeof(uint32_t));
  p.off_U = off;      off = align256(off + NU * s.Pmax * sizeof(float));
  p.istride = ((p.kcap + 3) & ~3) + kWave;   // 16-byte aligned rows, then the trash entries
  p.off_idx = off;    off = align256(off + NU * p.istride * sizeof(int32_t));
  p.off_cnt = off;    off = align256(off + NU * sizeof(int32_t));
  p.off_part = off;   off = align256(off + BH * p.nsplit * (kD + 2) * sizeof(float));
  if (stages == Stages::kCodesOnly) {   // distances and per-slice histograms of the scan
    p.off_dist = off;  off = align256(off + NU * s.Lmax * (s.NB == 128 ? 1 : 2));
    p.off_hist = off;  off = align256(off + NU * scan_slices(s) * (s.NB + 1) * sizeof(int32_t));
  }
  p.total = off;
  return p;
}

template <int G>
static void launch_bound_t(const Shape& s, const CacheView& c, const BoundArgs& a,
                           const DebugView& dbg, hipStream_t st) {
  dim3 grid((s.Pmax + kBoundPages - 1) / kBoundPages, s.Hkv, s.B);
  if (s.sum_bf16)
    launch_kernel(page_bound_kernel<G, 1>, grid, dim3(kBoundThreads), st, kernel_timer(dbg, 1),
                  s, c, a, dbg.bounds);
  else
    launch_kernel(page_bound_kernel<G, 0>, grid, dim3(kBoundThreads), st, kernel_timer(dbg, 1),
                  s, c, a, dbg.bounds);
}

template <int NB, int EPT, int NT>
static void launch_select_t(const Shape& s, const CacheView& c, const SelectArgs& a,
                            const DebugView& dbg, int shared, hipStream_t st) {
  if (shared)
    launch_kernel(select_kernel<NB, EPT, NT, 1>, dim3(s.Hkv, s.B), dim3(NT), st,
                  kernel_timer(dbg, 2), s, c, a, dbg);
  else
    launch_kernel(select_kernel<NB, EPT, NT, 0>, dim3(s.Hq, s.B), dim3(NT), st,
                  kernel_timer(dbg, 2), s, c, a, dbg);
}

// Workgroup size of the selection (measured on MI355X: 1024 and 512 threads tie; 256 threads
// are slower because the per-thread histogram and load batches grow); pages per thread follow
// from the page capacity.
constexpr int kSelNT = 1024;

template <int NB>
static void launch_select_nb(const Shape& s, const CacheView& c, const SelectArgs& a,
                             const DebugView& dbg, int shared, hipStream_t st) {
  static_assert(kMaxPages <= 16 * kSelNT, "16 pages per thread cover the page capacity");
  const int ept = (s.Pmax + kSelNT - 1) / kSelNT;
  if (ept <= 4) launch_select_t<NB, 4, kSelNT>(s, c, a, dbg, shared, st);
  else if (ept <= 8) launch_select_t<NB, 8, kSelNT>(s, c, a, dbg, shared, st);
  else launch_select_t<NB, 16, kSelNT>(s, c, a, dbg, shared, st);
}

hipError_t launch_decode(const Shape& s, const DecodePlan& p, const CacheView& c,
                         const void* k_new, const void* v_new, const void* q, const float* R,
                         const float* W, void* ws, float* out, const DebugView& dbg,
                         hipStream_t st) {
  char* base = static_cast<char*>(ws);
  float* qrot = reinterpret_cast<float*>(base + p.off_qrot);
  uint32_t* qcode = reinterpret_cast<uint32_t*>(base + p.off_qcode);
  float* U = reinterpret_cast<float*>(base + p.off_U);
  int32_t* idx = reinterpret_cast<int32_t*>(base + p.off_idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + p.off_cnt);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  hipError_t e = hipSuccess;
#define HHR_CHECK() \
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // seq_lens[b] stays t during the step; every kernel works on t + 1 tokens when a token is
  // appended, and the last kernel stores t + 1.
  e = launch_prep(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg.q_rot, dbg.q_code,
                  PrepMode::kDecode, kernel_timer(dbg, 0), st);
  if (e != hipSuccess) return e;
  // codes only: every page is kept, so no bound is needed (the selection reads U but keeps all)
  if (p.stages != Stages::kCodesOnly) {
    BoundArgs ba{qrot, U, k_new != nullptr ? 1 : 0, p.shared};
    switch (s.G) {
      case 1: launch_bound_t<1>(s, c, ba, dbg, st); break;
      case 2: launch_bound_t<2>(s, c, ba, dbg, st); break;
      case 4: launch_bound_t<4>(s, c, ba, dbg, st); break;
      default: launch_bound_t<8>(s, c, ba, dbg, st); break;
    }
    HHR_CHECK();
  }
  if (p.stages == Stages::kCodesOnly) {
    // every token is a candidate: the scan spread over slices of the context
    ScanArgs sc{qcode, base + p.off_dist, reinterpret_cast<int32_t*>(base + p.off_hist), idx, cnt,
                p.kcap, p.istride, scan_slices(s), k_new != nullptr ? 1 : 0, p.shared};
    e = launch_scan_select(s, c, sc, dbg, st);
    if (e != hipSuccess) return e;
  } else {
    SelectArgs sa{qcode, U, idx, cnt, p.rho, p.kcap, p.istride, k_new != nullptr ? 1 : 0,
                  p.stages == Stages::kPagesOnly ? 0 : 1};
    if (s.NB == 128) launch_select_nb<128>(s, c, sa, dbg, p.shared, st);
    else launch_select_nb<256>(s, c, sa, dbg, p.shared, st);
    HHR_CHECK();
  }
  AttnArgs aa{idx, cnt, part, p.kcap, p.istride, p.nsplit, p.shared,
              p.scale * 1.4426950408889634f};
  dim3 grid(p.nsplit, s.Hq, s.B);
  if (p.shared && s.kv_bf16) {
    e = launch_attn_gather(s, c, q, p.scale, idx, cnt, p.istride, part, p.nsplit,
                           kernel_timer(dbg, 3), st);
    if (e != hipSuccess) return e;
  } else if (s.kv_bf16) {
    launch_kernel(attn_kernel<1>, grid, dim3(256), st, kernel_timer(dbg, 3), s, c.K, c.V, q, aa);
  } else {
    launch_kernel(attn_kernel<0>, grid, dim3(256), st, kernel_timer(dbg, 3), s, c.K, c.V, q, aa);
  }
  HHR_CHECK();
  return launch_combine(s, part, p.nsplit, out, c.seq_lens, k_new != nullptr ? 1 : 0,
                        kernel_timer(dbg, 4), st);
#undef HHR_CHECK
}

hipError_t launch_combine(const Shape& s, const float* part, int nsplit, float* out,
                          int32_t* seq_lens, int appended, KernelTimer tm, hipStream_t st) {
  // one batch of 16 partials per group of 128 threads, up to 8 groups
  const dim3 grid(s.B * s.Hq);
  if (nsplit <= 16)
    launch_kernel(combine_kernel<1>, grid, dim3(kD), st, tm, part, nsplit, out, seq_lens, s.Hq,
                  s.Lmax, appended);
  else if (nsplit <= 32)
    launch_kernel(combine_kernel<2>, grid, dim3(2 * kD), st, tm, part, nsplit, out, seq_lens,
                  s.Hq, s.Lmax, appended);
  else if (nsplit <= 64)
    launch_kernel(combine_kernel<4>, grid, dim3(4 * kD), st, tm, part, nsplit, out, seq_lens,
                  s.Hq, s.Lmax, appended);
  else
    launch_kernel(combine_kernel<8>, grid, dim3(8 * kD), st, tm, part, nsplit, out, seq_lens,
                  s.Hq, s.Lmax, appended);
  return hipGetLastError();
}

}  // namespace hhr
