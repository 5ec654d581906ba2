// HHR decode step: coarse stage, fine stage and sparse attention.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation" (arXiv 2610.01230):
//   §3.3.1 Eq. 4  q~ = q R (row vector), the rotation of the query;
//   §3.3.1 Eq. 3  page bound U = sum_j max(q~_j l_j, q~_j u_j); pages above the threshold stay;
//   §3.1 Eq. 1, §3.3.2 Eq. 10  query code = sign(q W);
//   §3.1 Eq. 2    Hamming distance by XOR + popcount;
//   §3.3.2, §1    the closest candidates are kept and attended to exactly.
//
// Three kernels per step, all on the caller's stream:
//   page_bound_kernel  grid (ceil(Pmax/256), Hkv, B): streams the page extrema once for the G
//                      query heads of a KV head (HBM-bound), computing q~ on the fly.
//   select_kernel      grid (Hq, B), 1024 threads: query code, exact top-n_keep pages by a
//                      range-adapted radix select, Hamming distances of the kept pages' keys,
//                      exact top-k tokens by a histogram select; writes ascending indices.
//   attn_kernel        grid (nsplit, Hq, B): split-K softmax attention over gathered K/V rows;
//                      the last workgroup of each (b, h) merges the partial (m, l, o).
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

constexpr int kMaxPages = 16384;       // = HHR_MAX_PAGES
constexpr int kBoundPages = 256;       // pages per bound workgroup (4 per lane)
constexpr int kBoundThreads = 512;     // 8 waves x 16 channels
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kDistCache = 32768;      // candidate slots whose distance stays in LDS

// ---------------------------------------------------------------------------------------------
// Coarse stage: page bounds (Eq. 3) with the query rotated on the fly (Eq. 4).
// Lane l of wave w covers pages p0 + 4l .. p0 + 4l + 3 and channels 16w .. 16w + 15; the 16
// float4 loads of l and u are issued first, q~ for those channels is computed while they are in
// flight, and the 8 waves' partial sums meet in LDS.
// ---------------------------------------------------------------------------------------------
template <int G>
__global__ void __launch_bounds__(kBoundThreads)
page_bound_kernel(Shape s, const float* __restrict__ pmin, const float* __restrict__ pmax,
                  const int32_t* __restrict__ seq_lens, const void* __restrict__ q,
                  const float* __restrict__ R, float* __restrict__ U, float* __restrict__ dbg_U,
                  float* __restrict__ dbg_qrot) {
  const int b = blockIdx.z, g = blockIdx.y, p0 = blockIdx.x * kBoundPages;
  const int L = min(max(seq_lens[b], 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  if (p0 >= P) return;
  const int w = wave_id(), lane = lane_id();
  const int j0 = w * 16;
  const int pl = p0 + lane * 4;
  const bool live = pl < P;
  const size_t srow = (size_t(b) * s.Hkv + g) * kD + j0;

  float4 lo[16], hi[16];
  if (live) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      lo[jj] = *reinterpret_cast<const float4*>(pmin + (srow + jj) * s.Pmax + pl);
      hi[jj] = *reinterpret_cast<const float4*>(pmax + (srow + jj) * s.Pmax + pl);
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) lo[jj] = hi[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // q~[hh][j0 + (lane & 15)] for hh = (lane >> 4) + 4 r.
  constexpr int QPL = (G + 3) / 4;
  float qt[QPL];
  const float* Rg = R + size_t(g) * kD * kD + j0 + (lane & 15);
#pragma unroll
  for (int r = 0; r < QPL; ++r) {
    const int hh = (lane >> 4) + 4 * r;
    float a = 0.f;
    if (hh < G) {
      const size_t qo = (size_t(b) * s.Hq + g * G + hh) * kD;
#pragma unroll 8
      for (int i = 0; i < kD; ++i) a = fmaf(load_elem(q, qo + i, s.q_bf16), Rg[size_t(i) * kD], a);
      if (dbg_qrot && blockIdx.x == 0) dbg_qrot[qo + j0 + (lane & 15)] = a;
    }
    qt[r] = a;
  }

  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) acc[hh][0] = acc[hh][1] = acc[hh][2] = acc[hh][3] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // max(q l, q u) = q * (q >= 0 ? u : l) since l <= u; q is wave-uniform.
      const float qv = __int_as_float(
          __builtin_amdgcn_readlane(__float_as_int(qt[hh >> 2]), (hh & 3) * 16 + jj));
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
  for (int o = threadIdx.x; o < G * kBoundPages; o += kBoundThreads) {
    const int hh = o / kBoundPages, pp = o % kBoundPages;
    const int p = p0 + pp;
    if (p < P) {
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kBoundThreads / kWave; ++w2)
        sum += reinterpret_cast<const float*>(&red[w2][hh][0])[pp];
      const size_t oi = (size_t(b) * s.Hq + g * G + hh) * s.Pmax + p;
      U[oi] = sum;
      if (dbg_U) dbg_U[oi] = sum;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Block-wide scans for 1024 threads.
// ---------------------------------------------------------------------------------------------
struct ScanScratch {
  int wtot[kSelWaves];
};

// Exclusive prefix sum of v over the block in thread order; *total receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, ScanScratch& sc, int* total) {
  const int lane = lane_id(), w = wave_id();
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) sc.wtot[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int t = sc.wtot[i];
    base += (i < w) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Exclusive prefix count of a flag over the block in thread order.
__device__ __forceinline__ int block_flag_prefix(bool f, ScanScratch& sc, int* total) {
  const uint64_t m = __ballot(f);
  const int w = wave_id();
  if (lane_id() == 0) sc.wtot[w] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int t = sc.wtot[i];
    base += (i < w) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + int(lanes_below(m));
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, ScanScratch& sc) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, uint32_t(__shfl_xor(int(v), o)));
  if (lane_id() == 0) sc.wtot[wave_id()] = int(v);
  __syncthreads();
  uint32_t r = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) r = min(r, uint32_t(sc.wtot[i]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, ScanScratch& sc) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), o)));
  if (lane_id() == 0) sc.wtot[wave_id()] = int(v);
  __syncthreads();
  uint32_t r = 0u;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) r = max(r, uint32_t(sc.wtot[i]));
  __syncthreads();
  return r;
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
  const float* U;
  int32_t* idx;       // [B][Hq][kcap]
  int32_t* cnt;       // [B][Hq]
  uint32_t* tickets;  // [B][Hq]
  double rho;
  int kcap;
};

// ---------------------------------------------------------------------------------------------
// Selection, one workgroup per (b, h).
//   EPT: pages per thread (contiguous: thread i owns pages [i EPT, i EPT + EPT)).
// ---------------------------------------------------------------------------------------------
constexpr int kRadixBits = 12;
constexpr int kRadixBins = 1 << kRadixBits;

template <int NB, int EPT>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(Shape s, CacheView c, const void* __restrict__ q, const float* __restrict__ W,
              SelectArgs a, DebugView dbg) {
  constexpr int NW = NB / 32;
  const int h = blockIdx.x, b = blockIdx.y, g = h / s.G;
  const int bh = b * s.Hq + h;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int L = min(max(c.seq_lens[b], 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;

  __shared__ int32_t s_pages[kMaxPages];
  __shared__ uint16_t s_dist[kDistCache];
  __shared__ uint32_t s_hist[kRadixBins > kSelWaves * (NB + 1) ? kRadixBins : kSelWaves * (NB + 1)];
  __shared__ float s_q[kD];
  __shared__ uint32_t s_qw[NW];
  __shared__ ScanScratch sc;
  __shared__ int s_pick[2];

  if (L == 0) {
    if (tid == 0) {
      a.cnt[bh] = 0;
      a.tickets[bh] = 0;
      if (dbg.page_count) dbg.page_count[bh] = 0;
      if (dbg.token_count) dbg.token_count[bh] = 0;
    }
    return;
  }
  const int n_keep = min(P, max(1, int(ceil(a.rho * double(P)))));

  // ---- query to LDS, page keys to registers
  if (tid < kD) s_q[tid] = load_elem(q, size_t(bh) * kD + tid, s.q_bf16);
  uint32_t key[EPT];
  const float* Ub = a.U + size_t(bh) * s.Pmax;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int p = tid * EPT + e;
    key[e] = (p < P) ? desc_key(Ub[p]) : 0xFFFFFFFFu;
  }
  __syncthreads();

  // ---- query code (§3.1 Eq. 1): thread cc < NB computes bit cc, certified / exact
  {
    uint32_t bit = 0;
    if (tid < NB) bit = certified_bit(static_cast<const float*>(s_q), W + size_t(g) * kD * NB + tid, NB);
    const uint64_t m = __ballot(bit);
    if (lane == 0 && w < NB / kWave) {
      s_qw[2 * w] = uint32_t(m);
      s_qw[2 * w + 1] = uint32_t(m >> 32);
    }
  }

  // ---- coarse selection: the n_keep smallest keys, ties to the lower page index.
  // Radix select over rel = key - kmin, 12 bits at a time from the top set bit of the range.
  bool sel[EPT];
  {
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (tid * EPT + e < P) {
        lmin = min(lmin, key[e]);
        lmax = max(lmax, key[e]);
      }
    }
    const uint32_t kmin = block_min_u32(lmin, sc);
    const uint32_t kmax = block_max_u32(lmax, sc);
    int need = n_keep;           // still to take among elements matching `prefix`
    uint32_t prefix = 0;         // high bits of rel fixed so far
    int cur_hi = (kmax == kmin) ? -1 : 31 - __clz(int(kmax - kmin));
    int res_lo = 0;              // resolution: elements compare on rel >> res_lo
    if (n_keep < P) {
      while (cur_hi >= 0) {
        const int cur_lo = max(cur_hi - (kRadixBits - 1), 0);
        const int width = cur_hi - cur_lo + 1;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = tid; i < kRadixBins; i += kSelThreads) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          if (tid * EPT + e < P) {
            const uint32_t rel = key[e] - kmin;
            if (uint32_t(uint64_t(rel) >> (cur_hi + 1)) == prefix)
              atomicAdd(&s_hist[(rel >> cur_lo) & dmask], 1u);
          }
        }
        __syncthreads();
        // scan bins: thread i owns bins [4 i, 4 i + 4)
        constexpr int BPT = kRadixBins / kSelThreads;
        uint32_t hb[BPT];
        int loc = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          hb[j] = s_hist[tid * BPT + j];
          loc += int(hb[j]);
        }
        int tot;
        int run = block_excl_scan(loc, sc, &tot);
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          const int cnt = int(hb[j]);
          if (cnt > 0 && run < need && need <= run + cnt) {
            s_pick[0] = tid * BPT + j;
            s_pick[1] = run;
          }
          run += cnt;
        }
        __syncthreads();
        const int d = s_pick[0], before = s_pick[1];
        const int in_bin = int(s_hist[d]);
        __syncthreads();
        prefix = (prefix << width) | uint32_t(d);
        need -= before;
        res_lo = cur_lo;
        cur_hi = cur_lo - 1;
        if (in_bin == need) break;   // the whole bin is taken: no finer digit is needed
      }
    }
    // Final: rel >> res_lo below prefix -> taken; equal -> taken in index order up to `need`.
    bool lt[EPT], eq[EPT];
    int neq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool ok = tid * EPT + e < P;
      const uint32_t v = (key[e] - kmin) >> res_lo;
      lt[e] = ok && (n_keep < P) && v < prefix;
      eq[e] = ok && ((n_keep >= P) || v == prefix);
      neq += eq[e] ? 1 : 0;
    }
    if (n_keep >= P) need = P;
    int tot;
    int rank = block_excl_scan(neq, sc, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      sel[e] = lt[e] || (eq[e] && rank < need);
      rank += eq[e] ? 1 : 0;
    }
  }
  // compaction: kept pages in ascending order
  {
    int nsel = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) nsel += sel[e] ? 1 : 0;
    int tot;
    int pos = block_excl_scan(nsel, sc, &tot);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (sel[e]) {
        s_pages[pos] = tid * EPT + e;
        if (dbg.page_ids) dbg.page_ids[size_t(bh) * s.Pmax + pos] = tid * EPT + e;
        ++pos;
      }
    }
    if (tid == 0 && dbg.page_count) dbg.page_count[bh] = n_keep;
  }
  if (dbg.q_code && tid < NW) dbg.q_code[size_t(bh) * NW + tid] = s_qw[tid];
  for (int i = tid; i < kSelWaves * (NB + 1); i += kSelThreads) s_hist[i] = 0;
  __syncthreads();

  // ---- fine stage: Hamming distance of every candidate slot (§3.1 Eq. 2)
  uint32_t qw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) qw[i] = s_qw[i];
  const int lgS = (s.S == 16) ? 4 : 5;
  const int nslots = n_keep << lgS;
  const bool cache_d = nslots <= kDistCache;
  const uint32_t* cbase = c.codes + (size_t(b) * s.Hkv + g) * s.Lmax * NW;
  auto distance = [&](int slot, int* t_out) -> int {
    const int t = (s_pages[slot >> lgS] << lgS) + (slot & (s.S - 1));
    *t_out = t;
    if (t >= L) return 0xFFFF;
    const uint4* cp = reinterpret_cast<const uint4*>(cbase + size_t(t) * NW);
    int dd = 0;
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) {
      const uint4 x = cp[v];
      dd += __popc(x.x ^ qw[4 * v]) + __popc(x.y ^ qw[4 * v + 1]) + __popc(x.z ^ qw[4 * v + 2]) +
            __popc(x.w ^ qw[4 * v + 3]);
    }
    return dd;
  };
  uint32_t* whist = s_hist + w * (NB + 1);
  for (int slot = tid; slot < nslots; slot += kSelThreads) {
    int t;
    const int dd = distance(slot, &t);
    if (dd != 0xFFFF) atomicAdd(&whist[dd], 1u);
    if (cache_d) s_dist[slot] = uint16_t(dd);
    if (dbg.dist) dbg.dist[size_t(bh) * s.Lmax + slot] = uint16_t(dd);
  }
  __syncthreads();

  // ---- token threshold: smallest D* with #(D <= D*) >= k_eff
  int dstar, before, k_eff;
  {
    int tot_d = 0;
    if (tid <= NB) {
#pragma unroll 4
      for (int i = 0; i < kSelWaves; ++i) tot_d += int(s_hist[i * (NB + 1) + tid]);
    }
    int C;
    const int run = block_excl_scan(tot_d, sc, &C);
    k_eff = min(a.kcap, C);
    if (tot_d > 0 && run < k_eff && k_eff <= run + tot_d) {
      s_pick[0] = tid;
      s_pick[1] = run;
    }
    __syncthreads();
    dstar = s_pick[0];
    before = s_pick[1];
  }
  const int need_eq = k_eff - before;

  // ---- emit the selected tokens in ascending position (slots are in ascending t)
  int32_t* out_idx = a.idx + size_t(bh) * a.kcap;
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < nslots; base += kSelThreads) {
    const int slot = base + tid;
    int t = 0, dd = 0xFFFF;
    if (slot < nslots) {
      if (cache_d) {
        dd = s_dist[slot];
        t = (s_pages[slot >> lgS] << lgS) + (slot & (s.S - 1));
      } else {
        dd = distance(slot, &t);
      }
    }
    const bool is_eq = dd == dstar;
    const bool is_lt = dd < dstar;
    int eq_tot;
    const int eq_rank = run_eq + block_flag_prefix(is_eq, sc, &eq_tot);
    const bool take = is_lt || (is_eq && eq_rank < need_eq);
    int sel_tot;
    const int pos = run_sel + block_flag_prefix(take, sc, &sel_tot);
    if (take) {
      out_idx[pos] = t;
      if (dbg.token_idx) dbg.token_idx[size_t(bh) * a.kcap + pos] = t;
    }
    run_eq += eq_tot;
    run_sel += sel_tot;
  }
  if (tid == 0) {
    a.cnt[bh] = k_eff;
    a.tickets[bh] = 0;
    if (dbg.token_count) dbg.token_count[bh] = k_eff;
  }
}

// ---------------------------------------------------------------------------------------------
// Sparse attention over the selected rows: split-K with an in-kernel merge.
// A row of d = 128 is read as 16-byte pieces: 16 lanes per row for bf16, 32 for fp32. Every
// wave issues all its K and V loads up front, then computes logits, the workgroup maximum, the
// exponentials and the weighted V sum. The workgroup writes (o, m, l) for its chunk; the last
// workgroup of (b, h) to finish (ticket) merges them into the output.
// ---------------------------------------------------------------------------------------------
template <int BF16>
struct AttnShape {
  static constexpr int EPL = BF16 ? 8 : 4;        // elements per lane per row
  static constexpr int LPR = kD / EPL;            // lanes per row
  static constexpr int RPI = kWave / LPR;         // rows per wave-wide load
  static constexpr int ITER = 16;                 // loads per lane for K (and for V)
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
  const int32_t* idx;
  const int32_t* cnt;
  float* part;        // [B][Hq][nsplit][kD + 2]
  uint32_t* tickets;  // [B][Hq]
  int kcap, nsplit;
  float scale_log2e;
};

template <int BF16>
__global__ void __launch_bounds__(256)
attn_kernel(Shape s, const void* __restrict__ K, const void* __restrict__ V,
            const void* __restrict__ q, AttnArgs a, float* __restrict__ out) {
  using A = AttnShape<BF16>;
  constexpr int EPL = A::EPL, LPR = A::LPR, RPI = A::RPI, ITER = A::ITER;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / s.G;
  const int bh = b * s.Hq + h;
  const int count = a.cnt[bh];
  const int w = wave_id(), lane = lane_id();
  const int rg = lane / LPR, sub = lane % LPR;
  const int row0 = split * A::CHUNK + w * A::RPW;
  const size_t esz = BF16 ? 2 : 4;

  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    qv[e] = load_elem(q, size_t(bh) * kD + sub * EPL + e, s.q_bf16) * a.scale_log2e;

  const size_t kvrow0 = (size_t(b) * s.Hkv + g) * s.Lmax;
  const int32_t* ib = a.idx + size_t(bh) * a.kcap;
  int tok[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int r = row0 + it * RPI + rg;
    // indices come from select_kernel and are < seq_len; the clamp only keeps any reader in
    // bounds of the cache
    tok[it] = (r < count) ? min(max(ib[r], 0), s.Lmax - 1) : -1;
  }
  uint4 kr[ITER], vr[ITER];
  const char* Kc = static_cast<const char*>(K);
  const char* Vc = static_cast<const char*>(V);
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    if (tok[it] >= 0) {
      const size_t off = ((kvrow0 + size_t(tok[it])) * kD + sub * EPL) * esz;
      kr[it] = *reinterpret_cast<const uint4*>(Kc + off);
      vr[it] = *reinterpret_cast<const uint4*>(Vc + off);
    } else {
      kr[it] = vr[it] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

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
    for (int o = LPR / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o);
    sc[it] = (tok[it] >= 0) ? d : -INFINITY;
    mx = fmaxf(mx, sc[it]);
  }
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_o[4][kD];
  __shared__ int s_last;
  mx = wave_max(mx);
  if (lane == 0) s_m[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));

  float l = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const float p = (tok[it] >= 0) ? exp2f(sc[it] - M) : 0.f;
      l += p;
      float f[EPL];
      unpack(vr[it], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, f[e], o[e]);
    }
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
  float* pp = a.part + (size_t(bh) * a.nsplit + split) * (kD + 2);
  if (threadIdx.x < kD) {
    const int d = threadIdx.x;
    pp[d] = s_o[0][d] + s_o[1][d] + s_o[2][d] + s_o[3][d];
  }
  if (threadIdx.x == 0) {
    pp[kD] = M;
    pp[kD + 1] = s_l[0] + s_l[1] + s_l[2] + s_l[3];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&a.tickets[bh], 1u) == uint32_t(a.nsplit - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x < kD) {
    const int d = threadIdx.x;
    const float* pb = a.part + size_t(bh) * a.nsplit * (kD + 2);
    float Mx = -INFINITY;
    for (int i = 0; i < a.nsplit; ++i) Mx = fmaxf(Mx, pb[i * (kD + 2) + kD]);
    float Ls = 0.f, Os = 0.f;
    if (Mx != -INFINITY) {
      for (int i = 0; i < a.nsplit; ++i) {
        const float* pi = pb + i * (kD + 2);
        const float li = pi[kD + 1];
        if (li > 0.f) {
          const float f = exp2f(pi[kD] - Mx);
          Ls = fmaf(li, f, Ls);
          Os = fmaf(pi[d], f, Os);
        }
      }
    }
    out[size_t(bh) * kD + d] = (Ls > 0.f) ? Os / Ls : 0.f;
  }
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

DecodePlan plan_decode(const Shape& s, double rho, int k, float scale) {
  DecodePlan p{};
  p.kcap = k < s.Lmax ? k : s.Lmax;
  p.chunk = s.kv_bf16 ? AttnShape<1>::CHUNK : AttnShape<0>::CHUNK;
  p.nsplit = (p.kcap + p.chunk - 1) / p.chunk;
  p.rho = rho;
  p.scale = scale;
  const size_t BH = size_t(s.B) * s.Hq;
  size_t off = 0;
  p.off_U = off;      off = align256(off + BH * s.Pmax * sizeof(float));
  p.off_idx = off;    off = align256(off + BH * p.kcap * sizeof(int32_t));
  p.off_cnt = off;    off = align256(off + BH * sizeof(int32_t));
  p.off_ticket = off; off = align256(off + BH * sizeof(uint32_t));
  p.off_part = off;   off = align256(off + BH * p.nsplit * (kD + 2) * sizeof(float));
  p.total = off;
  return p;
}

template <int G>
static void launch_bound_t(const Shape& s, const CacheView& c, const void* q, const float* R,
                           float* U, const DebugView& dbg, hipStream_t st) {
  dim3 grid((s.Pmax + kBoundPages - 1) / kBoundPages, s.Hkv, s.B);
  hipLaunchKernelGGL((page_bound_kernel<G>), grid, dim3(kBoundThreads), 0, st, s, c.pmin, c.pmax,
                     c.seq_lens, q, R, U, dbg.bounds, dbg.q_rot);
}

template <int NB, int EPT>
static void launch_select_t(const Shape& s, const CacheView& c, const void* q, const float* W,
                            const SelectArgs& a, const DebugView& dbg, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<NB, EPT>), dim3(s.Hq, s.B), dim3(kSelThreads), 0, st, s, c,
                     q, W, a, dbg);
}

template <int NB>
static void launch_select_nb(const Shape& s, const CacheView& c, const void* q, const float* W,
                             const SelectArgs& a, const DebugView& dbg, hipStream_t st) {
  const int ept = (s.Pmax + kSelThreads - 1) / kSelThreads;
  if (ept <= 1) launch_select_t<NB, 1>(s, c, q, W, a, dbg, st);
  else if (ept <= 2) launch_select_t<NB, 2>(s, c, q, W, a, dbg, st);
  else if (ept <= 4) launch_select_t<NB, 4>(s, c, q, W, a, dbg, st);
  else if (ept <= 8) launch_select_t<NB, 8>(s, c, q, W, a, dbg, st);
  else launch_select_t<NB, 16>(s, c, q, W, a, dbg, st);
}

hipError_t launch_decode(const Shape& s, const DecodePlan& p, const CacheView& c, const void* q,
                         const float* R, const float* W, void* ws, float* out,
                         const DebugView& dbg, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  float* U = reinterpret_cast<float*>(base + p.off_U);
  int32_t* idx = reinterpret_cast<int32_t*>(base + p.off_idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + p.off_cnt);
  uint32_t* tick = reinterpret_cast<uint32_t*>(base + p.off_ticket);
  float* part = reinterpret_cast<float*>(base + p.off_part);

  hipError_t e = hipSuccess;
  if (dbg.events && (e = hipEventRecord(dbg.events[0], st)) != hipSuccess) return e;
  switch (s.G) {
    case 1: launch_bound_t<1>(s, c, q, R, U, dbg, st); break;
    case 2: launch_bound_t<2>(s, c, q, R, U, dbg, st); break;
    case 4: launch_bound_t<4>(s, c, q, R, U, dbg, st); break;
    default: launch_bound_t<8>(s, c, q, R, U, dbg, st); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dbg.events && (e = hipEventRecord(dbg.events[1], st)) != hipSuccess) return e;

  SelectArgs sa{U, idx, cnt, tick, p.rho, p.kcap};
  if (s.NB == 128) launch_select_nb<128>(s, c, q, W, sa, dbg, st);
  else launch_select_nb<256>(s, c, q, W, sa, dbg, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dbg.events && (e = hipEventRecord(dbg.events[2], st)) != hipSuccess) return e;

  AttnArgs aa{idx, cnt, part, tick, p.kcap, p.nsplit, p.scale * 1.4426950408889634f};
  dim3 grid(p.nsplit, s.Hq, s.B);
  if (s.kv_bf16)
    hipLaunchKernelGGL((attn_kernel<1>), grid, dim3(256), 0, st, s, c.K, c.V, q, aa, out);
  else
    hipLaunchKernelGGL((attn_kernel<0>), grid, dim3(256), 0, st, s, c.K, c.V, q, aa, out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dbg.events) e = hipEventRecord(dbg.events[3], st);
  return e;
}

}  // namespace hhr
