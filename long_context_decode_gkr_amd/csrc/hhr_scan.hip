// Fine stage over every token of the context (the fine-stage-only variant of the stage-wise
// ablation, "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", App. C, Table 8):
// Hamming distances by XOR + popcount (§3.1 Eq. 2) of every key code to the query code, then the
// k_eff tokens of smallest (D, t), reported in ascending position.
//
// With the whole context as candidates one workgroup per head would scan 2 MiB of codes at
// 128K, so the work is spread over slices of 4096 tokens in two kernels (no workgroup waits for
// another inside a launch):
//   hamming_scan_kernel  grid (slices, units, B): the distance of every token of the slice
//                        (the smallest over the group's query codes when the selection is
//                        shared by a KV head's heads), stored as one byte (two for 256-bit
//                        codes), and the slice's histogram of distances;
//   token_select_kernel  grid (slices, units, B): every workgroup sums its unit's histograms,
//                        finds the threshold D* (smallest with #(D <= D*) >= k_eff) and the
//                        counts of the slices before its own, then writes its slice's selected
//                        tokens at their final positions (one block scan per 4096 tokens).
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

constexpr int kScanNT = 256;
constexpr int kScanPer = kScanTok / kScanNT;   // tokens per thread (16)

template <int NB, int SHARED>
__global__ void __launch_bounds__(kScanNT)
hamming_scan_kernel(Shape s, CacheView c, ScanArgs a, DebugView dbg) {
  constexpr int NW = NB / 32;
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  const int sl = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int Hs = SHARED ? s.Hkv : s.Hq;
  const int g = SHARED ? u : u / s.G;
  const int bu = b * Hs + u;
  const int ncodes = SHARED ? s.G : 1;
  const int t = c.seq_lens[b];
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int t0 = sl * kScanTok;
  const int tid = threadIdx.x;

  __shared__ uint32_t s_h[NB + 1];
  __shared__ uint32_t s_qw[SHARED ? 8 : 1][NW];
  for (int i = tid; i <= NB; i += kScanNT) s_h[i] = 0;
  if (tid < ncodes * NW)
    s_qw[tid / NW][tid % NW] = a.qcode[(size_t(b) * s.Hq + (SHARED ? g * s.G : u)) * NW + tid];
  if (dbg.page_ids) {   // every page is a candidate: this slice's pages, in order
    const int P = (L + s.S - 1) / s.S;
    for (int p = t0 / s.S + tid; p < min((t0 + kScanTok) / s.S, P); p += kScanNT)
      dbg.page_ids[size_t(bu) * s.Pmax + p] = p;
    if (sl == 0 && tid == 0 && dbg.page_count) dbg.page_count[bu] = P;
  }
  __syncthreads();
  uint32_t qw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) qw[i] = s_qw[0][i];

  const uint32_t* cb = c.codes + (size_t(b) * s.Hkv + g) * s.Lmax * NW;
  DT* dout = reinterpret_cast<DT*>(a.dist) + size_t(bu) * s.Lmax;
  // token t0 + tid + 256 j, in batches whose code loads are all issued before any use
  constexpr int JB = NB == 128 ? 16 : 8;
  for (int j0 = 0; j0 < kScanPer; j0 += JB) {
    uint4 cw[JB][NW / 4];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int tk = min(t0 + tid + kScanNT * (j0 + j), max(L - 1, 0));
      const uint4* cp = reinterpret_cast<const uint4*>(cb + size_t(tk) * NW);
#pragma unroll
      for (int v = 0; v < NW / 4; ++v) cw[j][v] = cp[v];
    }
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int tk = t0 + tid + kScanNT * (j0 + j);
      uint32_t dd = 0;
#pragma unroll
      for (int v = 0; v < NW / 4; ++v)
        dd += __popc(cw[j][v].x ^ qw[4 * v]) + __popc(cw[j][v].y ^ qw[4 * v + 1]) +
              __popc(cw[j][v].z ^ qw[4 * v + 2]) + __popc(cw[j][v].w ^ qw[4 * v + 3]);
      if constexpr (SHARED) {
        for (int i = 1; i < ncodes; ++i) {   // uniform
          uint32_t di = 0;
#pragma unroll
          for (int v = 0; v < NW / 4; ++v)
            di += __popc(cw[j][v].x ^ s_qw[i][4 * v]) + __popc(cw[j][v].y ^ s_qw[i][4 * v + 1]) +
                  __popc(cw[j][v].z ^ s_qw[i][4 * v + 2]) + __popc(cw[j][v].w ^ s_qw[i][4 * v + 3]);
          dd = min(dd, di);
        }
      }
      if (tk < L) {
        atomicAdd(&s_h[dd], 1u);
        dout[tk] = DT(dd);
        if (dbg.dist) dbg.dist[size_t(bu) * s.Lmax + tk] = uint16_t(dd);
      } else if (dbg.dist && tk < (L + s.S - 1) / s.S * s.S) {
        dbg.dist[size_t(bu) * s.Lmax + tk] = 0xFFFFu;   // a slot of the last page past the end
      }
    }
  }
  __syncthreads();
  int32_t* hg = a.hist + (size_t(bu) * a.nsl + sl) * (NB + 1);
  for (int i = tid; i <= NB; i += kScanNT) hg[i] = int32_t(s_h[i]);
}

template <int NB>
__global__ void __launch_bounds__(kScanNT)
token_select_kernel(Shape s, CacheView c, ScanArgs a, DebugView dbg) {
  using DT = typename std::conditional<NB == 128, uint8_t, uint16_t>::type;
  constexpr int kWaves = kScanNT / kWave;
  const int sl = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
  const int Hs = a.shared ? s.Hkv : s.Hq;
  const int bu = b * Hs + u;
  const int t = c.seq_lens[b];
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int t0 = sl * kScanTok;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();

  __shared__ int s_tot[NB + 1], s_pre[NB + 1];
  __shared__ int s_pick[4];
  __shared__ int s_wt[2][kWaves];
  BlockScan<kWaves> scan{s_wt, 0};

  // totals over the unit's slices, and over the slices before this one, per distance: the
  // nsl x (NB + 1) counts are read 16 per thread at a time (all loads issued, then LDS adds)
  for (int bin = tid; bin <= NB; bin += kScanNT) s_tot[bin] = s_pre[bin] = 0;
  __syncthreads();
  const int32_t* hb = a.hist + size_t(bu) * a.nsl * (NB + 1);
  const int nh = a.nsl * (NB + 1);
  for (int i0 = 0; i0 < nh; i0 += 16 * kScanNT) {
    int v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = hb[min(i0 + r * kScanNT + tid, nh - 1)];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + r * kScanNT + tid;
      if (i < nh && v[r] != 0) {
        const int s2 = i / (NB + 1), bin = i - s2 * (NB + 1);
        atomicAdd(&s_tot[bin], v[r]);
        if (s2 < sl) atomicAdd(&s_pre[bin], v[r]);
      }
    }
  }
  __syncthreads();

  // threshold D* (wave 0): the smallest distance with #(D <= D*) >= k_eff; then where this
  // slice's selections start
  if (w == 0) {
    constexpr int BPL = (NB + 1 + kWave - 1) / kWave;
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
    // (no lane hits when k_eff = 0: an empty context)
    const uint64_t hm = __ballot(fbin >= 0);
    const int src = hm ? int(__builtin_ctzll(hm)) : 0;
    const int dstar = hm ? __builtin_amdgcn_readlane(fbin, src) : 0;
    const int before = hm ? __builtin_amdgcn_readlane(fbefore, src) : 0;
    // earlier slices: #(D < D*) and #(D == D*)
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
      s_pick[2] = k_eff - before;          // how many of the D* ties are taken
      s_pick[3] = lt;
    }
  }
  __syncthreads();
  const int dstar = s_pick[0], k_eff = s_pick[1], need_eq = s_pick[2];
  int run_lt = s_pick[3];
  int run_eq = s_pre[min(dstar, NB)];
  if (sl == 0 && tid == 0) {
    a.cnt[bu] = k_eff;
    if (dbg.token_count) dbg.token_count[bu] = k_eff;
  }
  if (k_eff == 0 || t0 >= L) return;

  // this slice's tokens in order: thread tid owns tokens [t0 + 16 tid, t0 + 16 tid + 16)
  const DT* din = reinterpret_cast<const DT*>(a.dist) + size_t(bu) * s.Lmax;
  int32_t* out = a.idx + size_t(bu) * a.istride;
  int32_t* trash = out + a.kcap + lane;
  int32_t* dbg_idx = dbg.token_idx ? dbg.token_idx + size_t(bu) * a.kcap : nullptr;
  const int tb = t0 + kScanPer * tid;
  // the thread's 16 distances as 16-byte loads (the row holds Lmax entries, Lmax a multiple of
  // 64; entries past the sequence are masked)
  constexpr int kWords = kScanPer * int(sizeof(DT)) / 4;
  uint32_t wv[kWords];
#pragma unroll
  for (int i = 0; i < kWords; i += 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(din + tb) + i);
    wv[i] = x.x; wv[i + 1] = x.y; wv[i + 2] = x.z; wv[i + 3] = x.w;
  }
  constexpr int kPer = 4 / int(sizeof(DT));
  uint32_t dv[kScanPer];
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) {
    const uint32_t d = (wv[e / kPer] >> (8 * sizeof(DT) * (e % kPer))) & (sizeof(DT) == 1 ? 0xFFu : 0xFFFFu);
    dv[e] = tb + e < L ? d : 0xFFFFFFFFu;
  }
  int nlt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) {
    nlt += dv[e] < uint32_t(dstar) ? 1 : 0;
    neq += dv[e] == uint32_t(dstar) ? 1 : 0;
  }
  int tot;
  const int ex = scan.excl((nlt << 16) | neq, &tot);
  int eq_seen = run_eq + (ex & 0xFFFF);
  int pos = run_lt + (ex >> 16) + min(eq_seen, need_eq);
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) {
    const bool is_eq = dv[e] == uint32_t(dstar);
    const bool take = dv[e] < uint32_t(dstar) || (is_eq && eq_seen < need_eq);
    eq_seen += is_eq ? 1 : 0;
    *(take ? out + pos : trash) = tb + e;
    if (dbg_idx && take) dbg_idx[pos] = tb + e;
    pos += take ? 1 : 0;
  }
}

int scan_slices(const Shape& s) { return (s.Lmax + kScanTok - 1) / kScanTok; }

hipError_t launch_scan_select(const Shape& s, const CacheView& c, const ScanArgs& a,
                              const DebugView& dbg, hipStream_t st) {
  const dim3 grid(a.nsl, a.shared ? s.Hkv : s.Hq, s.B);
  if (s.NB == 128) {
    if (a.shared)
      launch_kernel(hamming_scan_kernel<128, 1>, grid, dim3(kScanNT), st, kernel_timer(dbg, 1),
                    s, c, a, dbg);
    else
      launch_kernel(hamming_scan_kernel<128, 0>, grid, dim3(kScanNT), st, kernel_timer(dbg, 1),
                    s, c, a, dbg);
    launch_kernel(token_select_kernel<128>, grid, dim3(kScanNT), st, kernel_timer(dbg, 2), s, c,
                  a, dbg);
  } else {
    if (a.shared)
      launch_kernel(hamming_scan_kernel<256, 1>, grid, dim3(kScanNT), st, kernel_timer(dbg, 1),
                    s, c, a, dbg);
    else
      launch_kernel(hamming_scan_kernel<256, 0>, grid, dim3(kScanNT), st, kernel_timer(dbg, 1),
                    s, c, a, dbg);
    launch_kernel(token_select_kernel<256>, grid, dim3(kScanNT), st, kernel_timer(dbg, 2), s, c,
                  a, dbg);
  }
  return hipGetLastError();
}

}  // namespace hhr
