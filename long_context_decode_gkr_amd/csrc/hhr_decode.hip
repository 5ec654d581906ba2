// HHR decode step: coarse stage, fine stage and sparse attention.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation" (arXiv 2610.01230):
//   §3.3.1 Eq. 4  q~ = q R (row vector), the rotation of the query;
//   §3.3.1 Eq. 3  page bound U = sum_j max(q~_j l_j, q~_j u_j); pages above the threshold stay;
//   §3.1 Eq. 1, §3.3.2 Eq. 10  query code = sign(q W);
//   §3.1 Eq. 2    Hamming distance by XOR + popcount;
//   §3.3.2, §1    the closest candidates are kept and attended to exactly.
//
// Kernels of a step, all on the caller's stream (after the preparation kernel of hhr_build.hip,
// which appends the new token and writes q~ and the query codes; the selection between the
// bound and the attention is in hhr_select.hip):
//   page_bound_kernel  grid (ceil(Pmax/PB), Hkv, B), PB = 64, 128 or 256 pages: streams the
//                      page extrema once for the G query heads of a KV head (HBM-bound).
//   attn_kernel        grid (nsplit, Hq, B): split-K softmax attention over gathered K/V rows,
//                      one partial (m, l, o) per workgroup;
//   combine_kernel     grid (B * Hq): merges the partials of each (b, h) into the output and
//                      advances seq_lens when the step appended a token.
// The merge is a kernel of its own: an in-kernel "last workgroup merges" scheme needs a
// device-scope release and acquire in every workgroup, which on gfx950 write back and
// invalidate the whole L2 of an XCD, and costs far more than one small launch.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

constexpr int kBoundThreads = 512;     // 8 waves x 16 channels

// ---------------------------------------------------------------------------------------------
// Coarse stage: page bounds (Eq. 3) for the G query heads of one KV head from ONE read of the
// page extrema. A workgroup covers PB = 64 PPL pages: lane l of wave w covers pages
// p0 + PPL l .. + PPL - 1 and channels 16w .. 16w + 15, i.e. 32 loads of PPL consecutive extrema
// per lane, all issued at once; q~ (prepared by the preparation kernel) is read with
// wave-uniform loads, and the 8 waves' partial sums meet in LDS. PPL (4, 2 or 1) is the largest
// whose grid still gives every CU a workgroup, so that a short context's extrema are streamed
// by the whole chip; a page's bound is the same sequence of operations for every PPL (a chain of
// 16 fused multiply-adds per wave in channel order, then the 8 waves' sums in wave order), so
// the bounds do not depend on it.
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
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// PPL consecutive stored extrema (element i of the fp32 or bf16 array) as fp32, with one
// non-temporal load (the extrema are read once per step: 14.6 -> 13.8 us at 128K).
template <int PPL, int SB>
__device__ __forceinline__ void load_pages_nt(const void* base, size_t i, float (&v)[PPL]) {
  if constexpr (SB) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + i;
    if constexpr (PPL == 4) {
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
      v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
    } else if constexpr (PPL == 2) {
      const uint32_t x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
      v[0] = __uint_as_float(x << 16); v[1] = __uint_as_float(x & 0xFFFF0000u);
    } else {
      v[0] = __uint_as_float(uint32_t(__builtin_nontemporal_load(p)) << 16);
    }
  } else {
    const float* p = static_cast<const float*>(base) + i;
    if constexpr (PPL == 4) {
      const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (PPL == 2) {
      const f32x2v x = __builtin_nontemporal_load(reinterpret_cast<const f32x2v*>(p));
      v[0] = x.x; v[1] = x.y;
    } else {
      v[0] = __builtin_nontemporal_load(p);
    }
  }
}

template <int G, int SB, int PPL>   // SB: extrema stored as bf16; PPL: pages per lane
__global__ void __launch_bounds__(kBoundThreads)
page_bound_kernel(Shape s, CacheView c, BoundArgs a, float* __restrict__ dbg_U) {
  constexpr int PB = kWave * PPL;                  // pages per workgroup
  const int F = xcd_flat(linear_block_id(), grid_blocks());
  const int x = F % int(gridDim.x), g = (F / int(gridDim.x)) % s.Hkv;
  const int b = F / (int(gridDim.x) * s.Hkv), p0 = x * PB;
  const int t = c.seq_lens[b];
  const bool app = a.appended && t >= 0 && t < s.Lmax;
  const int L = min(max(t, 0) + (app ? 1 : 0), s.Lmax);
  const int P = (L + s.S - 1) / s.S;
  if (p0 >= P) return;
  const int w = wave_id(), lane = lane_id();
  const int j0 = w * 16;
  const int plc = min(p0 + lane * PPL, s.Pmax - PPL);   // in bounds for every lane
  const size_t srow = (size_t(b) * s.Hkv + g) * kD + j0;

  float lo[16][PPL], hi[16][PPL];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    load_pages_nt<PPL, SB>(c.pmin, (srow + jj) * s.Pmax + plc, lo[jj]);
    load_pages_nt<PPL, SB>(c.pmax, (srow + jj) * s.Pmax + plc, hi[jj]);
  }
  const float* qb = a.qrot + (size_t(b) * s.Hq + size_t(g) * G) * kD + j0;

  float acc[G][PPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int k = 0; k < PPL; ++k) acc[hh][k] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // max(q l, q u) = q * (q >= 0 ? u : l) since l <= u; q is wave-uniform.
      const float qv = qb[hh * kD + jj];
#pragma unroll
      for (int k = 0; k < PPL; ++k)
        acc[hh][k] = fmaf(qv, (qv >= 0.f) ? hi[jj][k] : lo[jj][k], acc[hh][k]);
    }
  }

  __shared__ __align__(16) float red[kBoundThreads / kWave][G][PB];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float* r = &red[w][hh][lane * PPL];
    if constexpr (PPL == 4) {
      *reinterpret_cast<float4*>(r) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
    } else if constexpr (PPL == 2) {
      *reinterpret_cast<float2*>(r) = make_float2(acc[hh][0], acc[hh][1]);
    } else {
      r[0] = acc[hh][0];
    }
  }
  __syncthreads();
  if (a.shared) {
    // one bound per page for the whole group: the largest of its heads' bounds (the group's
    // pages are chosen once; each head's own bound goes to the debug output only)
    for (int pp = threadIdx.x; pp < PB; pp += kBoundThreads) {
      const int p = p0 + pp;
      if (p < P) {
        float um = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float sum = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kBoundThreads / kWave; ++w2) sum += red[w2][hh][pp];
          um = fmaxf(um, sum);
          if (dbg_U) dbg_U[(size_t(b) * s.Hq + g * G + hh) * s.Pmax + p] = sum;
        }
        a.U[(size_t(b) * s.Hkv + g) * s.Pmax + p] = um;
      }
    }
    return;
  }
  for (int o = threadIdx.x; o < G * PB; o += kBoundThreads) {
    const int hh = o / PB, pp = o % PB;
    const int p = p0 + pp;
    if (p < P) {
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kBoundThreads / kWave; ++w2) sum += red[w2][hh][pp];
      const size_t oi = (size_t(b) * s.Hq + g * G + hh) * s.Pmax + p;
      a.U[oi] = sum;
      if (dbg_U) dbg_U[oi] = sum;
    }
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
    // query slice: raw bits now (16 bytes per lane), unpacked and scaled into the log2 domain
    // only after the row loads are issued, so that nothing waits for it before them
    const size_t qo = size_t(bh) * kD + sub * EPL;
    uint4 qraw[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    if (s.q_bf16) {
      const uint16_t* qb = static_cast<const uint16_t*>(q) + qo;
      if constexpr (EPL == 8) {
        qraw[0] = *reinterpret_cast<const uint4*>(qb);
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(qb);
        qraw[0].x = x.x; qraw[0].y = x.y;
      }
    } else {
      const float* qf = static_cast<const float*>(q) + qo;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) qraw[e / 4] = *reinterpret_cast<const uint4*>(qf + e);
    }

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

    float qv[EPL];
    if (s.q_bf16) {
      if constexpr (EPL == 8) {
        float f[8];
        unpack(qraw[0], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = f[e];
      } else {
        qv[0] = __uint_as_float(qraw[0].x << 16); qv[1] = __uint_as_float(qraw[0].x & 0xFFFF0000u);
        qv[2] = __uint_as_float(qraw[0].y << 16); qv[3] = __uint_as_float(qraw[0].y & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        float f[4];
        unpack(qraw[e / 4], f);
        qv[e] = f[0]; qv[e + 1] = f[1]; qv[e + 2] = f[2]; qv[e + 3] = f[3];
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= a.scale_log2e;

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
      d = row16_sum(d);                         // the row's LPR lanes: 16, or 32 for fp32
      if constexpr (LPR == 32) d += lane_xor(d, 16);
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
    // reduce across the row groups of the wave (lanes that share `sub`) into row group 0, the
    // lanes that store the result
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
      l += lane_from_above(l, off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] += lane_from_above(o[e], off);
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
  if (stages == Stages::kCodesOnly) rho = 1.0;   // every page is a candidate
  // most kept pages of any sequence (n_keep grows with the page count)
  const long long keep = (long long)ceil(rho * double(s.Pmax));
  p.kpages = int(keep < 1 ? 1 : (keep < s.Pmax ? keep : s.Pmax));
  if (stages == Stages::kPagesOnly) {
    // every token of the kept pages
    const long long toks = (long long)p.kpages * s.S;
    p.kcap = toks < s.Lmax ? int(toks) : s.Lmax;
  } else {
    p.kcap = k < s.Lmax ? k : s.Lmax;
  }
  // (group-shared bf16: the gathered matrix-core attention, kGatherChunk positions per
  // workgroup; otherwise the per-head kernel)
  p.chunk = shared && s.kv_bf16 ? kGatherChunk
                                : (s.kv_bf16 ? AttnShape<1>::CHUNK : AttnShape<0>::CHUNK);
  p.nsplit = (p.kcap + p.chunk - 1) / p.chunk;
  p.rho = rho;
  p.scale = scale;
  const size_t BH = size_t(s.B) * s.Hq;
  const size_t NU = size_t(s.B) * (shared ? s.Hkv : s.Hq);   // selection units
  // The selection form: one workgroup per unit when the candidates fit its LDS cache; the
  // sliced form otherwise (always for the fine stage alone). HHR_SELECT=sliced forces the sliced
  // form and HHR_SELECT_SLICES=n its slice count (1..1024): another decomposition of the same
  // selection, for checking that both give identical results.
  const char* force = getenv("HHR_SELECT");
  p.unit_select = stages != Stages::kCodesOnly && p.kpages * s.S <= kUnitSlots &&
                  !(force && strcmp(force, "sliced") == 0);
  // The one-workgroup form's size: 512 threads while they hold the pages 4 per thread, else
  // 1024 (fewer waves meet at each of its barriers: 9.2 -> 8.0 us at 32K, 9.1 -> 7.6 us at 16K,
  // where 256 threads measured no better; at 128K 1024 threads take 11.4 us against 13.2 with
  // 512 threads of 16 pages each). HHR_SELECT_THREADS=256, 512 or 1024 forces one (the smaller
  // ones only where the pages fit 16 per thread).
  p.unit_threads = s.Pmax <= 4 * 512 ? 512 : 1024;
  if (const char* nthr = getenv("HHR_SELECT_THREADS")) {
    const int n = atoi(nthr);
    if (n == 256 || n == 512 || n == 1024) p.unit_threads = n;
  }
  p.nsl = select_slices(p.kpages, int(NU), stages == Stages::kCodesOnly);
  if (const char* ns = getenv("HHR_SELECT_SLICES")) {
    const int n = atoi(ns);
    if (n >= 1 && n <= 1024 && (p.kpages + n - 1) / n <= kSlicePages) p.nsl = n;
  }
  p.dstride = (p.kpages * s.S + 15) & ~15;
  size_t off = 0;
  p.off_qrot = off;   off = align256(off + BH * kD * sizeof(float));
  p.off_qcode = off;  off = align256(off + BH * s.NW * sizeof(uint32_t));
  p.off_U = off;      off = align256(off + NU * s.Pmax * sizeof(float));
  p.istride = ((p.kcap + 3) & ~3) + kWave;   // 16-byte aligned rows, then the trash entries
  p.off_idx = off;    off = align256(off + NU * p.istride * sizeof(int32_t));
  p.off_cnt = off;    off = align256(off + NU * sizeof(int32_t));
  p.off_part = off;   off = align256(off + BH * p.nsplit * (kD + 2) * sizeof(float));
  p.off_pages = off;  off = align256(off + NU * p.kpages * sizeof(int32_t));
  p.off_dist = off;   off = align256(off + NU * p.dstride * (s.NB == 128 ? 1 : 2));
  p.off_hist = off;   off = align256(off + NU * p.nsl * (s.NB + 1) * sizeof(int32_t));
  p.total = off;
  return p;
}

template <int G, int SB, int PPL>
static hipError_t launch_bound_p(const Shape& s, const CacheView& c, const BoundArgs& a,
                                 const DebugView& dbg, hipStream_t st) {
  const dim3 grid((s.Pmax + kWave * PPL - 1) / (kWave * PPL), s.Hkv, s.B);
  return launch_kernel("page_bound_kernel", page_bound_kernel<G, SB, PPL>, grid,
                       dim3(kBoundThreads), st, kernel_timer(dbg, 1), s, c, a, dbg.bounds);
}

template <int G>
static hipError_t launch_bound_t(const Shape& s, const CacheView& c, const BoundArgs& a,
                                 int ppl, const DebugView& dbg, hipStream_t st) {
  if (s.sum_bf16) {
    if (ppl == 4) return launch_bound_p<G, 1, 4>(s, c, a, dbg, st);
    if (ppl == 2) return launch_bound_p<G, 1, 2>(s, c, a, dbg, st);
    return launch_bound_p<G, 1, 1>(s, c, a, dbg, st);
  }
  if (ppl == 4) return launch_bound_p<G, 0, 4>(s, c, a, dbg, st);
  if (ppl == 2) return launch_bound_p<G, 0, 2>(s, c, a, dbg, st);
  return launch_bound_p<G, 0, 1>(s, c, a, dbg, st);
}

// Compute units of the current device (queried once per device; 256 if the query fails).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Pages per lane of the bound kernel: the largest of 4, 2, 1 whose grid still gives every
// compute unit a workgroup (at batch 1: 4 from 128K, 2 at 64K, 1 at 32K and below).
// HHR_BOUND_PAGES=256, 128 or 64 forces the workgroup's page count (the bounds are identical
// for every choice).
static int bound_pages_per_lane(const Shape& s) {
  if (const char* e = getenv("HHR_BOUND_PAGES")) {
    const int n = atoi(e);
    if (n == 256 || n == 128 || n == 64) return n / kWave;
  }
  const int cus = device_cus();
  for (int ppl = 4; ppl > 1; ppl >>= 1) {
    const long long blocks =
        (long long)((s.Pmax + kWave * ppl - 1) / (kWave * ppl)) * s.Hkv * s.B;
    if (blocks >= cus) return ppl;
  }
  return 1;
}

// Both events of a kernel slot that has no launch of its own in this step, back to back.
static hipError_t record_empty_slot(const DebugView& dbg, int k, hipStream_t st) {
  const KernelTimer tm = kernel_timer(dbg, k);
  if (!tm.start) return hipSuccess;
  const hipError_t e = hipEventRecord(tm.start, st);
  return e != hipSuccess ? e : hipEventRecord(tm.stop, st);
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
  const int appended = k_new != nullptr ? 1 : 0;
  hipError_t e;
  if (trace_on()) {
    // sizes for full sequences (seq_lens is in device memory): what each kernel reads at most
    const double esz = s.kv_bf16 ? 2.0 : 4.0, xsz = s.sum_bf16 ? 2.0 : 4.0;
    const double NU = double(s.B) * (p.shared ? s.Hkv : s.Hq);
    trace_printf("decode B %d Hq %d Hkv %d S %d NB %d Lmax %d stages %d shared %d append %d: "
                 "kpages %d kcap %d, %d pages per bound workgroup, selection %s (%d threads; "
                 "%d slices), %d attention splits, workspace %zu B", s.B, s.Hq, s.Hkv, s.S, s.NB,
                 s.Lmax, int(p.stages), p.shared, appended, p.kpages, p.kcap,
                 kWave * bound_pages_per_lane(s),
                 p.unit_select ? "one workgroup per unit" : "sliced", p.unit_threads, p.nsl,
                 p.nsplit, p.total);
    trace_printf("bytes at most: prep %.0f (R, W, q), page_bound %.0f (extrema) + %.0f (U), "
                 "select %.0f (U, candidate codes), attention %.0f (K, V rows)",
                 double(s.Hkv) * 128 * (128 + s.NB) * 4 + double(s.B) * s.Hq * 128 * esz,
                 double(s.B) * s.Hkv * 128 * s.Pmax * 2 * xsz, NU * s.Pmax * 4,
                 NU * (s.Pmax * 4.0 + double(p.kpages) * s.S * s.NB / 8),
                 NU * double(p.kcap) * 2 * 128 * esz);
  }

  // seq_lens[b] stays t during the step; every kernel works on t + 1 tokens when a token is
  // appended, and the last kernel stores t + 1.
  e = launch_prep(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg.q_rot, dbg.q_code,
                  PrepMode::kDecode, kernel_timer(dbg, 0), st);
  if (e != hipSuccess) return e;
  if (p.stages == Stages::kCodesOnly) {
    // every page is kept: no bound is needed (its slot's events are recorded back to back)
    if ((e = record_empty_slot(dbg, 1, st)) != hipSuccess) return e;
  } else {
    BoundArgs ba{qrot, U, appended, p.shared};
    const int ppl = bound_pages_per_lane(s);
    switch (s.G) {
      case 1: e = launch_bound_t<1>(s, c, ba, ppl, dbg, st); break;
      case 2: e = launch_bound_t<2>(s, c, ba, ppl, dbg, st); break;
      case 4: e = launch_bound_t<4>(s, c, ba, ppl, dbg, st); break;
      default: e = launch_bound_t<8>(s, c, ba, ppl, dbg, st); break;
    }
    if (e != hipSuccess) return e;
  }
  SelectArgs sa{qcode, p.stages == Stages::kCodesOnly ? nullptr : U,
                reinterpret_cast<int32_t*>(base + p.off_pages), base + p.off_dist,
                reinterpret_cast<int32_t*>(base + p.off_hist), idx, cnt, p.rho, p.kcap,
                p.istride, p.nsl, p.kpages, p.dstride, appended,
                p.stages == Stages::kPagesOnly ? 0 : 1, p.shared};
  e = launch_select(s, c, sa, dbg, p.unit_select ? p.unit_threads : 0, st);
  if (e != hipSuccess) return e;
  AttnArgs aa{idx, cnt, part, p.kcap, p.istride, p.nsplit, p.shared,
              p.scale * 1.4426950408889634f};
  dim3 grid(p.nsplit, s.Hq, s.B);
  if (p.shared && s.kv_bf16)
    e = launch_attn_gather(s, c, q, p.scale, idx, cnt, p.istride, part, p.nsplit,
                           kernel_timer(dbg, 4), st);
  else if (s.kv_bf16)
    e = launch_kernel("attn_kernel",
                      attn_kernel<1>, grid, dim3(256), st, kernel_timer(dbg, 4), s, c.K, c.V, q,
                      aa);
  else
    e = launch_kernel("attn_kernel",
                      attn_kernel<0>, grid, dim3(256), st, kernel_timer(dbg, 4), s, c.K, c.V, q,
                      aa);
  if (e != hipSuccess) return e;
  return launch_combine(s, part, p.nsplit, out, c.seq_lens, appended, kernel_timer(dbg, 5), st);
}

hipError_t launch_combine(const Shape& s, const float* part, int nsplit, float* out,
                          int32_t* seq_lens, int appended, KernelTimer tm, hipStream_t st) {
  // one batch of 16 partials per group of 128 threads, up to 8 groups
  const dim3 grid(s.B * s.Hq);
  if (nsplit <= 16)
    return launch_kernel("combine_kernel",
                         combine_kernel<1>, grid, dim3(kD), st, tm, part, nsplit, out, seq_lens,
                         s.Hq, s.Lmax, appended);
  if (nsplit <= 32)
    return launch_kernel("combine_kernel",
                         combine_kernel<2>, grid, dim3(2 * kD), st, tm, part, nsplit, out,
                         seq_lens, s.Hq, s.Lmax, appended);
  if (nsplit <= 64)
    return launch_kernel("combine_kernel",
                         combine_kernel<4>, grid, dim3(4 * kD), st, tm, part, nsplit, out,
                         seq_lens, s.Hq, s.Lmax, appended);
  return launch_kernel("combine_kernel",
                       combine_kernel<8>, grid, dim3(8 * kD), st, tm, part, nsplit, out,
                       seq_lens, s.Hq, s.Lmax, appended);
}

}  // namespace hhr
