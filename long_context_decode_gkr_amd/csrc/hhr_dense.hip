// Dense decode attention over the whole context: the baseline the sparse step is compared with.
//
// "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", §4.3 and Fig. 7 compare the
// decode speed of HHR against full attention over every cached key; this is that full
// attention on the same cache layout, o_h = sum_t softmax_t(scale q_h . k_t) v_t over all
// t < seq_lens[b], fp32 accumulation.
//
// Split-K flash decoding with grouped-query sharing: workgroup (split, g, b) streams the K and V
// rows of tokens [split T, split T + T) of KV head g ONCE and computes the partial (m, l, o) of
// every one of the G query heads that read that KV head. Each wave keeps its own running
// (m, l, o) over the sub-chunks it streams (online softmax, no barrier inside the loop), with
// the next sub-chunk's loads in flight while one is consumed; the four waves meet in LDS at
// the end. The partials of a head are merged by the same kernel as
// the sparse step's.
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

template <int BF16, int G>
struct DenseShape {
  static constexpr int EPL = BF16 ? 8 : 4;          // elements per lane per row
  static constexpr int LPR = kD / EPL;              // lanes per row
  static constexpr int RPI = kWave / LPR;           // rows per wave-wide load
  static constexpr int ITER = G <= 4 ? 4 : 2;       // loads per lane per sub-chunk (K and V)
  static constexpr int RPW = RPI * ITER;            // rows per wave per sub-chunk
  static constexpr int SUB = 4 * RPW;               // rows per workgroup per sub-chunk
};

__device__ __forceinline__ void unpack_row(const uint4& x, float (&f)[8]) {
  f[0] = __uint_as_float(x.x << 16); f[1] = __uint_as_float(x.x & 0xFFFF0000u);
  f[2] = __uint_as_float(x.y << 16); f[3] = __uint_as_float(x.y & 0xFFFF0000u);
  f[4] = __uint_as_float(x.z << 16); f[5] = __uint_as_float(x.z & 0xFFFF0000u);
  f[6] = __uint_as_float(x.w << 16); f[7] = __uint_as_float(x.w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack_row(const uint4& x, float (&f)[4]) {
  f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
  f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
}

template <int BF16, int G>
__global__ void __launch_bounds__(256)
dense_attn_kernel(Shape s, const void* __restrict__ K, const void* __restrict__ V,
                  const void* __restrict__ q, const int32_t* __restrict__ seq_lens,
                  float* __restrict__ part, int nsplit, int tpw, float scale_log2e) {
  using A = DenseShape<BF16, G>;
  constexpr int EPL = A::EPL, LPR = A::LPR, RPI = A::RPI, ITER = A::ITER;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(max(seq_lens[b], 0), s.Lmax);
  const int w = wave_id(), lane = lane_id();
  const int rg = lane / LPR, sub = lane % LPR;
  const int t0 = split * tpw, t1 = min(t0 + tpw, L);
  const size_t esz = BF16 ? 2 : 4;

  // queries of the G heads, this lane's EPL elements, scaled into the log2 domain
  float qv[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const size_t qo = (size_t(b) * s.Hq + size_t(g) * G + hh) * kD + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = load_elem(q, qo + e, s.q_bf16) * scale_log2e;
  }

  float M[G], l[G], o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    M[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  const size_t kvrow0 = (size_t(b) * s.Hkv + g) * s.Lmax;
  const char* Kc = static_cast<const char*>(K);
  const char* Vc = static_cast<const char*>(V);
  // K and V of this lane's rows of the sub-chunk at c0 (rows past the range re-read the last
  // one, so every load is in bounds and the loop carries no branch around its loads)
  auto load = [&](int c0, uint4 (&kr)[ITER], uint4 (&vr)[ITER]) {
    const int r0 = c0 + w * A::RPW + rg;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int t = max(min(r0 + it * RPI, t1 - 1), 0);
      const size_t off = ((kvrow0 + size_t(t)) * kD + sub * EPL) * esz;
      kr[it] = *reinterpret_cast<const uint4*>(Kc + off);
      vr[it] = *reinterpret_cast<const uint4*>(Vc + off);
    }
  };
  // online softmax over one sub-chunk: logits, running maximum, rescale, weighted V sum
  auto consume = [&](int c0, const uint4 (&kr)[ITER], const uint4 (&vr)[ITER]) {
    const int r0 = c0 + w * A::RPW + rg;
    float sc[G][ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      float f[EPL];
      unpack_row(kr[it], f);
      const bool ok = r0 + it * RPI < t1;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qv[hh][e], f[e], d);
        d = row16_sum(d);                       // the row's LPR lanes: 16, or 32 for fp32
        if constexpr (LPR == 32) d += lane_xor(d, 16);
        sc[hh][it] = ok ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float cm = sc[hh][0];
#pragma unroll
      for (int it = 1; it < ITER; ++it) cm = fmaxf(cm, sc[hh][it]);
      cm = wave_max(cm);
      const float Mn = fmaxf(M[hh], cm);          // -inf while this wave has seen no live row
      const float f0 = M[hh] == -INFINITY ? 0.f : exp2f(M[hh] - Mn);
      l[hh] *= f0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] *= f0;
      M[hh] = Mn;
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      float f[EPL];
      unpack_row(vr[it], f);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = sc[hh][it] == -INFINITY ? 0.f : exp2f(sc[hh][it] - M[hh]);
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(p, f[e], o[hh][e]);
      }
    }
  };
  // two register buffers: the next sub-chunk's loads are in flight while one is consumed
  uint4 ka[ITER], va[ITER], kb[ITER], vb[ITER];
  if (t0 < t1) load(t0, ka, va);
  for (int c0 = t0; c0 < t1; c0 += 2 * A::SUB) {
    load(c0 + A::SUB, kb, vb);
    consume(c0, ka, va);
    if (c0 + A::SUB >= t1) break;                // uniform
    load(c0 + 2 * A::SUB, ka, va);
    consume(c0 + A::SUB, kb, vb);
  }

  // ---- per wave: sum over the row groups (lanes sharing `sub`); then the four waves merge
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
      l[hh] += lane_from_above(l[hh], off);   // into row group 0, which stores
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] += lane_from_above(o[hh][e], off);
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[w][hh][sub * EPL + e] = o[hh][e];
    }
    if (lane == 0) {
      s_m[w][hh] = M[hh];
      s_l[w][hh] = l[hh];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
    const int hh = i / kD, d = i % kD;
    const float Mw = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
    float os = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = s_m[ww][hh] == -INFINITY ? 0.f : exp2f(s_m[ww][hh] - Mw);
      os = fmaf(s_o[ww][hh][d], f, os);
      ls = fmaf(s_l[ww][hh], f, ls);
    }
    float* pp = part + ((size_t(b) * s.Hq + size_t(g) * G + hh) * nsplit + split) * (kD + 2);
    pp[d] = os;
    if (d == 0) {
      pp[kD] = Mw;
      pp[kD + 1] = ls;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 K/V: the logits of the G heads are one small matrix product per 16 tokens on the matrix
// cores, S[head][token] = Q K^T with v_mfma_f32_16x16x32_bf16 (Q padded to 16 rows with zeros;
// bf16 x bf16 products are exact, fp32 accumulation). A fp32 query enters as two bf16 pieces
// (hi + lo, relative remainder below 2^-16). The weighted V sum stays on the vector units in
// the row layout (16 lanes x 8 dimensions per row), the probabilities handed over through LDS
// inside the wave. Each wave streams 32 tokens per sub-chunk, two register buffers deep.
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDenseTokW = 32;                      // tokens per wave per sub-chunk
constexpr int kDenseSub = 4 * kDenseTokW;           // tokens per workgroup per sub-chunk
static_assert(kGatherChunk % kDenseSub == 0 && kGatherChunk <= 1024, "gathered chunk");

// Gathered rows (IDX): the workgroup's positions [t0, t1) index a KV head's list of selected
// tokens (group-shared selection) instead of the context itself.
struct GatherList {
  const int32_t* idx;   // [B][Hkv][istride]
  const int32_t* cnt;   // [B][Hkv]
  int istride;
};
constexpr int kGatherMax = 1024;                    // list positions per workgroup

template <int G, int QF32, int IDX>
__global__ void __launch_bounds__(256)
dense_attn_mfma_kernel(Shape s, const void* __restrict__ K, const void* __restrict__ V,
                       const void* __restrict__ q, const int32_t* __restrict__ seq_lens,
                       float* __restrict__ part, int nsplit, int tpw, float scale_log2e,
                       GatherList gl) {
  static_assert(G <= 8, "heads of a group fill rows 4 (l / 16) + i of the 16 x 16 tile");
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = IDX ? gl.cnt[size_t(b) * s.Hkv + g] : min(max(seq_lens[b], 0), s.Lmax);
  const int w = wave_id(), lane = lane_id();
  const int col = lane % 16, quad = lane / 16;      // MFMA: token column / k quarter
  const int t0 = split * tpw, t1 = min(t0 + tpw, L);
  // the workgroup's token positions (gathered rows): staged in LDS once
  __shared__ int32_t s_tok[IDX ? kGatherMax : 1];
  if constexpr (IDX) {
    const int32_t* il = gl.idx + (size_t(b) * s.Hkv + g) * gl.istride;
    for (int i = threadIdx.x; i < tpw; i += blockDim.x)
      s_tok[i] = t1 > t0 ? min(max(il[min(t0 + i, t1 - 1)], 0), s.Lmax - 1) : 0;
    __syncthreads();
  }
  // context position of list position pos (clamped into [t0, t1 - 1])
  auto token = [&](int pos) {
    const int c = max(min(pos, t1 - 1), 0);
    if constexpr (IDX) return s_tok[max(c - t0, 0)];
    else return c;
  };
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const uint16_t* Vb = static_cast<const uint16_t*>(V);
  const size_t kvrow0 = (size_t(b) * s.Hkv + g) * s.Lmax;

  // A operand: Q rows = heads (col < G), k elements 32 quad + 8 ks + i of block ks (the same
  // permutation of the 128 dimensions is used for K below, so the dot products are unchanged)
  bf16x8_t qa[4], qb[4];
  {
    const bool hv = col < G;
    const size_t qo = (size_t(b) * s.Hq + size_t(g) * G + (hv ? col : 0)) * kD + 32 * quad;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = 0.f;
        if constexpr (QF32) x = static_cast<const float*>(q)[qo + 8 * ks + i];
        else x = bf16_bits_to_f32(static_cast<const uint16_t*>(q)[qo + 8 * ks + i]);
        x = hv ? x : 0.f;
        const __bf16 hi = __bf16(x);
        qa[ks][i] = hi;
        qb[ks][i] = __bf16(x - float(hi));
      }
    }
  }

  // running state: M (per head, wave-uniform), l (per head, partial per MFMA lane), o (per
  // head and the lane's 8 dimensions, partial over the lane's rows)
  float M[G], lp[4], o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    M[hh] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) lp[i] = 0.f;

  __shared__ float s_p[4][kDenseTokW][8];           // probabilities [wave][token][head]
  const int rg = lane / 16, sub = lane % 16;        // row layout for V: row group, 8 dims

  // K: B operand of tile tt = token column col, elements 32 quad .. 32 quad + 31 (4 x 16 B);
  // V: row layout, rows rg + 4 it. Rows past the range re-read the last valid one.
  auto load = [&](int c0, uint4 (&kr)[2][4], uint4 (&vr)[8]) {
    const int base = c0 + w * kDenseTokW;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = token(base + 16 * tt + col);
      const uint4* kp = reinterpret_cast<const uint4*>(Kb + (kvrow0 + size_t(t)) * kD + 32 * quad);
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[tt][j] = kp[j];
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int t = token(base + rg + 4 * it);
      vr[it] = *reinterpret_cast<const uint4*>(Vb + (kvrow0 + size_t(t)) * kD + 8 * sub);
    }
  };
  auto consume = [&](int c0, const uint4 (&kr)[2][4], const uint4 (&vr)[8]) {
    const int base = c0 + w * kDenseTokW;
    // logits S[head 4 quad + i][token 16 tt + col], scaled into the log2 domain
    f32x4_t sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8_t, kr[tt][ks]),
                                                      acc, 0, 0, 0);
      if constexpr (QF32) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[ks], __builtin_bit_cast(bf16x8_t, kr[tt][ks]),
                                                        acc, 0, 0, 0);
      }
      const bool ok = base + 16 * tt + col < t1;
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[tt][i] = ok ? acc[i] * scale_log2e : -INFINITY;
    }
    // per-head maximum of the sub-chunk (over the 16 columns of the head's row of lanes)
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = row16_max(fmaxf(sc[0][i], sc[1][i]));
    }
    float f0[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx[hh % 4]), 16 * (hh / 4)));
      const float Mn = fmaxf(M[hh], m);            // -inf while this wave has seen no live row
      f0[hh] = M[hh] == -INFINITY ? 0.f : exp2f(M[hh] - Mn);
      M[hh] = Mn;
    }
    // probabilities into LDS (lanes of valid heads), l partials; o rescaled
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * quad + i;
      float Mh = M[0], fh = f0[0];
#pragma unroll
      for (int h2 = 1; h2 < G; ++h2) {
        Mh = hh == h2 ? M[h2] : Mh;
        fh = hh == h2 ? f0[h2] : fh;
      }
      const float p0 = sc[0][i] == -INFINITY ? 0.f : exp2f(sc[0][i] - Mh);
      const float p1 = sc[1][i] == -INFINITY ? 0.f : exp2f(sc[1][i] - Mh);
      lp[i] = fmaf(lp[i], fh, p0 + p1);
      if (hh < G) {
        s_p[w][col][hh] = p0;
        s_p[w][16 + col][hh] = p1;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= f0[hh];
    asm volatile("" ::: "memory");   // LDS writes of this wave before its reads (in order)
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      float pv[8];
      const float4 pa = *reinterpret_cast<const float4*>(&s_p[w][rg + 4 * it][0]);
      pv[0] = pa.x; pv[1] = pa.y; pv[2] = pa.z; pv[3] = pa.w;
      if constexpr (G > 4) {
        const float4 pb = *reinterpret_cast<const float4*>(&s_p[w][rg + 4 * it][4]);
        pv[4] = pb.x; pv[5] = pb.y; pv[6] = pb.z; pv[7] = pb.w;
      }
      float f[8];
      unpack_row(vr[it], f);
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pv[hh], f[e], o[hh][e]);
    }
    asm volatile("" ::: "memory");
  };

  uint4 ka[2][4], va[8], kb[2][4], vb[8];
  if (t0 < t1) load(t0, ka, va);
  for (int c0 = t0; c0 < t1; c0 += 2 * kDenseSub) {
    load(c0 + kDenseSub, kb, vb);
    consume(c0, ka, va);
    if (c0 + kDenseSub >= t1) break;                // uniform
    load(c0 + 2 * kDenseSub, ka, va);
    consume(c0 + kDenseSub, kb, vb);
  }

  // ---- per wave: o over the row groups, l over the 16 token columns; then the waves merge
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = row16_sum(lp[i]);
    const int hh = 4 * quad + i;
    if (col == 0 && hh < G) s_l[w][hh] = v;
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] += lane_from_above(o[hh][e], off);   // row group 0 stores
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[w][hh][sub * 8 + e] = o[hh][e];
    }
    if (lane == 0) s_m[w][hh] = M[hh];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += blockDim.x) {
    const int hh = i / kD, d = i % kD;
    const float Mw = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
    float os = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = s_m[ww][hh] == -INFINITY ? 0.f : exp2f(s_m[ww][hh] - Mw);
      os = fmaf(s_o[ww][hh][d], f, os);
      ls = fmaf(s_l[ww][hh], f, ls);
    }
    float* pp = part + ((size_t(b) * s.Hq + size_t(g) * G + hh) * nsplit + split) * (kD + 2);
    pp[d] = os;
    if (d == 0) {
      pp[kD] = Mw;
      pp[kD + 1] = ls;
    }
  }
}

// Tokens per workgroup: whole pairs of sub-chunks, sized so that the grid holds about 1024
// workgroups (four per CU) when the context allows, and at most 64 sub-chunks.
template <int BF16, int G>
static int dense_tpw(const Shape& s) {
  constexpr int SUB = BF16 ? kDenseSub : DenseShape<BF16, G>::SUB;
  const long long rows = (long long)s.Lmax * s.B * s.Hkv;
  long long subs = (rows + 1024LL * SUB - 1) / (1024LL * SUB);
  if (subs < 2) subs = 2;
  if (subs > 64) subs = 64;
  return int((subs + 1) & ~1LL) * SUB;   // pairs of sub-chunks (two register buffers)
}

int dense_tokens_per_split(const Shape& s) {
  switch (s.G * 2 + s.kv_bf16) {
    case 2: return dense_tpw<0, 1>(s);
    case 3: return dense_tpw<1, 1>(s);
    case 4: return dense_tpw<0, 2>(s);
    case 5: return dense_tpw<1, 2>(s);
    case 8: return dense_tpw<0, 4>(s);
    case 9: return dense_tpw<1, 4>(s);
    case 16: return dense_tpw<0, 8>(s);
    default: return dense_tpw<1, 8>(s);
  }
}

template <int BF16, int G>
static hipError_t launch_dense_t(const Shape& s, const CacheView& c, const void* q, float* part,
                           int nsplit, int tpw, float scale_log2e, KernelTimer tm,
                           hipStream_t st) {
  const dim3 grid(nsplit, s.Hkv, s.B);
  const GatherList none{nullptr, nullptr, 0};
  if constexpr (BF16) {
    if (s.q_bf16)
      return launch_kernel("dense_attn_mfma_kernel",
                           dense_attn_mfma_kernel<G, 0, 0>, grid, dim3(256), st, tm, s, c.K, c.V,
                           q, c.seq_lens, part, nsplit, tpw, scale_log2e, none);
    return launch_kernel("dense_attn_mfma_kernel",
                         dense_attn_mfma_kernel<G, 1, 0>, grid, dim3(256), st, tm, s, c.K, c.V, q,
                         c.seq_lens, part, nsplit, tpw, scale_log2e, none);
  } else {
    return launch_kernel("dense_attn_kernel",
                         dense_attn_kernel<BF16, G>, grid, dim3(256), st, tm, s, c.K, c.V, q,
                         c.seq_lens, part, nsplit, tpw, scale_log2e);
  }
}

hipError_t launch_dense(const Shape& s, const CacheView& c, const void* q, float scale,
                        void* ws, float* out, const DebugView& dbg, hipStream_t st) {
  const int tpw = dense_tokens_per_split(s);
  const int nsplit = (s.Lmax + tpw - 1) / tpw;
  float* part = static_cast<float*>(ws);
  const float sl2 = scale * 1.4426950408889634f;
  const KernelTimer tm = kernel_timer(dbg, 0);
  hipError_t e;
  switch (s.G * 2 + s.kv_bf16) {
    case 2: e = launch_dense_t<0, 1>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 3: e = launch_dense_t<1, 1>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 4: e = launch_dense_t<0, 2>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 5: e = launch_dense_t<1, 2>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 8: e = launch_dense_t<0, 4>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 9: e = launch_dense_t<1, 4>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 16: e = launch_dense_t<0, 8>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    default: e = launch_dense_t<1, 8>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
  }
  if (e != hipSuccess) return e;
  return launch_combine(s, part, nsplit, out, c.seq_lens, 0, kernel_timer(dbg, 1), st);
}

template <int G>
static hipError_t launch_gather_t(const Shape& s, const CacheView& c, const void* q, float* part,
                            int nsplit, float scale_log2e, const GatherList& gl, KernelTimer tm,
                            hipStream_t st) {
  const dim3 grid(nsplit, s.Hkv, s.B);
  if (s.q_bf16)
    return launch_kernel("dense_attn_mfma_kernel",
                         dense_attn_mfma_kernel<G, 0, 1>, grid, dim3(256), st, tm, s, c.K, c.V, q,
                         c.seq_lens, part, nsplit, kGatherChunk, scale_log2e, gl);
  return launch_kernel("dense_attn_mfma_kernel",
                       dense_attn_mfma_kernel<G, 1, 1>, grid, dim3(256), st, tm, s, c.K, c.V, q,
                       c.seq_lens, part, nsplit, kGatherChunk, scale_log2e, gl);
}

hipError_t launch_attn_gather(const Shape& s, const CacheView& c, const void* q, float scale,
                              const int32_t* idx, const int32_t* cnt, int istride, float* part,
                              int nsplit, KernelTimer tm, hipStream_t st) {
  const GatherList gl{idx, cnt, istride};
  const float sl2 = scale * 1.4426950408889634f;
  switch (s.G) {
    case 1: return launch_gather_t<1>(s, c, q, part, nsplit, sl2, gl, tm, st);
    case 2: return launch_gather_t<2>(s, c, q, part, nsplit, sl2, gl, tm, st);
    case 4: return launch_gather_t<4>(s, c, q, part, nsplit, sl2, gl, tm, st);
    default: return launch_gather_t<8>(s, c, q, part, nsplit, sl2, gl, tm, st);
  }
}

size_t dense_workspace_bytes(const Shape& s) {
  const int tpw = dense_tokens_per_split(s);
  const int nsplit = (s.Lmax + tpw - 1) / tpw;
  return size_t(s.B) * s.Hq * nsplit * (kD + 2) * sizeof(float);
}

}  // namespace hhr
