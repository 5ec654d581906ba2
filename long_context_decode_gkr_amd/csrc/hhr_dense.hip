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
// (m, l, o) over the sub-chunks it streams (online softmax, no barrier inside the loop); the
// four waves meet in LDS at the end. The partials of a head are merged by the same kernel as
// the sparse step's.
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

template <int BF16, int G>
struct DenseShape {
  static constexpr int EPL = BF16 ? 8 : 4;          // elements per lane per row
  static constexpr int LPR = kD / EPL;              // lanes per row
  static constexpr int RPI = kWave / LPR;           // rows per wave-wide load
  static constexpr int ITER = G <= 4 ? 8 : 4;       // loads per lane per sub-chunk (K and V)
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
  for (int c0 = t0; c0 < t1; c0 += A::SUB) {
    const int r0 = c0 + w * A::RPW + rg;          // this lane's first row of the sub-chunk
    uint4 kr[ITER], vr[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int t = min(r0 + it * RPI, t1 - 1);   // rows past the range re-read the last one
      const size_t off = ((kvrow0 + size_t(t)) * kD + sub * EPL) * esz;
      kr[it] = *reinterpret_cast<const uint4*>(Kc + off);
      vr[it] = *reinterpret_cast<const uint4*>(Vc + off);
    }
    __builtin_amdgcn_sched_barrier(0);
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
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
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
  }

  // ---- per wave: sum over the row groups (lanes sharing `sub`); then the four waves merge
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
      l[hh] += __shfl_xor(l[hh], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] += __shfl_xor(o[hh][e], off);
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

// Tokens per workgroup: whole sub-chunks, sized so that the grid holds about 1024 workgroups
// (four per CU) when the context allows, and at most 64 sub-chunks.
template <int BF16, int G>
static int dense_tpw(const Shape& s) {
  constexpr int SUB = DenseShape<BF16, G>::SUB;
  const long long rows = (long long)s.Lmax * s.B * s.Hkv;
  long long subs = (rows + 1024LL * SUB - 1) / (1024LL * SUB);
  if (subs < 1) subs = 1;
  if (subs > 64) subs = 64;
  return int(subs) * SUB;
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
static void launch_dense_t(const Shape& s, const CacheView& c, const void* q, float* part,
                           int nsplit, int tpw, float scale_log2e, KernelTimer tm,
                           hipStream_t st) {
  launch_kernel(dense_attn_kernel<BF16, G>, dim3(nsplit, s.Hkv, s.B), dim3(256), st, tm, s,
                c.K, c.V, q, c.seq_lens, part, nsplit, tpw, scale_log2e);
}

hipError_t launch_dense(const Shape& s, const CacheView& c, const void* q, float scale,
                        void* ws, float* out, const DebugView& dbg, hipStream_t st) {
  const int tpw = dense_tokens_per_split(s);
  const int nsplit = (s.Lmax + tpw - 1) / tpw;
  float* part = static_cast<float*>(ws);
  const float sl2 = scale * 1.4426950408889634f;
  const KernelTimer tm = kernel_timer(dbg, 0);
  switch (s.G * 2 + s.kv_bf16) {
    case 2: launch_dense_t<0, 1>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 3: launch_dense_t<1, 1>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 4: launch_dense_t<0, 2>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 5: launch_dense_t<1, 2>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 8: launch_dense_t<0, 4>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 9: launch_dense_t<1, 4>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    case 16: launch_dense_t<0, 8>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
    default: launch_dense_t<1, 8>(s, c, q, part, nsplit, tpw, sl2, tm, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(s, part, nsplit, out, c.seq_lens, 0, kernel_timer(dbg, 1), st);
}

size_t dense_workspace_bytes(const Shape& s) {
  const int tpw = dense_tokens_per_split(s);
  const int nsplit = (s.Lmax + tpw - 1) / tpw;
  return size_t(s.B) * s.Hq * nsplit * (kD + 2) * sizeof(float);
}

}  // namespace hhr
