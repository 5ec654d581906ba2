// Index build on the fp64 vector units, and the per-token append.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", §3.3.1 (pages,
// per-dimension extrema of the rotated keys k~ = k R, Eq. 4) and §3.1 Eq. 1 / §3.3.2 Eq. 10
// (key code = sign of z = k W at inference).
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

// ---------------------------------------------------------------------------------------------
// fp64 build: one workgroup per (sequence, KV head, tile of 32 tokens); one thread per output
// column: threads [0, 128) produce the rotated key columns (fp64 dot products, one rounding
// to fp32, then the per-page min / max), threads [128, 128 + NB) produce the code bits
// (fp64 sums of exact products, certified, exact fallback).
// ---------------------------------------------------------------------------------------------
constexpr int kBuildTile = 32;

template <int NB, int S>
__global__ void __launch_bounds__(kD + NB)
build_fp64_kernel(Shape s, CacheView c, const float* __restrict__ R, const float* __restrict__ W) {
  constexpr int T = kBuildTile;
  constexpr int NW = NB / 32;
  const int b = blockIdx.z, g = blockIdx.y, t0 = blockIdx.x * T;
  const int L = min(max(c.seq_lens[b], 0), s.Lmax);
  if (t0 >= L) return;
  const int nval = min(T, L - t0);

  __shared__ float xt[kD][T];  // xt[i][m] = K[t0 + m][i]
  const size_t row0 = (size_t(b) * s.Hkv + g) * s.Lmax + t0;
  for (int e = threadIdx.x; e < T * kD; e += blockDim.x) {
    const int m = e / kD, i = e % kD;
    xt[i][m] = (m < nval) ? load_elem(c.K, (row0 + m) * kD + i, s.kv_bf16) : 0.f;
  }
  __syncthreads();

  const int col = threadIdx.x;
  double acc[T];
#pragma unroll
  for (int m = 0; m < T; ++m) acc[m] = 0.0;

  if (col < kD) {
    // ---- rotated keys: k~[m][col] = sum_i x[m][i] R[i][col]
    const float* rc = R + size_t(g) * kD * kD + col;
    for (int i = 0; i < kD; ++i) {
      const double w = double(rc[size_t(i) * kD]);
      const float4* xr = reinterpret_cast<const float4*>(&xt[i][0]);
#pragma unroll
      for (int q4 = 0; q4 < T / 4; ++q4) {
        const float4 v = xr[q4];
        acc[4 * q4 + 0] += double(v.x) * w;
        acc[4 * q4 + 1] += double(v.y) * w;
        acc[4 * q4 + 2] += double(v.z) * w;
        acc[4 * q4 + 3] += double(v.w) * w;
      }
    }
    const size_t sidx = ((size_t(b) * s.Hkv + g) * kD + col) * s.Pmax;
#pragma unroll
    for (int pp = 0; pp < T / S; ++pp) {
      if (pp * S < nval) {
        float lo = float(acc[pp * S]), hi = lo;
#pragma unroll
        for (int m = pp * S + 1; m < pp * S + S; ++m) {
          if (m < nval) {
            const float v = float(acc[m]);
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
          }
        }
        const int p = (t0 + pp * S) / S;
        c.pmin[sidx + p] = lo;
        c.pmax[sidx + p] = hi;
      }
    }
  } else {
    // ---- code bits: z[m][cc] = sum_i x[m][i] W[i][cc]
    const int cc = col - kD;
    const float* wc = W + size_t(g) * kD * NB + cc;
    double sab[T];
#pragma unroll
    for (int m = 0; m < T; ++m) sab[m] = 0.0;
    for (int i = 0; i < kD; ++i) {
      const double w = double(wc[size_t(i) * NB]);
      const float4* xr = reinterpret_cast<const float4*>(&xt[i][0]);
#pragma unroll
      for (int q4 = 0; q4 < T / 4; ++q4) {
        const float4 v = xr[q4];
        const double p0 = double(v.x) * w, p1 = double(v.y) * w;
        const double p2 = double(v.z) * w, p3 = double(v.w) * w;
        acc[4 * q4 + 0] += p0; sab[4 * q4 + 0] += fabs(p0);
        acc[4 * q4 + 1] += p1; sab[4 * q4 + 1] += fabs(p1);
        acc[4 * q4 + 2] += p2; sab[4 * q4 + 2] += fabs(p2);
        acc[4 * q4 + 3] += p3; sab[4 * q4 + 3] += fabs(p3);
      }
    }
    uint32_t bits = 0;
#pragma unroll
    for (int m = 0; m < T; ++m) {
      int cb = certain_bit(acc[m], sab[m]);
      if (cb < 0) cb = int(exact_bit(Strided{&xt[0][m], T}, wc, NB));
      bits |= uint32_t(cb) << m;
    }
    // Pack: lane l of W-wave v holds bit 64 v + l of every token's code.
    const int v = cc / kWave;
    const int lane = lane_id();
#pragma unroll
    for (int m = 0; m < T; ++m) {
      const uint64_t mask = __ballot((bits >> m) & 1u);
      if (lane == 0 && m < nval) {
        uint2 wds = make_uint2(uint32_t(mask), uint32_t(mask >> 32));
        *reinterpret_cast<uint2*>(c.codes + (row0 + m) * NW + 2 * v) = wds;
      }
    }
  }
}

template <int NB, int S>
static hipError_t launch_build_fp64_t(const Shape& s, const CacheView& c, const float* R,
                                      const float* W, hipStream_t st) {
  dim3 grid((s.Lmax + kBuildTile - 1) / kBuildTile, s.Hkv, s.B);
  hipLaunchKernelGGL((build_fp64_kernel<NB, S>), grid, dim3(kD + NB), 0, st, s, c, R, W);
  return hipGetLastError();
}

hipError_t launch_build_fp64(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st) {
  if (s.NB == 128) return s.S == 16 ? launch_build_fp64_t<128, 16>(s, c, R, W, st)
                                    : launch_build_fp64_t<128, 32>(s, c, R, W, st);
  return s.S == 16 ? launch_build_fp64_t<256, 16>(s, c, R, W, st)
                   : launch_build_fp64_t<256, 32>(s, c, R, W, st);
}

// ---------------------------------------------------------------------------------------------
// Append: one workgroup per (KV head, sequence). Writes the token's K and V rows, folds its
// rotated key into page t / S, writes its code; the last workgroup of a sequence to finish
// advances seq_lens[b] (a per-sequence ticket counts the finished KV heads and is left at 0).
// ---------------------------------------------------------------------------------------------
template <int NB>
__global__ void __launch_bounds__(256)
append_kernel(Shape s, CacheView c, const void* __restrict__ kn, const void* __restrict__ vn,
              const float* __restrict__ R, const float* __restrict__ W) {
  constexpr int NW = NB / 32;
  const int g = blockIdx.x, b = blockIdx.y;
  const int t = c.seq_lens[b];
  if (t < 0 || t >= s.Lmax) return;
  const int tid = threadIdx.x;
  __shared__ float xk[kD];

  const size_t src = (size_t(b) * s.Hkv + g) * kD;
  const size_t row = (size_t(b) * s.Hkv + g) * s.Lmax + t;
  if (tid < kD) {
    if (s.kv_bf16) {
      const uint16_t kb = reinterpret_cast<const uint16_t*>(kn)[src + tid];
      reinterpret_cast<uint16_t*>(c.K)[row * kD + tid] = kb;
      reinterpret_cast<uint16_t*>(c.V)[row * kD + tid] = reinterpret_cast<const uint16_t*>(vn)[src + tid];
      xk[tid] = bf16_bits_to_f32(kb);
    } else {
      const float kf = reinterpret_cast<const float*>(kn)[src + tid];
      reinterpret_cast<float*>(c.K)[row * kD + tid] = kf;
      reinterpret_cast<float*>(c.V)[row * kD + tid] = reinterpret_cast<const float*>(vn)[src + tid];
      xk[tid] = kf;
    }
  }
  __syncthreads();

  // Rotated key on threads [128, 256): fp64 dot, one rounding; fold into the page extrema.
  if (tid >= kD) {
    const int j = tid - kD;
    const float* rc = R + size_t(g) * kD * kD + j;
    double a = 0.0;
#pragma unroll 8
    for (int i = 0; i < kD; ++i) a += double(xk[i]) * double(rc[size_t(i) * kD]);
    const float kt = float(a);
    const int p = t / s.S;
    const size_t si = ((size_t(b) * s.Hkv + g) * kD + j) * s.Pmax + p;
    if (t % s.S == 0) {
      c.pmin[si] = kt;
      c.pmax[si] = kt;
    } else {
      c.pmin[si] = fminf(c.pmin[si], kt);
      c.pmax[si] = fmaxf(c.pmax[si], kt);
    }
  }

  // Code bit c on thread c.
  uint32_t bit = 0;
  if (tid < NB) bit = certified_bit(static_cast<const float*>(xk), W + size_t(g) * kD * NB + tid, NB);
  const uint64_t mask = __ballot(bit);
  if (lane_id() == 0 && tid < NB) {
    *reinterpret_cast<uint2*>(c.codes + row * NW + 2 * (tid / kWave)) =
        make_uint2(uint32_t(mask), uint32_t(mask >> 32));
  }

  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int done = atomicAdd(&c.ticket[b], 1);
    if (done == s.Hkv - 1) {
      c.ticket[b] = 0;
      c.seq_lens[b] = t + 1;
    }
  }
}

hipError_t launch_append(const Shape& s, const CacheView& c, const void* k_new,
                         const void* v_new, const float* R, const float* W, hipStream_t st) {
  dim3 grid(s.Hkv, s.B);
  if (s.NB == 128)
    hipLaunchKernelGGL((append_kernel<128>), grid, dim3(256), 0, st, s, c, k_new, v_new, R, W);
  else
    hipLaunchKernelGGL((append_kernel<256>), grid, dim3(256), 0, st, s, c, k_new, v_new, R, W);
  return hipGetLastError();
}

}  // namespace hhr
