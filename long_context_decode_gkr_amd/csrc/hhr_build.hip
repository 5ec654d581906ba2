// Index build on the fp64 vector units, and the per-token append.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", §3.3.1 (pages,
// per-dimension extrema of the rotated keys k~ = k R, Eq. 4) and §3.1 Eq. 1 / §3.3.2 Eq. 10
// (key code = sign of z = k W at inference).
#include <type_traits>

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
        store_extrema(s, c, sidx + p, lo, hi);
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
  return launch_kernel("build_fp64_kernel", build_fp64_kernel<NB, S>, grid, dim3(kD + NB), st,
                       KernelTimer{nullptr, nullptr}, s, c, R, W);
}

hipError_t launch_build_fp64(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st) {
  if (s.NB == 128) return s.S == 16 ? launch_build_fp64_t<128, 16>(s, c, R, W, st)
                                    : launch_build_fp64_t<128, 32>(s, c, R, W, st);
  return s.S == 16 ? launch_build_fp64_t<256, 16>(s, c, R, W, st)
                   : launch_build_fp64_t<256, 32>(s, c, R, W, st);
}

// ---------------------------------------------------------------------------------------------
// Step preparation, grid (4 column slices x 2 roles, KV head g, sequence b), max(256, 2 NB)
// threads. Workgroups 0-3 own 32 channels of the rotation each, workgroups 4-7 NB / 4 code
// columns each (the two roles on separate CUs: 6.8 -> 5.3 us at the 128K workload against one
// workgroup doing both). Vector 0 is the new key (when k_new is given and seq_lens[b] <
// max_seq_len), vectors 1 .. G the queries (decode mode). Each R_g / W_g column of the slice
// is read once and applied to every vector.
//   * rotation lanes [0, 256): column j over 8 lanes of 16 terms, fp64 sums of exact products
//     reduced by DPP: k~ is folded into page t / S (which it opens when t % S == 0), q~
//     (Eq. 4) goes to the decode workspace; the workgroup also stores its slice of the K and V
//     rows of t;
//   * code lanes: column c of W the same way in fp32 with a certificate for the sign, the few
//     uncertain bits recomputed in fp64 and, where that is not certain either, exactly:
//     sign(k W_g) into the cache and sign(q W_g) (Eq. 1, Eq. 10) into the decode workspace.
// Append mode (hhr_append) also advances seq_lens[b]: the last workgroup of the sequence to
// finish does it (a per-sequence ticket, left at 0). In decode mode the step's last kernel
// does it, after every kernel of the step has worked on t + 1 tokens.
// ---------------------------------------------------------------------------------------------
constexpr int kPrepSlices = 4;
constexpr int kPrepParts = 8;
// workgroup size: 256 rotation lanes, or 8 lanes per code column of a slice if more
template <int NB>
constexpr int prep_threads() {
  return 256 > kPrepParts * NB / kPrepSlices ? 256 : kPrepParts * NB / kPrepSlices;
}
// KB, QB: keys/values, queries in bf16; DEC: the number of queries (the group size G) in a
// decode step, 0 for a plain append. Vector 0 is the key, vectors 1 .. DEC the queries.
template <int NB, int KB, int QB, int DEC>
__global__ void __launch_bounds__(prep_threads<NB>())
prep_kernel(Shape s, CacheView c, const void* __restrict__ kn, const void* __restrict__ vn,
            const void* __restrict__ q, const float* __restrict__ R, const float* __restrict__ W,
            float* __restrict__ qrot, uint32_t* __restrict__ qcode, float* __restrict__ dbg_qrot,
            uint32_t* __restrict__ dbg_qcode) {
  constexpr int NW = NB / 32;
  constexpr int CC = NB / kPrepSlices;          // code columns per slice (32 or 64)
  constexpr int WPS = CC / 32;                  // code words per slice (1 or 2)
  constexpr int T = kD / kPrepParts;            // terms per lane (16)
  constexpr int NT = prep_threads<NB>();        // workgroup size
  constexpr int QPT = DEC ? (DEC * kD + NT - 1) / NT : 1;   // query elements per thread
  constexpr int NV = 1 + DEC;                                 // vectors
  const int sl = blockIdx.x % kPrepSlices, g = blockIdx.y, b = blockIdx.z;
  const bool rotwg = blockIdx.x < kPrepSlices;  // rotation workgroup; else code workgroup
  const int tid = threadIdx.x;
  const int part = tid & (kPrepParts - 1);
  const bool rot = rotwg && tid < 256;          // rotation lanes
  const bool codel = !rotwg && tid < kPrepParts * CC;   // code lanes
  constexpr int nq = DEC;
  const bool has_k = kn != nullptr;
  if (!has_k && nq == 0) return;

  __shared__ float xs[NV][kD];
  __shared__ uint8_t bits[NV][CC];

  // Everything that does not depend on the sequence length is loaded together with it: the
  // new key and value elements, the queries, then this lane's 16 column terms.
  const int t = c.seq_lens[b];
  const int j = sl * 32 + (tid >> 3);           // rotation column (rotation lanes)
  const int lc = (tid >> 3) % CC;               // code column within the slice (code lanes)
  const int cc = sl * CC + lc;
  // The vector loads carry no branch (a branch would make the compiler wait for each load
  // before the join): a missing key or query input is replaced by the other input, whose
  // values are then loaded but not used, and indices are clamped.
  const size_t krow = (size_t(b) * s.Hkv + g) * kD;
  const bool own = rotwg && (tid >> 5) == sl;   // this workgroup stores K/V element tid
  const int kel = min(tid, kD - 1);
  const uint32_t kraw = load_raw(has_k ? kn : q, has_k ? krow + kel : 0, KB);
  const uint32_t vraw = load_raw(has_k ? vn : q, has_k ? krow + kel : 0, KB);
  uint32_t qraw[QPT];
  if constexpr (DEC) {
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int e = min(tid + r * NT, nq * kD - 1);
      qraw[r] = load_raw(q, (size_t(b) * s.Hq + g * s.G) * kD + e, QB);
    }
  }
  float cv[T];
  {
    const float* col = rot ? R + size_t(g) * kD * kD + size_t(part * T) * kD + j
                           : W + size_t(g) * kD * NB + size_t(part * T) * NB + cc;
    const int stride = rot ? kD : NB;
#pragma unroll
    for (int i = 0; i < T; ++i) cv[i] = col[size_t(i) * stride];
  }
  // The open page's extrema (page t / S) for this lane's rotation column (code lanes read
  // column 32 sl, unused): in bounds whatever t is; needed only after the dot products.
  const bool app = has_k && t >= 0 && t < s.Lmax;
  const int p = app ? t / s.S : 0;
  const size_t si = ((size_t(b) * s.Hkv + g) * kD + (rot ? j : sl * 32)) * s.Pmax + p;
  // raw bits, converted where they are used (a conversion inside the load's branch would make
  // the compiler wait for every load issued before it)
  const uint32_t omin_raw = load_raw(c.pmin, si, s.sum_bf16);
  const uint32_t omax_raw = load_raw(c.pmax, si, s.sum_bf16);

  const size_t row = (size_t(b) * s.Hkv + g) * s.Lmax + (app ? t : 0);
  if (tid < kD && has_k) {
    if (app && own) {
      if (KB) {
        reinterpret_cast<uint16_t*>(c.K)[row * kD + tid] = uint16_t(kraw);
        reinterpret_cast<uint16_t*>(c.V)[row * kD + tid] = uint16_t(vraw);
      } else {
        reinterpret_cast<uint32_t*>(c.K)[row * kD + tid] = kraw;
        reinterpret_cast<uint32_t*>(c.V)[row * kD + tid] = vraw;
      }
    }
    xs[0][tid] = raw_to_f32(kraw, KB);
  }
  if constexpr (DEC) {
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int e = tid + r * NT;
      if (e < nq * kD) xs[1 + e / kD][e % kD] = raw_to_f32(qraw[r], QB);
    }
  }
  __syncthreads();

  auto active = [&](int v) { return v == 0 ? app : v <= nq; };
  if (rot) {
    // ---- rotation column j, terms [16 part, 16 part + 16)
    double acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      double a = 0.0;
      if (active(v)) {
        const float* x = &xs[v][part * T];
#pragma unroll
        for (int i = 0; i < T; ++i) a += double(x[i]) * double(cv[i]);
      }
      acc[v] = group_sum_f64<3>(a);
    }
    if (part == 0) {
      if (app) {
        const float kt = float(acc[0]);
        const bool first = t % s.S == 0;        // the key opens page p
        // (a stored bf16 extremum is already rounded outward, so rounding the fp32 min / max
        // of it and k~ outward equals folding the rounded k~ into it)
        const float omin = raw_to_f32(omin_raw, s.sum_bf16);
        const float omax = raw_to_f32(omax_raw, s.sum_bf16);
        store_extrema(s, c, si, first ? kt : fminf(omin, kt), first ? kt : fmaxf(omax, kt));
      }
#pragma unroll
      for (int v = 1; v < NV; ++v) {
        if (v <= nq) {
          const size_t o = (size_t(b) * s.Hq + g * s.G + (v - 1)) * kD + j;
          qrot[o] = float(acc[v]);
          if (dbg_qrot) dbg_qrot[o] = float(acc[v]);
        }
      }
    }
  } else if (codel) {
    // ---- code column cc, terms [16 part, 16 part + 16): fp32 with a certificate
    float z[NV], sa[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float zz = 0.f, ss = 0.f;
      if (active(v)) {
        const float* x = &xs[v][part * T];
#pragma unroll
        for (int i = 0; i < T; ++i) {
          zz = fmaf(x[i], cv[i], zz);
          ss = fmaf(fabsf(x[i]), fabsf(cv[i]), ss);
        }
      }
      z[v] = group8_sum(zz);
      sa[v] = group8_sum(ss);
    }
    if (part == 0) {
      const float* wcol = W + size_t(g) * kD * NB + cc;
      for (int v = 0; v < NV; ++v) {
        if (!active(v)) continue;
        int cb = certain_bit_f32(z[v], sa[v]);
        if (cb < 0) cb = int(certified_bit(static_cast<const float*>(&xs[v][0]), wcol, NB));
        bits[v][lc] = uint8_t(cb);
      }
    }
  }
  __syncthreads();
  // ---- pack this slice's code words: thread (v, w) builds word w of vector v
  if (!rotwg && tid < (1 + nq) * WPS) {
    const int v = tid / WPS, wi = tid % WPS;
    if (active(v)) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) word |= uint32_t(bits[v][32 * wi + i]) << i;
      const int wg = sl * WPS + wi;               // word index within the code
      if (v == 0) {
        c.codes[row * NW + wg] = word;
      } else {
        const size_t o = (size_t(b) * s.Hq + g * s.G + (v - 1)) * NW + wg;
        qcode[o] = word;
        if (dbg_qcode) dbg_qcode[o] = word;
      }
    }
  }
  if constexpr (!DEC) {
    if (app) {
      // Every workgroup of sequence b has read seq_lens[b] (the load completed before the
      // barrier) before it takes a ticket, so the last one can advance it; the following
      // kernels see the new value at the kernel boundary. No device-scope fence is needed (on
      // gfx950 one would write back and invalidate the whole L2 of the XCD).
      __syncthreads();
      if (tid == 0) {
        const int done = atomicAdd(&c.ticket[b], 1);
        if (done == s.Hkv * kPrepSlices * 2 - 1) {
          c.ticket[b] = 0;
          c.seq_lens[b] = t + 1;
        }
      }
    }
  }
}

template <int NB, int KB, int QB>
static hipError_t launch_prep_t(const Shape& s, const CacheView& c, const void* k_new,
                                const void* v_new, const void* q, const float* R, const float* W,
                                float* qrot, uint32_t* qcode, float* dbg_qrot,
                                uint32_t* dbg_qcode, PrepMode mode, KernelTimer tm,
                                hipStream_t st) {
  dim3 grid(2 * kPrepSlices, s.Hkv, s.B);
  dim3 block(prep_threads<NB>());
  if (mode == PrepMode::kDecode) {
    switch (s.G) {
      case 1: return launch_kernel("prep_kernel",
                                   prep_kernel<NB, KB, QB, 1>, grid, block, st, tm, s, c, k_new,
                                   v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode);
      case 2: return launch_kernel("prep_kernel",
                                   prep_kernel<NB, KB, QB, 2>, grid, block, st, tm, s, c, k_new,
                                   v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode);
      case 4: return launch_kernel("prep_kernel",
                                   prep_kernel<NB, KB, QB, 4>, grid, block, st, tm, s, c, k_new,
                                   v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode);
      default: return launch_kernel("prep_kernel",
                                    prep_kernel<NB, KB, QB, 8>, grid, block, st, tm, s, c, k_new,
                                    v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode);
    }
  }
  return launch_kernel("prep_kernel",
                       prep_kernel<NB, KB, QB, 0>, grid, block, st, tm, s, c, k_new, v_new, q, R,
                       W, qrot, qcode, dbg_qrot, dbg_qcode);
}

template <int NB>
static hipError_t launch_prep_nb(const Shape& s, const CacheView& c, const void* k_new,
                                 const void* v_new, const void* q, const float* R,
                                 const float* W, float* qrot, uint32_t* qcode, float* dbg_qrot,
                                 uint32_t* dbg_qcode, PrepMode mode, KernelTimer tm,
                                 hipStream_t st) {
  if (s.kv_bf16 && s.q_bf16)
    return launch_prep_t<NB, 1, 1>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode,
                                   mode, tm, st);
  if (s.kv_bf16)
    return launch_prep_t<NB, 1, 0>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode,
                                   mode, tm, st);
  if (s.q_bf16)
    return launch_prep_t<NB, 0, 1>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode,
                                   mode, tm, st);
  return launch_prep_t<NB, 0, 0>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode,
                                 mode, tm, st);
}

hipError_t launch_prep(const Shape& s, const CacheView& c, const void* k_new, const void* v_new,
                       const void* q, const float* R, const float* W, float* qrot,
                       uint32_t* qcode, float* dbg_qrot, uint32_t* dbg_qcode, PrepMode mode,
                       KernelTimer tm, hipStream_t st) {
  if (s.NB == 128)
    return launch_prep_nb<128>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode,
                               mode, tm, st);
  return launch_prep_nb<256>(s, c, k_new, v_new, q, R, W, qrot, qcode, dbg_qrot, dbg_qcode, mode,
                             tm, st);
}

}  // namespace hhr
