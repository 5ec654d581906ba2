// Index build on the matrix cores (MFMA) for bf16 keys.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", §3.3.1 (page extrema of
// the rotated keys k~ = k R, Eq. 4) and §3.1 Eq. 1 / §3.3.2 Eq. 10 (key code = sign of z = k W).
// Both are one GEMM of the key tile against [R_g | W_g], done with v_mfma_f32_32x32x16_bf16.
//
// Precision. The keys are bf16, so they are exact MFMA A operands. The fp32 R and W are split
// into bf16 pieces (R = r1 + r2 + r3 to ~2^-27, W = w1 + w2 to ~2^-18 relative); every
// bf16 x bf16 product is exact in fp32 and the MFMA accumulates in fp32.
//   * Rotation: k~ carries fp32 accumulation error only (a few ulps of |k|); the page extrema
//     are taken from it.
//   * Codes: a bit is accepted when |z| > tau = 2^-13 |k|_2 |w_c|_2. By Cauchy-Schwarz the
//     accumulated error is at most about 256 * 2^-23 + 2^-18 <= 2^-14.9 times |k|_2 |w_c|_2,
//     so tau has a margin of ~4x. Bits inside tau (about 1e-3 of them for Gaussian data) are
//     queued in LDS and recomputed from the stored operands in fp64 (exact products), with
//     the exact long accumulator behind that: every code equals the sign of the exact z.
//
// Grid (nper x roles, Hkv, B): role 0 = rotation and page extrema, role 1 + s = code words
// [4 s, 4 s + 4) (128 code columns). A workgroup stages its role's B operand once, then builds
// every nper-th tile of 512 tokens of its sequence. Per tile, each of its 8 waves walks
// 32-token sub-tiles: 8 A fragments (one 16-byte load each per lane) are reused against all
// 4 column tiles x 8 k-steps x pieces, B fragments come from LDS.
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMTok = 512;            // tokens per workgroup
constexpr int kMThreads = 512;       // 8 waves: two per SIMD, so MFMA and VALU work overlap
constexpr int kBStride = kD + 8;      // padded k-stride of a transposed B column (bf16 elements)
constexpr int kFbCap = 2048;          // queued uncertain code bits per workgroup
constexpr float kCertScale = 1.0f / 8192.0f;   // 2^-13

// One stored bf16 key row, read as fp32 values.
struct Bf16Row {
  const uint16_t* p;
  __device__ __forceinline__ float operator[](int j) const { return bf16_bits_to_f32(p[j]); }
};


template <int S>
__global__ void __launch_bounds__(kMThreads)
build_mfma_kernel(Shape s, CacheView c, const float* __restrict__ R, const float* __restrict__ W,
                  int ntiles, int nper) {
  // workgroup (role, first) stages its role's B operand once, then builds tiles first,
  // first + nper, ... of the sequence
  const int role = blockIdx.x / nper, first = blockIdx.x % nper;
  const int g = blockIdx.y, b = blockIdx.z;
  const int L = min(max(c.seq_lens[b], 0), s.Lmax);
  if (first * kMTok >= L) return;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int npieces = role == 0 ? 3 : 2;

  __shared__ __align__(16) uint16_t Bt[3][kD][kBStride];     // Bt[piece][n][k]
  // page min / max (role 0); rows padded by one word so that the 32 channels a wave writes
  // at once fall in different LDS banks
  __shared__ float stage_f[2][kD][kMTok / 16 + 1];
  __shared__ uint32_t stage_c[kMTok][4];                     // code words (role > 0)
  __shared__ float wnorm[kD];
  __shared__ float wpart[kMThreads];
  __shared__ uint32_t fb_list[kFbCap];
  __shared__ int fb_n;

  // ---- B operand: split the fp32 matrix into bf16 pieces (hardware round-to-nearest-even,
  // two values per conversion), transposed (k contiguous). Thread tid owns column
  // n = tid % 128 and the row pairs k = 2 (tid / 128 + 4 i), +1: its 32 loads are issued
  // together, and its quarter of the column's squared norm (code roles) is summed on the way.
  constexpr int kTPC = kMThreads / kD;                // threads per column
  constexpr int kPPT = kD * kD / (2 * kMThreads);     // row pairs per thread
  const float* src = role == 0 ? R + size_t(g) * kD * kD
                               : W + size_t(g) * kD * s.NB + (role - 1) * kD;
  const int src_ld = role == 0 ? kD : s.NB;
  const int bn = tid % kD, bk0 = tid / kD;
  float bx[kPPT][2];
#pragma unroll
  for (int i = 0; i < kPPT; ++i) {
    const int k = 2 * (bk0 + kTPC * i);
    bx[i][0] = src[size_t(k) * src_ld + bn];
    bx[i][1] = src[size_t(k + 1) * src_ld + bn];
  }
  float ss = 0.f;
  auto pack = [](float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
  };
  auto lo16 = [](uint32_t v) { return __uint_as_float(v << 16); };
  auto hi16 = [](uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); };
#pragma unroll
  for (int i = 0; i < kPPT; ++i) {
    const int k = 2 * (bk0 + kTPC * i);
    const float x0 = bx[i][0], x1 = bx[i][1];
    const uint32_t p1 = pack(x0, x1);
    const float r0 = x0 - lo16(p1), r1 = x1 - hi16(p1);
    const uint32_t p2 = pack(r0, r1);
    *reinterpret_cast<uint32_t*>(&Bt[0][bn][k]) = p1;
    *reinterpret_cast<uint32_t*>(&Bt[1][bn][k]) = p2;
    if (role == 0)
      *reinterpret_cast<uint32_t*>(&Bt[2][bn][k]) = pack(r0 - lo16(p2), r1 - hi16(p2));
    ss = fmaf(x0, x0, fmaf(x1, x1, ss));
  }
  wpart[tid] = ss;
  __syncthreads();
  // |w_c| from fp32 sums of squares (relative error below 2^-16), rounded up by 2^-14
  if (role != 0 && tid < kD) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kTPC; ++i) q += wpart[tid + i * kD];
    wnorm[tid] = sqrtf(q) * (1.0f + 0x1p-14f);
  }
  __syncthreads();

  const size_t row0 = (size_t(b) * s.Hkv + g) * s.Lmax;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(c.K);
  const int half = lane >> 5, col = lane & 31;

  for (int tile = first; tile < ntiles; tile += nper) {
    const int t0 = tile * kMTok;
    if (t0 >= L) break;
    const int ntok = min(kMTok, L - t0);
    if (tid == 0) fb_n = 0;
    __syncthreads();
    // A fragments of a sub-tile: row tl0 + col, k = 16 ks + 8 half + 0..7 (rows past the end
    // read the last valid row).
    auto load_a = [&](int tl0, bf16x8 (&a)[8]) {
      const int trc = min(t0 + tl0 + col, L - 1);
      const uint4* ap = reinterpret_cast<const uint4*>(Kb + (row0 + trc) * kD + 8 * half);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a[ks] = __builtin_bit_cast(bf16x8, ap[2 * ks]);
    };
    constexpr int kStep = kMThreads / kWave;   // sub-tiles between a wave's consecutive ones
    for (int st = w; st < kMTok / 32; st += kStep) {
      const int tl0 = st * 32;                 // first token of the sub-tile (block-local)
      if (tl0 >= ntok) break;
      bf16x8 a[8];
      load_a(tl0, a);
      f32x16 acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
      for (int p = 0; p < npieces; ++p) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&Bt[p][nt * 32 + col][16 * ks + 8 * half]);
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bv, acc[nt], 0, 0, 0);
          }
        }
      }
      // result rows of this lane: i(r) = 8 (r / 4) + 4 half + r % 4
      if (role == 0) {
        // ---- page extrema of k~ over the valid rows (pages are 16 or 32 rows of the sub-tile).
        // Rows past the end repeat the last valid row (load_a clamps), which lies in the same
        // page, so they leave the partial page's extrema unchanged; pages with no valid row are
        // not written out.
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int j = nt * 32 + col;
          constexpr int PPS = 32 / S;            // pages per sub-tile
#pragma unroll
          for (int pp = 0; pp < PPS; ++pp) {
            float lo = INFINITY, hi = -INFINITY;
#pragma unroll
            for (int r = pp * (16 / PPS); r < (pp + 1) * (16 / PPS); ++r) {
              lo = fminf(lo, acc[nt][r]);
              hi = fmaxf(hi, acc[nt][r]);
            }
            lo = fminf(lo, __shfl_xor(lo, 32));
            hi = fmaxf(hi, __shfl_xor(hi, 32));
            if (half == 0) {
              stage_f[0][j][tl0 / S + pp] = lo;
              stage_f[1][j][tl0 / S + pp] = hi;
            }
          }
        }
      } else {
        // ---- code bits: certified sign of z, or queued for the exact path
        float xn2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = float(a[ks][e]);
            xn2 = fmaf(v, v, xn2);
          }
        xn2 += __shfl_xor(xn2, 32);
        const float xnorm = sqrtf(xn2) * (1.0f + 1e-6f);   // |k_row|, row = tl0 + col
        float xr[16];                                      // |k| of the rows of acc[.][r]
#pragma unroll
        for (int r = 0; r < 16; ++r) xr[r] = __shfl(xnorm, 8 * (r / 4) + 4 * half + (r % 4));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int lc = nt * 32 + col;                    // code column within the slice
          const float wn = wnorm[lc];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * half + (r % 4);
            const float xi = xr[r];
            const float tau = kCertScale * xi * wn;
            const float z = acc[nt][r];
            const bool valid = tl0 + i < ntok;
            const bool sure = fabsf(z) > tau && xi * wn > 1e-30f;
            bool bit = z > 0.f;
            if (valid && !sure) {
              // queued for the exact path (past the capacity only counted: see below)
              const int pos = atomicAdd(&fb_n, 1);
              if (pos < kFbCap) fb_list[pos] = (uint32_t(tl0 + i) << 8) | uint32_t(lc);
            }
            const uint64_t m = __ballot(bit);
            if (lane == 0) {
              // bits 0..31 of the ballot are row i(r) of half 0, bits 32..63 row i(r) + 4
              const int i0 = 8 * (r / 4) + (r % 4);
              stage_c[tl0 + i0][nt] = uint32_t(m);
              stage_c[tl0 + i0 + 4][nt] = uint32_t(m >> 32);
            }
          }
        }
      }
    }
    __syncthreads();

    if (role == 0) {
      // ---- write the page extrema: channel-major rows of this tile's pages
      const int npg = (ntok + S - 1) / S;
      const int pg0 = t0 / S;
      const size_t sbase = (size_t(b) * s.Hkv + g) * kD;
      for (int e = tid; e < kD * npg; e += kMThreads) {
        const int j = e / npg, pl = e % npg;
        store_extrema(s, c, (sbase + j) * s.Pmax + pg0 + pl, stage_f[0][j][pl], stage_f[1][j][pl]);
      }
    } else {
      // ---- exact path for the queued bits, then the code words. 8 lanes per queued bit form
      // the fp64 sum of exact products (16 terms per lane: two 16-byte key loads and 16 W
      // loads, all in flight together), certified as in any summation order; the exact long
      // accumulator decides the rest. If more bits were uncertain than the queue holds
      // (degenerate projections), every word of the tile is recomputed from the stored
      // operands instead: slow, and only for such inputs.
      const float* wbase_p = W + size_t(g) * kD * s.NB + (role - 1) * kD;
      if (fb_n <= kFbCap) {
        const int gl = tid & 7;
        for (int e = tid >> 3; e < fb_n; e += kMThreads / 8) {
          const uint32_t ent = fb_list[e];
          const int tl = int(ent >> 8), lc = int(ent & 0xFFu);
          const uint16_t* kr = Kb + (row0 + t0 + tl) * kD;
          const uint4 k0 = *reinterpret_cast<const uint4*>(kr + 16 * gl);
          const uint4 k1 = *reinterpret_cast<const uint4*>(kr + 16 * gl + 8);
          const float* wc = wbase_p + lc + size_t(16 * gl) * s.NB;
          float wv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) wv[i] = wc[size_t(i) * s.NB];
          const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
          double z = 0.0, sa = 0.0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x =
                __uint_as_float((i & 1) ? (kw[i >> 1] & 0xFFFF0000u) : (kw[i >> 1] << 16));
            const double pr = double(x) * double(wv[i]);
            z += pr;
            sa += fabs(pr);
          }
#pragma unroll
          for (int o = 4; o >= 1; o >>= 1) {
            z += __shfl_xor(z, o, 8);
            sa += __shfl_xor(sa, o, 8);
          }
          if (gl == 0) {
            int cb = certain_bit(z, sa);
            if (cb < 0) cb = int(exact_bit(Bf16Row{kr}, wbase_p + lc, s.NB));
            const uint32_t mask = 1u << (lc & 31);
            if (cb) atomicOr(&stage_c[tl][lc >> 5], mask);
            else atomicAnd(&stage_c[tl][lc >> 5], ~mask);
          }
        }
      } else {
        for (int e = tid; e < ntok * 4; e += kMThreads) {
          const int tl = e >> 2, wd = e & 3;
          const uint16_t* kr = Kb + (row0 + t0 + tl) * kD;
          uint32_t word = 0;
          for (int i = 0; i < 32; ++i)
            word |= certified_bit(Bf16Row{kr}, wbase_p + 32 * wd + i, s.NB) << i;
          stage_c[tl][wd] = word;
        }
      }
      __syncthreads();
      const int wbase = (role - 1) * 4;
      for (int tl = tid; tl < ntok; tl += kMThreads) {
        const uint4 v = make_uint4(stage_c[tl][0], stage_c[tl][1], stage_c[tl][2], stage_c[tl][3]);
        *reinterpret_cast<uint4*>(c.codes + (row0 + t0 + tl) * s.NW + wbase) = v;
      }
    }
    __syncthreads();   // this tile's LDS staging is read out before the next tile reuses it
  }
}

hipError_t launch_build_mfma(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st) {
  const int ntiles = (s.Lmax + kMTok - 1) / kMTok;
  const int nroles = 1 + s.NB / kD;
  // The LDS staging (about 156 KB) keeps one workgroup per CU, so the build takes
  // ceil(workgroups / CUs) rounds of ceil(ntiles / nper) tiles each. nper is the split with the
  // fewest tiles in sequence, counting one tile for each round's B staging, among the splits
  // of at least 4 rounds (measured on MI355X at 128K: 4 rounds of 4 tiles 340 us, 1 round of
  // 16 tiles 372 us; sequences shorter than max_seq_len also leave room to rebalance); among
  // equals the fewest workgroups (fewest stagings).
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    ncu = 256;
  const long long units = (long long)nroles * s.Hkv * s.B;
  int nper = 1;
  long long best = -1;
  for (int n = 1; n <= ntiles; ++n) {
    const long long rounds = (units * n + ncu - 1) / ncu;
    const long long cost = rounds * ((ntiles + n - 1) / n + 1);
    if (rounds < 4 && n < ntiles) continue;
    if (best < 0 || cost < best) {
      best = cost;
      nper = n;
    }
  }
  dim3 grid(nper * nroles, s.Hkv, s.B);
  const KernelTimer none{nullptr, nullptr};
  if (s.S == 16)
    return launch_kernel("build_mfma_kernel",
                         build_mfma_kernel<16>, grid, dim3(kMThreads), st, none, s, c, R, W,
                         ntiles, nper);
  return launch_kernel("build_mfma_kernel",
                       build_mfma_kernel<32>, grid, dim3(kMThreads), st, none, s, c, R, W, ntiles,
                       nper);
}

}  // namespace hhr
