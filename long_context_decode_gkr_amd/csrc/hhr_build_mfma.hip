// Index build on the matrix cores (MFMA) for bf16 keys.
//
// Method: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", §3.3.1 (page extrema of
// the rotated keys k~ = k R, Eq. 4) and §3.1 Eq. 1 / §3.3.2 Eq. 10 (key code = sign of z = k W).
// Both are products of the key tile with R_g and W_g, done with v_mfma_f32_32x32x16_bf16.
//
// Precision. The keys are bf16, so they are exact MFMA operands. The fp32 R and W are split into
// bf16 pieces by round-to-nearest (8-bit significands, so each piece leaves at most 2^-8 of
// what it splits): R = r1 + r2 + r3 exactly, W = w1 + w2 to 2^-16 relative; every
// bf16 x bf16 product is exact in fp32 and the MFMA accumulates in fp32.
//   * Rotation: k~ carries fp32 accumulation error only (a few ulps of |k|); the page extrema
//     are taken from it.
//   * Codes: a code column w_c is first scaled by the power of two that brings |w_c| into
//     [1, 2) (exact; the sign of k w_c is unchanged). z then differs from the exact k w_c by at
//     most 256 * 2^-23 + 2^-16 <= 2^-14.4 times |k|_2 |w_c|_2 (256 additions, each rounding at
//     most 2^-23 of a partial sum bounded by sum |k_i w_i| <= |k|_2 |w_c|_2 by Cauchy-Schwarz,
//     in any order; plus the dropped third piece of W), so a bit is certain when
//     |z| > tau = 2^-13 |k|_2 >= 2^-14 |k|_2 |w_c|_2. The other bits (about 8e-4 of them for
//     Gaussian data) are queued in LDS and recomputed from the stored operands in fp64 (exact
//     products), with the exact long accumulator behind that: every code equals the sign of
//     the exact z.
//
// One workgroup reads each key once for both products. Its waves own output columns and keep
// their pieces of R_g or W_g in registers for the whole launch; the keys pass through LDS:
//   * rotation waves (with ROT, the even ones): channels 32 (w / 2) .. + 31, the 3 R pieces as
//     MFMA B
//     fragments, the key sub-tile as A, so a lane holds one channel of 16 tokens and the page
//     extrema are minima / maxima over its own registers;
//   * code waves: code columns coff + 32 v .. + 31 (v the code wave's index), the 2 W pieces as
//     MFMA A fragments, the keys as B, so a lane holds 16 code columns of one token and
//     assembles its bits without any cross-lane vote.
// Grid (nper, Hkv, ceil(B / 64)): the 512-token chunks of KV head g of a group of at most 64
// sequences form one list (sequence by sequence, in order), and workgroup `first` builds its
// entries first, first + nper, ..., so the workgroups of a batch of unequal lengths get equal
// shares (one workgroup per sequence and KV head had left the longest sequence's workgroups
// with 14 chunks against 10 at 8 sequences of 8K-32K tokens); the key rows stream through two LDS buffers of 128 rows (the next tile's
// global loads in flight while the current one is multiplied), each staged row with its norm.
// 256-bit codes take a second launch for code columns 128..255 without rotation waves: 8 code
// waves, two per 32-column block, each taking half of every tile's rows (4 waves over all the
// rows had left one wave per SIMD: 667 -> 582 us for the Qwen3-8B-shaped layer's build).
#include "hhr_device.h"
#include "hhr_launch.h"

namespace hhr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 512;           // tokens per output chunk (page extrema, code words)
constexpr int kKTile = 128;           // key rows per LDS tile (4 sub-tiles of 32)
constexpr int kKRow = kD + 8;         // bf16 elements per staged row: 272 B, so that the 16-byte
                                      // fragment reads of 32 consecutive rows hit distinct banks
constexpr int kCodeWaves = 4;         // 128 code columns per launch
constexpr int kFbCap = 4096;          // queued uncertain code bits per workgroup
constexpr int kSeqGroup = 64;         // sequences whose chunks one list covers (one per lane)
constexpr float kCertScale = 1.0f / 8192.0f;   // 2^-13

// One stored bf16 key row, read as fp32 values.
struct Bf16Row {
  const uint16_t* p;
  __device__ __forceinline__ float operator[](int j) const { return bf16_bits_to_f32(p[j]); }
};

template <bool ROT>
constexpr int build_threads() { return kWave * 8; }   // 4 rotation + 4 code waves, or 8 code
// Code waves of a launch: 4 (with rotation), else 8, two per code block, each taking half of a
// tile's rows (so that every SIMD runs two waves)
template <bool ROT>
constexpr int code_waves() { return ROT ? kCodeWaves : 2 * kCodeWaves; }

// Row of the accumulator element r of a 32 x 32 MFMA tile held by a lane of half 0 (half 1:
// + 4): 8 (r / 4) + r % 4.
__device__ __forceinline__ constexpr int acc_row(int r) { return 8 * (r / 4) + (r % 4); }

template <int S, bool ROT>
__global__ void __launch_bounds__(build_threads<ROT>())
build_mfma_kernel(Shape s, CacheView c, const float* __restrict__ R, const float* __restrict__ W,
                  int coff, int nper) {
  constexpr int NT = build_threads<ROT>();
  constexpr int RW = ROT ? 4 : 0;                 // rotation waves
  constexpr int KPT = kKTile * (kD / 8) / NT;     // 16-byte key pieces per thread per tile
  static_assert(KPT * NT == kKTile * (kD / 8), "whole tiles");
  const int first = blockIdx.x, g = blockIdx.y, grp = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  // lane l of every wave: the length of sequence 64 grp + l (0 past the batch), its chunk count
  // and the number of chunks up to and including it, so that the sequence of list entry f is
  // the number of lanes whose inclusive count is at most f (one ballot)
  const int bl = kSeqGroup * grp + lane;
  const int lenl = bl < s.B ? min(max(c.seq_lens[bl], 0), s.Lmax) : 0;
  const int nchl = (lenl + kChunk - 1) / kChunk;
  const int cincl = wave_incl_sum(nchl);
  const int ntot = __builtin_amdgcn_readlane(cincl, kWave - 1);
  if (first >= ntot) return;
  // with rotation waves, even waves rotate (channel block w / 2) and odd waves hash (code
  // block w / 2): consecutive waves share a SIMD, so each SIMD runs one wave of each kind
  // (measured 227 -> 209 us at 128K against waves 0..3 rotating)
  const bool rot = RW > 0 && (w & 1) == 0;
  const int half = lane >> 5, col = lane & 31;
  const int cw = RW > 0 ? (w >> 1) : (w & 3);    // code block (code waves)
  const int rh = RW > 0 ? 0 : (w >> 2);          // without rotation: the half of the rows
  constexpr int NCW = code_waves<ROT>();
  const int seg = RW > 0 ? cw : w;               // the code wave's queue segment

  __shared__ __align__(16) uint16_t Kt[2][kKTile][kKRow];
  __shared__ float knorm[2][kKTile];              // 2^-13 |k| of the staged rows (inf if tiny)
  // page min / max (rotation): rows padded by one word so that the 32 channels a wave writes
  // at once fall in different banks
  __shared__ float stage_f[ROT ? 2 : 1][ROT ? kD : 1][kChunk / S + 1];
  __shared__ uint32_t stage_c[kChunk][kCodeWaves + 1];   // code words, padded rows
  // queued uncertain bits (row of K, column), one segment of kSeg per code wave, and each
  // wave's count (which may pass kSeg: the rest is lost, see the drain). A row index is below
  // 2^32 for any K cache under 1 TiB.
  constexpr int kSeg = kFbCap / NCW;
  __shared__ uint2 fb_list[kFbCap];
  __shared__ int fb_cnt[NCW];
  if (tid < NCW) fb_cnt[tid] = 0;                 // published by the first staging barrier
  int qn = 0;                                     // this code wave's count (uniform)

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(c.K);
  // list entry f: its sequence, the chunk's index in it and the sequence's length (uniform)
  struct ChunkPos { int f, b, ch, L; };
  auto locate = [&](int f) {
    const int l = int(__popcll(__ballot(cincl <= f)));   // < 64 since f < ntot
    ChunkPos p;
    p.f = f;
    p.b = kSeqGroup * grp + l;
    p.ch = f - (__builtin_amdgcn_readlane(cincl, l) - __builtin_amdgcn_readlane(nchl, l));
    p.L = __builtin_amdgcn_readlane(lenl, l);
    return p;
  };
  auto kv_row0 = [&](const ChunkPos& p) { return (size_t(p.b) * s.Hkv + g) * s.Lmax; };
  auto chunk_tiles = [&](const ChunkPos& p) {
    return min(kChunk / kKTile, (p.L - p.ch * kChunk + kKTile - 1) / kKTile);
  };

  // ---- key tile staging: thread piece e = tid + i NT is row e / 16, bytes 16 (e % 16) .. + 15;
  // rows past the end repeat the last valid row
  uint4 kv[KPT];
  auto load_tile = [&](size_t row0, int L, int t0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + i * NT;
      const int t = min(t0 + (e >> 4), L - 1);
      kv[i] = *reinterpret_cast<const uint4*>(Kb + (row0 + t) * kD + (e & 15) * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + i * NT;
      *reinterpret_cast<uint4*>(&Kt[buf][e >> 4][(e & 15) * 8]) = kv[i];
      // the row's squared norm over its 16 pieces (16 consecutive lanes), rounded up
      float q = 0.f;
      q = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv[i].x),
                                          __builtin_bit_cast(bf16x2, kv[i].x), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv[i].y),
                                          __builtin_bit_cast(bf16x2, kv[i].y), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv[i].z),
                                          __builtin_bit_cast(bf16x2, kv[i].z), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv[i].w),
                                          __builtin_bit_cast(bf16x2, kv[i].w), q, false);
      q = row16_sum(q);
      if ((e & 15) == 0) {
        const float n = sqrtf(q) * (1.0f + 0x1p-10f);
        knorm[buf][e >> 4] = n > 1e-15f ? n * kCertScale : INFINITY;
      }
    }
  };
  ChunkPos cp = locate(first);                    // the chunk being built
  int tq = 0;                                     // its tile
  load_tile(kv_row0(cp), cp.L, cp.ch * kChunk);

  // ---- stationary operand pieces (bf16, hardware round-to-nearest-even): lane (half, col)
  // holds rows 16 ks + 8 half .. + 7 of column `col` of its 32-column block, for ks = 0..7.
  // A code column is first scaled by the power of two 2^-e that brings its norm into [1, 2)
  // (exact, and sign(k w_c 2^-e) = sign(k w_c)), so that the certainty test needs no per-column
  // factor: |z| > 2^-13 |k| >= 2^-14 |k| |w_c 2^-e|. Columns of tiny norm (below 1e-15) or of
  // norm 2^126 and above are never certain.
  bf16x8 frag[3][8];
  uint32_t tiny_mask = 0;                          // code waves: never-certain bit positions
  {
    const float* src = rot ? R + size_t(g) * kD * kD + 32 * (w >> 1) + col
                           : W + size_t(g) * kD * s.NB + coff + 32 * cw + col;
    const int ld = rot ? kD : s.NB;
    // the lane's 64 values (rows 16 ks + 8 half + e), loaded once for the norm and the pieces
    float xv[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[ks][e] = src[size_t(16 * ks + 8 * half + e) * ld];
    float scale = 1.0f;
    if (!rot) {
      // |w_c| from fp32 sums of squares (relative error below 2^-16), rounded up by 2^-14
      float nrm = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) nrm = fmaf(xv[i >> 3][i & 7], xv[i >> 3][i & 7], nrm);
      nrm += lane_xor(nrm, 32);
      const float wn = sqrtf(nrm) * (1.0f + 0x1p-14f);
      const uint32_t be = (__float_as_uint(wn) >> 23) & 0xFFu;   // wn in [2^(be-127), 2^(be-126))
      const bool tiny = !(wn > 1e-15f) || be >= 253u;
      scale = tiny ? 1.0f : __uint_as_float((254u - be) << 23);   // 2^-(be - 127)
      const uint64_t tb = __ballot(tiny);                          // lanes 0..31: columns
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tiny_mask |= uint32_t((tb >> (acc_row(r) + 4 * half)) & 1u) << (acc_row(r) + 4 * half);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = xv[ks][e] * scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 p1 = __bf16(x[e]);
        const float r1 = x[e] - float(p1);
        const __bf16 p2 = __bf16(r1);
        frag[0][ks][e] = p1;
        frag[1][ks][e] = p2;
        frag[2][ks][e] = __bf16(r1 - float(p2));
      }
    }
  }
  store_tile(0);
  __syncthreads();

  const uint32_t pos_mask = 0x0F0F0F0Fu << (4 * half);   // the code bits a lane's half holds
  const int NWd = s.NB / 32;
  const float* wcols = W + size_t(g) * kD * s.NB;       // column c at wcols + c, stride NB

  // Exact path for the queued bits, after every code word written so far has completed (the
  // corrections are device atomics on those words). The launch's 128 fp32 columns of W are
  // staged transposed in the key buffers (free at that point), then 4 lanes per queued bit form
  // the fp64 sum of exact products (32 terms per lane: four 16-byte key loads, all in flight
  // together), certified as in any summation order; the exact long accumulator decides the
  // rest. Called by every thread; the caller re-stages a key tile afterwards if one is pending.
  constexpr int kWTs = kD + 1;                    // staged row stride: conflict-free transposes
  static_assert(sizeof(Kt) >= sizeof(float) * kD * kWTs, "W^T fits in the key buffers");
  // Every load of a thread's share of W, and of a pass's two entries, is issued before any of
  // them is used (a loop that stored each value as it arrived took one memory round trip per
  // value).
  constexpr int kWPer = kD * kD / NT;              // staged W values per thread
  constexpr int kWBatch = kWPer < 32 ? kWPer : 32;
  static_assert(kWPer % kWBatch == 0, "whole batches");
  constexpr int kEnt = 2;                          // queued entries per 4 lanes per pass
  auto drain_queue = [&](int nseg, size_t row_any) {   // nseg entries from each wave's segment;
                                                         // row_any: a valid row of K
    const int n = nseg * NCW;
    float* WT = reinterpret_cast<float*>(&Kt[0][0][0]);   // WT[c * kWTs + k] = W[k][coff + c]
    {
      // value tid + j NT is W[(tid >> 7) + j NT / 128][coff + tid % 128]; the thread's offsets
      // are formed here (materialized), not hoisted into the setup where they would stay live
      // through the whole launch
      const int gofs = materialize(int((tid >> 7) * s.NB + coff + (tid & (kD - 1))));
      const int lofs = materialize(int((tid & (kD - 1)) * kWTs + (tid >> 7)));
#pragma unroll 1
      for (int j0 = 0; j0 < kWPer; j0 += kWBatch) {
        float wv[kWBatch];
#pragma unroll
        for (int j = 0; j < kWBatch; ++j)
          wv[j] = wcols[gofs + size_t(j0 + j) * (NT / kD) * s.NB];
#pragma unroll
        for (int j = 0; j < kWBatch; ++j) WT[lofs + (j0 + j) * (NT / kD)] = wv[j];
      }
    }
    __syncthreads();
    const int q = tid & 3;
    for (int e0 = tid >> 2; e0 < n; e0 += kEnt * (NT / 4)) {   // the 4 lanes of an entry agree
      bool ok[kEnt];
      uint2 ent[kEnt];
#pragma unroll
      for (int j = 0; j < kEnt; ++j) {
        const int e = min(e0 + j * (NT / 4), n - 1);
        const int sg = e / nseg, se = e % nseg;
        ok[j] = e0 + j * (NT / 4) < n && se < min(fb_cnt[sg], kSeg);   // else a shorter segment
        ent[j] = ok[j] ? fb_list[sg * kSeg + se]
                       : make_uint2(uint32_t(row_any), uint32_t(coff));   // else a dummy
      }
      uint4 kq[kEnt][4];
#pragma unroll
      for (int j = 0; j < kEnt; ++j) {
        const uint16_t* kr = Kb + size_t(ent[j].x) * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i) kq[j][i] = *reinterpret_cast<const uint4*>(kr + 32 * q + 8 * i);
      }
#pragma unroll
      for (int j = 0; j < kEnt; ++j) {
        const size_t row = ent[j].x;
        const int cc = int(ent[j].y);
        const float* wq = WT + (cc - coff) * kWTs + 32 * q;
        double z = 0.0, sa = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t kw = (&kq[j][i >> 2].x)[i & 3];
          const double p0 = double(__uint_as_float(kw << 16)) * double(wq[2 * i]);
          const double p1 = double(__uint_as_float(kw & 0xFFFF0000u)) * double(wq[2 * i + 1]);
          z += p0;
          sa += fabs(p0);
          z += p1;
          sa += fabs(p1);
        }
        z = group_sum_f64<2>(z);
        sa = group_sum_f64<2>(sa);
        if (q == 0 && ok[j]) {
          const uint16_t* kr = Kb + row * kD;
          int cb = certain_bit(z, sa);
          if (cb < 0) cb = int(exact_bit(Bf16Row{kr}, wcols + cc, s.NB));
          uint32_t* word = c.codes + row * NWd + (cc >> 5);
          const uint32_t mask = 1u << (cc & 31);
          if (cb) atomicOr(word, mask);
          else atomicAnd(word, ~mask);
        }
      }
    }
  };

  for (int T = 0;; ++T) {
    const size_t row0 = kv_row0(cp);              // row of token 0 of the chunk's (b, g)
    const int L = cp.L;
    const int cbase = cp.ch * kChunk;
    const int t0 = cbase + tq * kKTile;           // < L
    const int tc = t0 - cbase;                    // the tile's first token within its chunk
    // the next tile: this chunk's next one, else the first of the workgroup's next chunk
    const bool chunk_done = tq + 1 >= chunk_tiles(cp);
    const bool more = !chunk_done || cp.f + nper < ntot;
    const ChunkPos np = chunk_done && more ? locate(cp.f + nper) : cp;
    const int nq = chunk_done ? 0 : tq + 1;
    if (more) load_tile(kv_row0(np), np.L, np.ch * kChunk + nq * kKTile);   // in flight during
                                                                             // the products
    const int buf = T & 1;

    // ---- products: sub-tiles (2 sp, 2 sp + 1) of 32 rows, two accumulators in flight; the
    // role is uniform over the wave, and each role's loop is straight-line code of its own
    auto load_kf = [&](int sp, int ks, bf16x8 (&kf)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        kf[u] = *reinterpret_cast<const bf16x8*>(
            &Kt[buf][32 * (2 * sp + u) + col][16 * ks + 8 * half]);
    };
    if (rot) {
      if constexpr (ROT) {
#pragma unroll 1
        for (int sp = 0; sp < 2; ++sp) {
          f32x16 acc[2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            bf16x8 kf[2];
            load_kf(sp, ks, kf);
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
              for (int u = 0; u < 2; ++u)
                acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[u], frag[p][ks], acc[u], 0, 0,
                                                                 0);
          }
          // page extrema of channel 32 w + col over each sub-tile's rows (pages of 16 or 32
          // rows): rows past the end repeat the last valid row, of the same page, and pages
          // with no valid row are not written out
          const int j = 32 * (w >> 1) + col;
          constexpr int PPS = 32 / S;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int tl0 = 32 * (2 * sp + u);
#pragma unroll
            for (int pp = 0; pp < PPS; ++pp) {
              float lo = INFINITY, hi = -INFINITY;
#pragma unroll
              for (int r = pp * (16 / PPS); r < (pp + 1) * (16 / PPS); ++r) {
                lo = fminf(lo, acc[u][r]);
                hi = fmaxf(hi, acc[u][r]);
              }
              lo = fminf(lo, lane_from_above(lo, 32));   // lanes 0-31 store
              hi = fmaxf(hi, lane_from_above(hi, 32));
              if (half == 0) {
                stage_f[0][j][(tc + tl0) / S + pp] = lo;
                stage_f[1][j][(tc + tl0) / S + pp] = hi;
              }
            }
          }
        }
      }
    } else {
#pragma unroll 1
      for (int sp = ROT ? 0 : rh; sp < (ROT ? 2 : rh + 1); ++sp) {
        f32x16 acc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          bf16x8 kf[2];
          load_kf(sp, ks, kf);
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int u = 0; u < 2; ++u)
              acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[p][ks], kf[u], acc[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          // ---- code bits of token t0 + tl0 + col, columns coff + 32 cw + acc_row(r) + 4 half:
          // sign bits, and certainty |z| > 2^-13 |k| |w_c|
          const int tl0 = 32 * (2 * sp + u);
          const float tau = knorm[buf][tl0 + col];
          uint32_t neg = 0, sure = 0;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float z = acc[u][r];
            neg |= (__float_as_uint(z) >> 31) << acc_row(r);
            sure |= (fabsf(z) > tau) ? (1u << acc_row(r)) : 0u;
          }
          neg <<= 4 * half;
          sure <<= 4 * half;
          uint32_t word = ~neg & pos_mask;
          word |= lane_from_above_u(word, 32);   // lanes 0-31 store
          const int t = t0 + tl0 + col;
          uint32_t uns = t < L ? (~sure | tiny_mask) & pos_mask : 0u;
          // queue the uncertain bits in the wave's own segment, each lane at its prefix (no
          // atomics; skipped when no lane has one)
          if (__ballot(uns != 0u)) {
            const int nu = __popc(uns);
            const int incl = wave_incl_sum(nu);
            int pos = qn + incl - nu;
            qn += __builtin_amdgcn_readlane(incl, 63);
            while (uns) {
              const int bi = __builtin_ctz(uns);
              uns &= uns - 1;
              if (pos < kSeg)
                fb_list[seg * kSeg + pos] =
                    make_uint2(uint32_t(row0 + t), uint32_t(coff + 32 * cw + bi));
              ++pos;
            }
          }
          if (half == 0) stage_c[tc + tl0 + col][cw] = word;
        }
      }
    }
    if (!rot && lane == 0) fb_cnt[seg] = qn;
    if (more) store_tile(buf ^ 1);
    __syncthreads();

    if (chunk_done) {
      // ---- the chunk is complete: write its page extrema and code words out (certain bits
      // final; the queued ones are decided by the exact path)
      const int ntok = min(kChunk, L - cbase);
      if constexpr (ROT) {
        constexpr int PPC = kChunk / S;           // pages per chunk
        const int npg = (ntok + S - 1) / S;
        const int pg0 = cbase / S;
        const size_t sbase = (size_t(cp.b) * s.Hkv + g) * kD;
        for (int e = tid; e < kD * PPC; e += NT) {
          const int j = e / PPC, pl = e % PPC;
          if (pl < npg)
            store_extrema(s, c, (sbase + j) * s.Pmax + pg0 + pl, stage_f[0][j][pl],
                          stage_f[1][j][pl]);
        }
      }
      for (int tl = tid; tl < ntok; tl += NT) {
        const uint4 v = make_uint4(stage_c[tl][0], stage_c[tl][1], stage_c[tl][2], stage_c[tl][3]);
        *reinterpret_cast<uint4*>(c.codes + (row0 + cbase + tl) * NWd + coff / 32) = v;
      }
      // ---- drain the queue when a segment is 3/4 full, and at the end. Entries past a
      // segment's capacity (more uncertain bits in one chunk than it holds: degenerate
      // projections) are lost; then every word of this chunk is recomputed from the stored
      // operands instead (slow, only for such inputs).
      int nfb = 0;
#pragma unroll
      for (int i = 0; i < NCW; ++i) nfb = max(nfb, fb_cnt[i]);
      if (nfb >= 3 * kSeg / 4 || !more) {
        wait_memory();
        __syncthreads();
        drain_queue(min(nfb, kSeg), row0);
        if (nfb > kSeg) {
          wait_memory();
          __syncthreads();
          for (int e = tid; e < ntok * kCodeWaves; e += NT) {
            const int tl = e >> 2, wd = e & 3;
            const uint16_t* kr = Kb + (row0 + cbase + tl) * kD;
            uint32_t word = 0;
            for (int i = 0; i < 32; ++i)
              word |= certified_bit(Bf16Row{kr}, wcols + coff + 32 * wd + i, s.NB) << i;
            c.codes[(row0 + cbase + tl) * NWd + coff / 32 + wd] = word;
          }
        }
        __syncthreads();
        if (tid < NCW) fb_cnt[tid] = 0;
        qn = 0;
        if (more) store_tile((T + 1) & 1);        // the drain used the key buffers
      }
      __syncthreads();   // the chunk's LDS staging is read out before the next chunk reuses it
    }
    if (!more) break;
    cp = np;
    tq = nq;
  }
}

hipError_t launch_build_mfma(const Shape& s, const CacheView& c, const float* R, const float* W,
                             hipStream_t st) {
  // about one workgroup per CU (about 144 KB of LDS each): nper workgroups per (KV head, group
  // of 64 sequences), each building every nper-th entry of the group's list of chunks
  const int nch = (s.Lmax + kChunk - 1) / kChunk;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    ncu = 256;
  const int ngrp = (s.B + kSeqGroup - 1) / kSeqGroup;
  const int units = s.Hkv * ngrp;
  const int nper = std::max(1, std::min(std::min(s.B, kSeqGroup) * nch, (ncu + units - 1) / units));
  const dim3 grid(nper, s.Hkv, ngrp);
  const KernelTimer none{nullptr, nullptr};
  hipError_t e;
  if (s.S == 16)
    e = launch_kernel("build_mfma_kernel", build_mfma_kernel<16, true>, grid,
                      dim3(build_threads<true>()), st, none, s, c, R, W, 0, nper);
  else
    e = launch_kernel("build_mfma_kernel", build_mfma_kernel<32, true>, grid,
                      dim3(build_threads<true>()), st, none, s, c, R, W, 0, nper);
  if (e != hipSuccess || s.NB == 128) return e;
  // code columns 128 .. 255
  if (s.S == 16)
    return launch_kernel("build_mfma_kernel", build_mfma_kernel<16, false>, grid,
                         dim3(build_threads<false>()), st, none, s, c, R, W, 128, nper);
  return launch_kernel("build_mfma_kernel", build_mfma_kernel<32, false>, grid,
                       dim3(build_threads<false>()), st, none, s, c, R, W, 128, nper);
}

}  // namespace hhr
