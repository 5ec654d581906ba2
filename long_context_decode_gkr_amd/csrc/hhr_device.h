// Device-side helpers shared by the HHR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "hhr_launch.h"

namespace hhr {

constexpr int kD = 128;         // head dimension
constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// Element loads: K, V, q are fp32 or bf16; everything is computed in fp32 / fp64.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// bf16 rounded toward -inf / +inf (bits). A page minimum stored rounded down and a maximum
// stored rounded up keep max(q l, q u) >= the exact value, so the page bound stays an upper
// bound. The fp32 value truncated to its top 16 bits is rounded toward zero; an inexact value
// on the wrong side of zero takes one more bf16 step away from zero.
__device__ __forceinline__ uint32_t bf16_round_down(float x) {
  const uint32_t u = __float_as_uint(x), t = u & 0xFFFF0000u;
  return (t != u && x < 0.f ? t + 0x10000u : t) >> 16;
}
__device__ __forceinline__ uint32_t bf16_round_up(float x) {
  const uint32_t u = __float_as_uint(x), t = u & 0xFFFF0000u;
  return (t != u && x > 0.f ? t + 0x10000u : t) >> 16;
}

// Page extrema element i of the cache: read as fp32; written from fp32 values (as bf16 rounded
// outward when the cache stores bf16 extrema).
__device__ __forceinline__ float load_pmin(const Shape& s, const CacheView& c, size_t i) {
  return s.sum_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(c.pmin)[i])
                    : static_cast<const float*>(c.pmin)[i];
}
__device__ __forceinline__ float load_pmax(const Shape& s, const CacheView& c, size_t i) {
  return s.sum_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(c.pmax)[i])
                    : static_cast<const float*>(c.pmax)[i];
}
__device__ __forceinline__ void store_extrema(const Shape& s, const CacheView& c, size_t i,
                                              float lo, float hi) {
  if (s.sum_bf16) {
    static_cast<uint16_t*>(c.pmin)[i] = uint16_t(bf16_round_down(lo));
    static_cast<uint16_t*>(c.pmax)[i] = uint16_t(bf16_round_up(hi));
  } else {
    static_cast<float*>(c.pmin)[i] = lo;
    static_cast<float*>(c.pmax)[i] = hi;
  }
}

// Raw 16- or 32-bit element load; convert with raw_to_f32 after the other loads are issued so
// that the conversion's wait does not sit in front of them.
__device__ __forceinline__ uint32_t load_raw(const void* base, size_t i, int is_bf16) {
  return is_bf16 ? uint32_t(reinterpret_cast<const uint16_t*>(base)[i])
                 : reinterpret_cast<const uint32_t*>(base)[i];
}
__device__ __forceinline__ float raw_to_f32(uint32_t r, int is_bf16) {
  return is_bf16 ? __uint_as_float(r << 16) : __uint_as_float(r);
}

__device__ __forceinline__ float load_elem(const void* base, size_t i, int is_bf16) {
  if (is_bf16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  return reinterpret_cast<const float*>(base)[i];
}

// ---------------------------------------------------------------------------------------------
// Exact sign of a dot product of finite fp32 values (the code bit of §3.1 Eq. 1 is defined on
// the exact real value of z = x . w).
//
// Every finite fp32 value is m * 2^(e - 150) with an integer m < 2^24 and e in [1, 254]
// (subnormals: e = 1). A product is then a 48-bit integer times 2^(ea + eb - 300), i.e. the
// integer placed at bit ea + eb - 2 >= 0 of a fixed-point number whose unit is 2^-298. The
// accumulator keeps that number in 18 signed 64-bit limbs of 32 bits each (576 bits, enough
// for 128 products of at most 2^555 plus a sign); carries are resolved once at the end.
// ---------------------------------------------------------------------------------------------
struct LongAcc {
  int64_t limb[18];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < 18; ++i) limb[i] = 0;
  }
  __device__ __forceinline__ void add_product(float a, float b) {
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    uint32_t ea = (ua >> 23) & 0xFFu, eb = (ub >> 23) & 0xFFu;
    uint64_t ma = ua & 0x7FFFFFu, mb = ub & 0x7FFFFFu;
    if (ea) ma |= 0x800000u; else ea = 1;
    if (eb) mb |= 0x800000u; else eb = 1;
    const uint64_t m = ma * mb;
    const int sh = int(ea + eb) - 2;
    const int li = sh >> 5, bs = sh & 31;
    const uint64_t t0 = (m & 0xFFFFFFFFull) << bs;
    const uint64_t t1 = (m >> 32) << bs;
    int64_t c0 = int64_t(t0 & 0xFFFFFFFFull);
    int64_t c1 = int64_t((t0 >> 32) + (t1 & 0xFFFFFFFFull));
    int64_t c2 = int64_t(t1 >> 32);
    if ((ua ^ ub) >> 31) { c0 = -c0; c1 = -c1; c2 = -c2; }
    // limbs li, li + 1, li + 2 receive c0, c1, c2; unrolled selects keep the limbs in
    // registers (a runtime index would place them in scratch memory)
#pragma unroll
    for (int i = 0; i < 18; ++i)
      limb[i] += (i == li) ? c0 : (i == li + 1) ? c1 : (i == li + 2) ? c2 : 0;
  }
  // +1, 0 or -1.
  __device__ __forceinline__ int sign() {
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      const int64_t carry = limb[i] >> 32;  // floor division by 2^32
      limb[i] -= carry * 4294967296ll;
      limb[i + 1] += carry;
    }
    int sg = limb[17] > 0 ? 1 : (limb[17] < 0 ? -1 : 0);
#pragma unroll
    for (int i = 16; i >= 0; --i) sg = (sg == 0 && limb[i] != 0) ? 1 : sg;
    return sg;
  }
};

// Certainty test for a code bit from an fp64 sum z of exact products and the fp64 sum s of
// their magnitudes (n <= 128 terms, any summation order): |z - exact| <= gamma_n * sum|p|, so
// the sign of z is the exact sign when |z| > 4 * 128 * 2^-53 * s (the factor also covers the
// rounding of s). Returns 1 or 0 when certain, -1 when the exact path must decide.
__device__ __forceinline__ int certain_bit(double z, double s) {
  const double tau = s * (double(kD) * 0x1p-51);
  if (z > tau) return 1;
  if (z < -tau || s == 0.0) return 0;
  return -1;
}

// Certainty test for a code bit from fp32 sums over 128 products p_i = x_i w_i, computed as
// 8 lanes of 16 fused multiply-adds in index order (the first with a zero addend) combined by
// a 3-level tree: z = sum p_i, s = sum |p_i|. Along any path a product meets 19 roundings and
// no other error (inside an FMA the product is exact), so |z - exact| <= gamma_19 sum|p| with
// gamma_19 = 19 u / (1 - 19 u), u = 2^-24, i.e. below 1.2e-6 sum|p|, and s differs from sum|p|
// by the same relative amount; tau = 2^-19 s (1.9e-6 s) covers both, and 2^-140 covers the
// absolute error of underflowing additions (each below 2^-150). Returns 1 / 0 when the sign of
// z is certain, -1 otherwise (also for s == 0, whose products may have underflowed, and for
// an overflow to inf or NaN, where both comparisons fail).
__device__ __forceinline__ int certain_bit_f32(float z, float s) {
  const float tau = s * 0x1p-19f + 0x1p-140f;
  if (s > 0.f && z > tau) return 1;
  if (s > 0.f && z < -tau) return 0;
  return -1;
}

// Exact code bit [sum_j x[j] * w[j * w_stride] > 0] (j < 128); x: fp32 values through any
// indexable accessor, w: fp32 in global memory.
template <typename XPtr>
__device__ __forceinline__ uint32_t exact_bit(XPtr xs, const float* __restrict__ w, int w_stride) {
  LongAcc acc;
  acc.clear();
  for (int j = 0; j < kD; ++j) acc.add_product(float(xs[j]), w[size_t(j) * w_stride]);
  return acc.sign() > 0 ? 1u : 0u;
}

// Code bit of z = x . w computed in fp64 (exact products), certified, exact where needed.
template <typename XPtr>
__device__ __forceinline__ uint32_t certified_bit(XPtr xs, const float* __restrict__ w,
                                                  int w_stride) {
  double z = 0.0, s = 0.0;
#pragma unroll 8
  for (int j = 0; j < kD; ++j) {
    double p = double(xs[j]) * double(w[size_t(j) * w_stride]);
    z += p;
    s += fabs(p);
  }
  int c = certain_bit(z, s);
  if (c >= 0) return uint32_t(c);
  return exact_bit(xs, w, w_stride);
}

// Strided view of fp32 values (e.g. one column of a transposed tile in LDS).
struct Strided {
  const float* p;
  int stride;
  __device__ __forceinline__ float operator[](int j) const { return p[j * stride]; }
};

// ---------------------------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The value x, computed by every lane at this point: an empty asm statement with x as an
// in/out VGPR operand, which keeps the compiler from sinking x's computation (a load, an LDS
// read) into a branch when x is only used under a condition. No instruction is emitted.
template <class T>
__device__ __forceinline__ T materialize(T x) {
  static_assert(sizeof(T) == 4, "one VGPR");
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// ---- DPP (data-parallel primitives): cross-lane moves at ALU latency, no LDS round trip.
// Controls (gfx9 encoding): quad_perm, row_shr:n = 0x110 + n, row_mirror = 0x140,
// row_half_mirror = 0x141, row_bcast:15 = 0x142, row_bcast:31 = 0x143. Lanes whose source is
// outside the row keep `old` (bound_ctrl off), which the scans set to the identity.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += dpp_i<0x111>(0, v);
  v += dpp_i<0x112>(0, v);
  v += dpp_i<0x114>(0, v);
  v += dpp_i<0x118>(0, v);
  v += dpp_i<0x142, 0xa>(0, v);
  v += dpp_i<0x143, 0xc>(0, v);
  return v;
}

// Inclusive prefix sum within each row of 16 lanes.
__device__ __forceinline__ int row16_incl_sum(int v) {
  v += dpp_i<0x111>(0, v);
  v += dpp_i<0x112>(0, v);
  v += dpp_i<0x114>(0, v);
  v += dpp_i<0x118>(0, v);
  return v;
}

// Sum / min / max over the wave, returned in every lane (through lane 63).
__device__ __forceinline__ int wave_total(int v) {
  return __builtin_amdgcn_readlane(wave_incl_sum(v), 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int big = int(0xFFFFFFFFu);
  v = min(v, uint32_t(dpp_i<0x111>(big, int(v))));
  v = min(v, uint32_t(dpp_i<0x112>(big, int(v))));
  v = min(v, uint32_t(dpp_i<0x114>(big, int(v))));
  v = min(v, uint32_t(dpp_i<0x118>(big, int(v))));
  v = min(v, uint32_t(dpp_i<0x142, 0xa>(big, int(v))));
  v = min(v, uint32_t(dpp_i<0x143, 0xc>(big, int(v))));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(dpp_i<0x111>(0, int(v))));
  v = max(v, uint32_t(dpp_i<0x112>(0, int(v))));
  v = max(v, uint32_t(dpp_i<0x114>(0, int(v))));
  v = max(v, uint32_t(dpp_i<0x118>(0, int(v))));
  v = max(v, uint32_t(dpp_i<0x142, 0xa>(0, int(v))));
  v = max(v, uint32_t(dpp_i<0x143, 0xc>(0, int(v))));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Sum over each row of 16 lanes, returned in every lane of the row (butterfly: quad
// exchanges, then half-row and row mirrors).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

// Sum of an fp32 value over aligned groups of 8 lanes, returned in every lane of the group.
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  return v;
}

// Sum of an fp64 value over aligned groups of 2^LOG lanes (LOG <= 3), returned in every lane
// of the group: quad exchanges, then the half-row mirror.
template <int LOG>
__device__ __forceinline__ double group_sum_f64(double v) {
  auto step = [](double x, auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), C, 0xf, 0xf, false);
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), C, 0xf, 0xf, false);
    return x + __hiloint2double(hi, lo);
  };
  if constexpr (LOG >= 1) v = step(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  if constexpr (LOG >= 2) v = step(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  if constexpr (LOG >= 3) v = step(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  return v;
}

// Maximum over each row of 16 lanes, returned in every lane of the row (the same butterfly).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return v;
}

// The value of lane l ^ 32 (l ^ 16) in lane l, from one v_permlane32_swap (v_permlane16_swap)
// and a select: VALU only, no LDS round trip (a __shfl_xor becomes ds_bpermute). With both
// operands x, the swap returns {x of lanes 0-31 in both halves, x of lanes 32-63 in both
// halves}; the 16-lane form does the same per pair of rows (rows 0 and 1, rows 2 and 3).
__device__ __forceinline__ uint32_t lane_xor32_u(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (lane_id() & 32) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor16_u(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (lane_id() & 16) ? r[0] : r[1];
}
// x of lane l ^ off for off = 16 or 32 (a compile-time value once the caller's loop is unrolled)
__device__ __forceinline__ float lane_xor(float x, int off) {
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(off == 16 ? lane_xor16_u(u) : lane_xor32_u(u));
}
// The same exchange where only the lower lane of each pair uses the result (lanes with bit
// log2(off) clear get lane l + off's value; the others keep their own): the swap alone, no select.
__device__ __forceinline__ uint32_t lane_from_above_u(uint32_t x, int off) {
  return off == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)[1]
                   : __builtin_amdgcn_permlane32_swap(x, x, false, false)[1];
}
__device__ __forceinline__ float lane_from_above(float x, int off) {
  return __uint_as_float(lane_from_above_u(__float_as_uint(x), off));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, lane_xor(v, 16));
  return fmaxf(v, lane_xor(v, 32));
}

// XCD-aware placement. Workgroups are dealt to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2 and address translation. A grid of T workgroups (T a multiple of 8) handled
// by flat work index F = (L % 8) (T / 8) + L / 8 gives XCD k the contiguous eighth
// [k T / 8, (k + 1) T / 8) of the work, e.g. one KV head's page extrema. Other grid sizes keep
// F = L.
__device__ __forceinline__ int xcd_flat(int L, int T) {
  return (T & 7) ? L : (L & 7) * (T >> 3) + (L >> 3);
}
__device__ __forceinline__ int linear_block_id() {
  return int(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
}
__device__ __forceinline__ int grid_blocks() { return int(gridDim.x * gridDim.y * gridDim.z); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): every global load and store of
// this wave has completed. A workgroup barrier does not wait for them by itself.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------------------------
// Block-wide scan for up to 1024 threads: DPP wave scans, then the wave totals through LDS,
// scanned again by DPP in the first row of 16 lanes of every wave (one LDS read per lane).
// The totals are double-buffered, so one barrier per scan suffices as long as consecutive scans
// alternate buffers (the barrier of the scan in between orders the reuse).
// ---------------------------------------------------------------------------------------------
template <int NWV>
struct BlockScan {
  static_assert(NWV <= 16, "wave totals are scanned within one row of 16 lanes");
  int (*wt)[NWV];
  int buf;
  // Exclusive prefix of v in thread order; *total gets the block sum.
  __device__ __forceinline__ int excl(int v, int* total) {
    const int incl = wave_incl_sum(v);
    const int w = wave_id();
    int* t = wt[buf];
    buf ^= 1;
    if (lane_id() == kWave - 1) t[w] = incl;
    __syncthreads();
    const int ts = row16_incl_sum(t[lane_id() % NWV]);   // lanes 0 .. NWV-1: prefix of totals
    const int base = w > 0 ? __builtin_amdgcn_readlane(ts, w - 1) : 0;
    *total = __builtin_amdgcn_readlane(ts, NWV - 1);
    return base + incl - v;
  }
};

}  // namespace hhr
