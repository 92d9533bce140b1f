// Device helpers shared by the NVFP4 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlock = 16;            // elements per E4M3 block scale
constexpr double kGsDivisor = 2688.0; // 6 (largest E2M1) * 448 (largest E4M3)
constexpr float kAmaxFloor = 1e-8f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& v) {
  static_assert(sizeof(To) == sizeof(From), "size");
  To r;
  __builtin_memcpy(&r, &v, sizeof(To));
  return r;
}

// Global scale from an amax: RN32(max(amax, 1e-8) / 2688).  The float64
// quotient rounded to float32 is the correctly rounded float32 quotient.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  float a = fmaxf(amax, kAmaxFloor);
  return (float)((double)a / kGsDivisor);
}

// ---- wave / block reductions (max of non-negative floats) -----------------
// DPP row shifts 1/2/4/8 (lanes shifted in from outside a 16-lane row read 0,
// the identity for non-negative values) leave each row's max in its lane 15;
// row broadcasts 15 and 31 fold the rows into lane 63, which every lane reads.
// The max is exact, so the order does not matter.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Wave sum in a fixed butterfly order (the same on every run).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Wave sum of unsigned integers (exact in any order).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block-wide max; `lds` holds at least blockDim.x / 64 floats.  All threads
// get the result.
__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < nw; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// ---- E4M3 (OCP FN) block scale -------------------------------------------
// Exact value of an E4M3 code 0..0x7E as a double.
__device__ __forceinline__ double e4m3_value(uint32_t c) {
  if (c < 8) return (double)c * 0x1p-9;
  return (double)(8 + (c & 7)) * ldexp(1.0, (int)(c >> 3) - 10);
}

// Scale code = E4M3 round-to-nearest-even of amax_b / (6 gs) in exact real
// arithmetic, saturating at 448.  The float64 quotient decides every case
// except one where it lands exactly on a midpoint between two codes (the
// midpoints are representable, and rounding is monotone); that case is
// settled by comparing amax_b with 6 * midpoint * gs, an exact float64
// product (<= 31 significant bits).
__device__ __forceinline__ uint32_t e4m3_block_scale(float amax_b, float gs) {
  const double a = (double)amax_b;
  const double gsd = (double)gs;
  const double r = a / (6.0 * gsd);
  if (r >= 448.0) return 0x7E;
  uint32_t base;
  double n, unit, lead;
  if (r < 0x1p-6) {           // subnormal codes 0..8: value c * 2^-9
    n = r * 512.0;
    base = 0;
    unit = 0x1p-9;
    lead = 0.0;
  } else {                    // codes (E+7)<<3 | m: value (8 + m) 2^(E-3)
    int e;
    (void)frexp(r, &e);       // r = f 2^e, f in [0.5, 1)
    const int E = e - 1;
    n = ldexp(r, 3 - E) - 8.0;
    base = (uint32_t)(E + 7) << 3;
    unit = ldexp(1.0, E - 3);
    lead = 8.0;
  }
  const double fl = floor(n);
  const double frac = n - fl;
  uint32_t c = base + (uint32_t)fl;
  if (frac > 0.5) {
    c += 1;
  } else if (frac == 0.5) {
    const double thr = (6.0 * ((lead + fl + 0.5) * unit)) * gsd;
    if (a > thr || (a == thr && (c & 1u))) c += 1;
  }
  return c > 0x7Eu ? 0x7Eu : c;
}

// ---- E2M1 element codes ---------------------------------------------------
// Thresholds T[i] (float32) such that the magnitude index of |x| is the
// number of i with |x| >= T[i].  The exact decision threshold between
// magnitudes i and i+1 is t_i = mid_i * d * gs (exact in float64); on a tie
// the even index wins, so for even i the condition is |x| > t_i, for odd i
// |x| >= t_i.  T[i] is the smallest float32 above (even i) or at-or-above
// (odd i) t_i, which makes the float32 comparison exact.  A zero block scale
// gives magnitude 0 everywhere (T = +inf).
__device__ __forceinline__ void e2m1_thresholds(double dgs, float T[7]) {
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    if (dgs == 0.0) {
      T[i] = __builtin_huge_valf();
      continue;
    }
    const double t = mids[i] * dgs;
    float f = (float)t;
    const bool bump = (i & 1) ? ((double)f < t) : ((double)f <= t);
    if (bump) f = __uint_as_float(__float_as_uint(f) + 1u);
    T[i] = f;
  }
}

__device__ __forceinline__ uint32_t e2m1_code(float x, const float T[7]) {
  const float a = fabsf(x);
  uint32_t idx = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) idx += (a >= T[i]) ? 1u : 0u;
  return ((__float_as_uint(x) >> 31) << 3) | idx;
}

// ---- the same decisions in float32 ------------------------------------------
// For a global scale in [2^-90, 2^100] every decision threshold above is a
// product P * gs of a float32 P with at most 7 significant bits (6 * mid for
// the block scale, mid * dec(S) for the element codes) and gs: at most 31
// significant bits, with no underflow or overflow, so t = RN32(P * gs) and its
// rounding error fma(P, gs, -t) (exact: the error of a product is a float32
// when nothing underflows) decide every comparison exactly.
constexpr float kGsFastMin = 0x1p-90f;
constexpr float kGsFastMax = 0x1p100f;

__host__ __device__ __forceinline__ bool gs_fast(float gs) { return gs >= kGsFastMin && gs <= kGsFastMax; }

// Value of an E4M3 code 0..0x7E as a float32 (exact).
__host__ __device__ __forceinline__ float e4m3_valuef(uint32_t c) {
  if (c < 8) return (float)c * 0x1p-9f;
  uint32_t bits = (((c >> 3) + 120u) << 23) | ((c & 7u) << 20);   // (1 + m/8) 2^(E-7)
  float f;
  __builtin_memcpy(&f, &bits, 4);
  return f;
}

// Sign of a - P * g in exact arithmetic (a >= 0; P * g in the range above).
__host__ __device__ __forceinline__ int cmp_exact(float a, float P, float g) {
  const float t = P * g;
  if (a != t) return a > t ? 1 : -1;
  const float err = fmaf(P, g, -t);            // P g - t
  return err < 0.f ? 1 : (err > 0.f ? -1 : 0);
}

// E4M3 block scale code, as e4m3_block_scale, with inv6 = 1 / (6 gs) (any
// float32 within a relative 2^-21 of it): the code nearest to amax_b * inv6
// is at most one code from the exact answer (E4M3 codes lie at least a
// relative 2^-4 apart), and the two midpoints around it settle which.
__host__ __device__ __forceinline__ uint32_t e4m3_block_scale_f32(float amax_b, float gs, float inv6) {
  const float q = amax_b * inv6;
  uint32_t c;
  if (!(q < 448.f)) {
    c = 0x7E;
  } else if (q < 0x1p-6f) {
    c = (uint32_t)rintf(q * 512.f);              // subnormal codes 0..8
  } else {
    const int E = ilogbf(q);                     // q in [2^E, 2^(E+1)), E in -6..8
    const int m = (int)rintf(ldexpf(q, 3 - E));  // 8..16; 16 carries into the next binade
    c = (uint32_t)((E + 7) * 8 + m - 8);
  }
  if (c < 0x7E) {                                // between c and c+1: the even code on a tie
    const int s = cmp_exact(amax_b, 6.f * (0.5f * (e4m3_valuef(c) + e4m3_valuef(c + 1))), gs);
    if (s > 0 || (s == 0 && (c & 1u))) return c + 1;
  }
  if (c > 0) {                                   // between c-1 and c
    const int s = cmp_exact(amax_b, 6.f * (0.5f * (e4m3_valuef(c - 1) + e4m3_valuef(c))), gs);
    if (s < 0 || (s == 0 && (c & 1u))) return c - 1;
  }
  return c;
}

// E2M1 thresholds as e2m1_thresholds for the block scale value d = dec(S):
// T[i] is t = RN32(mid_i * d * gs), moved one float32 up when t is at or
// below the exact threshold (even i) or below it (odd i).
__host__ __device__ __forceinline__ void e2m1_thresholds_f32(float d, float gs, float T[7]) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const float P = mids[i] * d;                 // exact: at most 7 significant bits
    const float t = P * gs;
    const float err = fmaf(P, gs, -t);           // exact threshold minus t
    const bool bump = (i & 1) ? (err > 0.f) : (err >= 0.f);
    uint32_t u;
    __builtin_memcpy(&u, &t, 4);
    u += bump ? 1u : 0u;
    float f;
    __builtin_memcpy(&f, &u, 4);
    T[i] = d == 0.f ? __builtin_huge_valf() : f;
  }
}

// Byte J of the two code words from below and from above: elements 2J, 2J+1
// (low nibble first) and 8 + 2J, 9 + 2J.
template <int J>
__device__ __forceinline__ void cvt8_fp4(const float v[16], float lo, float hi, uint32_t& l0, uint32_t& h0,
                                         uint32_t& l1, uint32_t& h1) {
  l0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l0, v[2 * J] * lo, v[2 * J + 1] * lo, 1.0f, J);
  h0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h0, v[2 * J] * hi, v[2 * J + 1] * hi, 1.0f, J);
  l1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l1, v[8 + 2 * J] * lo, v[9 + 2 * J] * lo, 1.0f, J);
  h1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h1, v[8 + 2 * J] * hi, v[9 + 2 * J] * hi, 1.0f, J);
}

// Element codes of a block with block scale value d > 0 from the hardware
// E2M1 conversion (round to nearest, ties to even, saturating at magnitude 6,
// sign kept) of x * inv from below and from above: inv is within a relative
// 2^-22 of 1 / (d gs) (reciprocal of the rounded product), so x * lo and
// x * hi (lo, hi = inv (1 -/+ 2^-19)) bracket the exact quotient x / (d gs)
// strictly.  Rounding is monotone, so where both give the same code that code
// is the exact one; an exact tie always lies strictly inside the bracket and
// gives two codes.  Returns whether all sixteen codes agree (w0, w1: the
// codes from below).
__device__ __forceinline__ bool e2m1_codes_bracketed(const float v[16], float d, float gs, uint32_t& w0,
                                                     uint32_t& w1) {
  const float inv = __builtin_amdgcn_rcpf(d * gs);
  const float lo = inv * (1.0f - 0x1p-19f), hi = inv * (1.0f + 0x1p-19f);
  uint32_t l0 = 0, l1 = 0, h0 = 0, h1 = 0;
  cvt8_fp4<0>(v, lo, hi, l0, h0, l1, h1);
  cvt8_fp4<1>(v, lo, hi, l0, h0, l1, h1);
  cvt8_fp4<2>(v, lo, hi, l0, h0, l1, h1);
  cvt8_fp4<3>(v, lo, hi, l0, h0, l1, h1);
  w0 = l0;
  w1 = l1;
  return l0 == h0 && l1 == h1;
}

// One 16-element block with global scale gs -> its E4M3 scale code (the
// return value) and its sixteen E2M1 codes packed low nibble first (w0:
// elements 0..7, w1: elements 8..15).  Both roundings are decided exactly:
// in float32 for a global scale in [2^-90, 2^100] (every one the amax of a
// float32 tensor up to 2^111 gives), the element codes by the bracketed
// hardware conversion where it is conclusive, else by the thresholds; in
// float64 for other global scales.
__device__ __forceinline__ uint32_t quantize_block16(const float v[16], float gs, uint32_t& w0, uint32_t& w1) {
  float amax_b = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
  uint32_t s;
  float thr[7];
  if (gs_fast(gs)) {                             // uniform: one global scale per call
    s = e4m3_block_scale_f32(amax_b, gs, 1.0f / (6.0f * gs));
    const float d = e4m3_valuef(s);
    if (d > 0.f && e2m1_codes_bracketed(v, d, gs, w0, w1)) return s;
    e2m1_thresholds_f32(d, gs, thr);
  } else {
    s = e4m3_block_scale(amax_b, gs);
    e2m1_thresholds(e4m3_value(s) * (double)gs, thr);
  }
  w0 = 0;
  w1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w0 |= e2m1_code(v[i], thr) << (4 * i);
    w1 |= e2m1_code(v[8 + i], thr) << (4 * i);
  }
  return s;
}

// ---- NVFP4 -> f16 expansion for the matrix cores ---------------------------
// Eight packed E2M1 codes (one dword, element j in bits 4j+3:4j) and their
// E4M3 scale code s -> eight f16 values code_j * dec(s), exactly.  The
// hardware converter honours only the exponent of its float32 scale, so it
// is given 2^8: code * 256 is exact in f16.  The f16 with bit pattern
// (s << 7) has the value dec(s) * 2^-8 for every E4M3 code (normal codes map
// onto the f16 exponent/mantissa fields, subnormal codes onto f16
// subnormals), and the product code * dec(s) has at most 6 significant bits
// and lies in [2^-10, 2688]: exact in f16.
__device__ __forceinline__ f16x8 expand8(uint32_t codes, uint32_t s) {
  const uint32_t sh = s << 7;
  const f16x2 sc = bitcast<f16x2>(sh | (sh << 16));
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * sc;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// float32 -> bf16 bits, round to nearest even (finite inputs): the hardware
// conversion (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// SiLU(g) * u in float32, SiLU(g) = g / (1 + e^-g), with the hardware
// exp2 and reciprocal (each within about one ulp; the result is within a few
// ulp of the correctly rounded value).  Large |g| saturate correctly: e^-g
// overflows to +inf for g << 0 (SiLU -> -0) and underflows to 0 for g >> 0.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Work-group index remapped so that each XCD (work-groups are dealt
// round-robin to the 8 XCDs) receives one contiguous range of tiles.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t pid, uint32_t grid) {
  const uint32_t q = grid / 8u, r = grid % 8u;
  const uint32_t x = pid % 8u, local = pid / 8u;
  return x * q + (x < r ? x : r) + local;
}

}  // namespace nvfp4
