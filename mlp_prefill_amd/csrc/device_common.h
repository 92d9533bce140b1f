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

// One 16-element block with global scale gs -> its E4M3 scale code (the
// return value) and its sixteen E2M1 codes packed low nibble first (w0:
// elements 0..7, w1: elements 8..15).  Both roundings are decided exactly.
__device__ __forceinline__ uint32_t quantize_block16(const float v[16], float gs, uint32_t& w0, uint32_t& w1) {
  float amax_b = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
  const uint32_t s = e4m3_block_scale(amax_b, gs);
  float thr[7];
  e2m1_thresholds(e4m3_value(s) * (double)gs, thr);
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

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
