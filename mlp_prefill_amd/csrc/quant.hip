// NVFP4 activation quantisation on the device: tensor amax, global scale,
// E4M3 block scales and packed E2M1 codes.
//
// The activation global scale amax/(6*448), clamped at 1e-8, is the runtime
// scale of the DSV4 audit page (section P0); here it is produced and consumed
// on the device and never read back to the host.  Packing happens on the
// device (vllm.cpp issue, "Fix directions" 3).
//
// Two kernels (one for tensors of at most 8192 blocks, see
// quantize_small_kernel): amax_partials writes one partial maximum per work-group;
// quantize reduces those partials again in every work-group (a few KiB from
// L2, no atomics, no zero-initialised state), forms the global scale, and
// quantises 16-element blocks in a grid-stride loop (one block per thread per
// iteration, at most 2048 work-groups).  Both are HBM-bound: the
// quantiser reads 2 (bf16) or 4 (float32) bytes per element and writes
// 0.5 + 1/16 bytes.
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

template <typename T>
struct Load16;

// 16 bf16 values (32 B, 16-B aligned) -> float32
template <>
struct Load16<uint16_t> {
  __device__ __forceinline__ static void run(const uint16_t* p, float v[16]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// 16 float32 values (64 B, 16-B aligned)
template <>
struct Load16<float> {
  __device__ __forceinline__ static void run(const float* p, float v[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = *reinterpret_cast<const float4*>(p + 4 * i);
      v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
  }
};

template <typename T>
__global__ void __launch_bounds__(256) amax_partials_kernel(const T* __restrict__ x, uint32_t nbc,
                                                            uint32_t nblocks, int64_t ld,
                                                            float* __restrict__ partials) {
  __shared__ float red[4];
  float m = 0.f;
  for (uint32_t b = blockIdx.x * 256u + threadIdx.x; b < nblocks; b += gridDim.x * 256u) {
    const uint32_t row = b / nbc, cb = b - row * nbc;
    float v[16];
    Load16<T>::run(x + (int64_t)row * ld + (int64_t)cb * kBlock, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// When x16 is given, the block's dequantised values code * scale (exact in
// f16) also go to x16 [rows][cols]: the operand copy the matrix-core
// contraction reads, written here instead of by a separate expansion pass.
__device__ __forceinline__ void store_expanded(_Float16* x16, int64_t boff, uint32_t w0, uint32_t w1, uint32_t s) {
  if (x16 == nullptr) return;
  f16x8* o = reinterpret_cast<f16x8*>(x16 + boff * 16);
  o[0] = expand8(w0, s);
  o[1] = expand8(w1, s);
}

// mode 0: gs from the partial maxima (written to gs_ptr by work-group 0);
// mode 1: gs read from gs_ptr.
// NORM: quantise y = (x * rinv[row]) * gamma[col] (float32, the RMSNorm
// output) instead of x.
template <typename T, bool NORM = false>
__global__ void __launch_bounds__(256) quantize_kernel(const T* __restrict__ x, uint32_t nbc,
                                                       uint32_t nblocks, int64_t ld,
                                                       const float* __restrict__ partials,
                                                       uint32_t npart, float* gs_ptr, int mode,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const float* __restrict__ rinv = nullptr,
                                                       const float* __restrict__ gamma = nullptr,
                                                       _Float16* __restrict__ x16 = nullptr) {
  __shared__ float red[4];
  float gs;
  if (mode == 0) {
    // eight independent loads per step: the reduction is latency-bound when
    // there are thousands of partials (max is exact in any order)
    float m = 0.f;
    for (uint32_t i = threadIdx.x; i < npart; i += 8u * 256u) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = i + k * 256u < npart ? partials[i + k * 256u] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, v[k]);
    }
    m = block_max(m, red);
    gs = global_scale_from_amax(m);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gs_ptr = gs;
  } else {
    gs = *gs_ptr;
  }
  for (uint32_t b = blockIdx.x * 256u + threadIdx.x; b < nblocks; b += gridDim.x * 256u) {
    const uint32_t row = b / nbc, cb = b - row * nbc;
    float v[16];
    Load16<T>::run(x + (int64_t)row * ld + (int64_t)cb * kBlock, v);
    if constexpr (NORM) {
      const float r = rinv[row];
      float g[16];
      Load16<float>::run(gamma + (int64_t)cb * kBlock, g);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (v[i] * r) * g[i];
    }
    uint32_t w0, w1;
    const uint32_t s = quantize_block16(v, gs, w0, w1);
    const int64_t boff = (int64_t)row * nbc + cb;
    *reinterpret_cast<uint2*>(codes + boff * 8) = make_uint2(w0, w1);
    scales[boff] = (uint8_t)s;
    store_expanded(x16, boff, w0, w1, s);
  }
}

// RMSNorm fused into the quantiser, first pass: one wave per row (grid-stride)
// forms r = 1 / sqrt(mean(x^2) + eps) (float32 sum in a fixed order, IEEE
// sqrt and division) and stores it in rinv[row]; the work-group's max of
// |(x * r) * gamma| goes to partials[blockIdx.x].  The second pass is
// quantize_kernel<T, true>, which forms the same float32 products.
template <typename T>
__global__ void __launch_bounds__(256) rms_amax_kernel(const T* __restrict__ x, int64_t rows, uint32_t nbc,
                                                       int64_t ld, const float* __restrict__ gamma, float eps,
                                                       float* __restrict__ rinv, float* __restrict__ partials) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
    const T* xr = x + row * ld;
    float ss = 0.f;
    for (uint32_t cb = lane; cb < nbc; cb += 64) {
      float v[16];
      Load16<T>::run(xr + (int64_t)cb * kBlock, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(v[i], v[i], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)(nbc * kBlock) + eps);
    if (lane == 0) rinv[row] = r;
    for (uint32_t cb = lane; cb < nbc; cb += 64) {
      float v[16], g[16];
      Load16<T>::run(xr + (int64_t)cb * kBlock, v);
      Load16<float>::run(gamma + (int64_t)cb * kBlock, g);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf((v[i] * r) * g[i]));
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Small tensors (decode activations: at most kSmallBlocks = 8192 blocks of
// 16) in one launch of ceil(blocks / 1024) work-groups of 1024 threads: every
// work-group reduces the amax of the whole tensor itself -- each thread loads
// up to four blocks per round, all in flight at once, one round per 4096
// blocks (at most 256 KiB of bf16, from L2 after the first work-group) -- and
// then quantises its own 1024 blocks, the one whose index matches its
// work-group kept in registers from its round.  No work-group waits for
// another, and a kernel boundary costs more than the repeated reduction.  The
// max is exact in any order and the per-block routine is the same, so the
// result equals the two-kernel path bit for bit.
constexpr uint32_t kSmallBlocks = kSmallQuantBlocks;
static_assert(kSmallBlocks <= 8u * 1024u, "at most eight work-groups, two rounds");
static_assert(kAmaxSlots <= 1024u, "one given partial maximum per thread");

//
// As the first launch of a whole-MLP call it also clears `nzero` words
// (the split-K tickets and output-amax slots the later launches of the call
// use), and it can take the amax from `given` (npart <= 1024 partial maxima
// written by an earlier call's output-amax epilogue) instead of reducing x.
template <typename T>
__global__ void __launch_bounds__(1024) quantize_small_kernel(const T* __restrict__ x, uint32_t nbc,
                                                              uint32_t nblocks, int64_t ld, float* gs_ptr,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              uint32_t* __restrict__ zero = nullptr,
                                                              uint32_t nzero = 0,
                                                              const float* __restrict__ given = nullptr,
                                                              uint32_t npart = 0,
                                                              uint32_t* __restrict__ zero2 = nullptr,
                                                              uint32_t nzero2 = 0,
                                                              _Float16* __restrict__ x16 = nullptr) {
  __shared__ float red[16];
  const uint32_t tid = blockIdx.x * 1024u + threadIdx.x, nthr = gridDim.x * 1024u;
  for (uint32_t i = tid; i < nzero; i += nthr) zero[i] = 0u;
  for (uint32_t i = tid; i < nzero2; i += nthr) zero2[i] = 0u;
  float w[16];
  float m = 0.f;
  if (given != nullptr) {
    if (threadIdx.x < npart) m = given[threadIdx.x];
  } else {
    for (uint32_t r0 = 0; r0 < nblocks; r0 += 4096u) {
      float v[4][16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t b = r0 + threadIdx.x + q * 1024u;
        if (b < nblocks) {
          const uint32_t row = b / nbc, cb = b - row * nbc;
          Load16<T>::run(x + (int64_t)row * ld + (int64_t)cb * kBlock, v[q]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[q][i] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[q][i]));
        if (r0 / 1024u + q == blockIdx.x) {           // this work-group's own block
#pragma unroll
          for (int i = 0; i < 16; ++i) w[i] = v[q][i];
        }
      }
    }
  }
  m = block_max(m, red);
  const float gs = global_scale_from_amax(m);
  if (tid == 0) *gs_ptr = gs;
  const uint32_t b = tid;
  if (b >= nblocks) return;
  const uint32_t row = b / nbc, cb = b - row * nbc;
  if (given != nullptr) Load16<T>::run(x + (int64_t)row * ld + (int64_t)cb * kBlock, w);
  uint32_t w0, w1;
  const uint32_t sc = quantize_block16(w, gs, w0, w1);
  const int64_t boff = (int64_t)row * nbc + cb;
  *reinterpret_cast<uint2*>(codes + boff * 8) = make_uint2(w0, w1);
  scales[boff] = (uint8_t)sc;
  store_expanded(x16, boff, w0, w1, sc);
}

// Work-groups of the quantiser: enough to fill the chip, few enough that the
// per-work-group re-reduction of the partial maxima stays cheap.
#ifndef NVFP4_QUANT_GRID
#define NVFP4_QUANT_GRID 2048
#endif
constexpr uint32_t kQuantGrid = NVFP4_QUANT_GRID;

static uint32_t amax_grid(uint32_t nblocks) {
  uint32_t g = (nblocks + 1023u) / 1024u;   // ~4 blocks of 16 per thread
  if (g < 1) g = 1;
  if (g > kMaxPartials) g = kMaxPartials;
  return g;
}

size_t quantize_ws_bytes(int64_t rows, int64_t cols, int gs_mode) {
  if (gs_mode == 2) return kAmaxSlots * sizeof(float);   // the given partial maxima
  if (gs_mode != 0) return 0;
  (void)rows; (void)cols;
  return kMaxPartials * sizeof(float);
}

template <typename T>
static int quantize_launch_t(const T* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                             uint8_t* scales, float* gs, int gs_mode, float* partials,
                             const float* ext_partials, uint32_t ext_npart, hipStream_t st,
                             _Float16* x16 = nullptr) {
  const uint32_t nbc = (uint32_t)(cols / kBlock);
  const uint32_t nblocks = (uint32_t)rows * nbc;
  uint32_t qgrid = (nblocks + 255u) / 256u;
  if (qgrid > kQuantGrid) qgrid = kQuantGrid;
  if (qgrid < 1) qgrid = 1;
  if (gs_mode == 0 && ext_partials == nullptr && nblocks <= kSmallBlocks) {
    const int s0 = launch_begin(KC_QUANTIZE, st);
    hipLaunchKernelGGL(quantize_small_kernel<T>, dim3((nblocks + 1023u) / 1024u), dim3(1024), 0, st, x, nbc,
                       nblocks, ld, gs, codes, scales,
                       (uint32_t*)nullptr, 0u, (const float*)nullptr, 0u, (uint32_t*)nullptr, 0u, x16);
    launch_end(s0, st);
  } else if (gs_mode == 0 && ext_partials == nullptr) {
    const uint32_t g = amax_grid(nblocks);
    const int s0 = launch_begin(KC_QUANTIZE, st);
    hipLaunchKernelGGL(amax_partials_kernel<T>, dim3(g), dim3(256), 0, st, x, nbc, nblocks, ld, partials);
    launch_end(s0, st);
    const int s1 = launch_begin(KC_QUANTIZE, st);
    hipLaunchKernelGGL(quantize_kernel<T>, dim3(qgrid), dim3(256), 0, st, x, nbc, nblocks, ld,
                       (const float*)partials, g, gs, 0, codes, scales, (const float*)nullptr, (const float*)nullptr,
                       x16);
    launch_end(s1, st);
  } else {
    const int s1 = launch_begin(KC_QUANTIZE, st);
    if (gs_mode == 0)
      hipLaunchKernelGGL(quantize_kernel<T>, dim3(qgrid), dim3(256), 0, st, x, nbc, nblocks, ld,
                         ext_partials, ext_npart, gs, 0, codes, scales, (const float*)nullptr, (const float*)nullptr,
                         x16);
    else
      hipLaunchKernelGGL(quantize_kernel<T>, dim3(qgrid), dim3(256), 0, st, x, nbc, nblocks, ld,
                         (const float*)nullptr, 0u, gs, 1, codes, scales, (const float*)nullptr,
                         (const float*)nullptr, x16);
    launch_end(s1, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                    uint8_t* scales, float* gs, int gs_mode, void* ws, hipStream_t st, _Float16* x16) {
  float* partials = reinterpret_cast<float*>(ws);
  if (gs_mode == 2) {
    // the workspace holds kAmaxSlots partial maxima of |x| (written on the
    // device by an earlier call's output-amax epilogue): the quantise kernel
    // reduces them, forms the global scale and quantises, in one launch
    if (x_dtype == 1)
      return quantize_launch_t(reinterpret_cast<const uint16_t*>(x), rows, cols, ld, codes, scales, gs, 0, nullptr,
                               partials, kAmaxSlots, st, x16);
    return quantize_launch_t(reinterpret_cast<const float*>(x), rows, cols, ld, codes, scales, gs, 0, nullptr,
                             partials, kAmaxSlots, st, x16);
  }
  if (x_dtype == 1)
    return quantize_launch_t(reinterpret_cast<const uint16_t*>(x), rows, cols, ld, codes, scales, gs,
                             gs_mode, partials, nullptr, 0, st, x16);
  return quantize_launch_t(reinterpret_cast<const float*>(x), rows, cols, ld, codes, scales, gs, gs_mode,
                           partials, nullptr, 0, st, x16);
}

// ---- allocation-free variant ---------------------------------------------------
// The partial maxima of the amax pass (the whole workspace a COMPUTE call
// needs, at most kMaxPartials floats = 16 KiB whatever the tensor size) live in
// this array instead of a caller's workspace.  Each GPU holds its own copy
// until the process ends; every call on that GPU shares it.
static __device__ __align__(256) float scratch[kMaxPartials];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

size_t quantize_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on the current device: looked up once per device
// (hipGetSymbolAddress with that device current), then reused.  In host code
// the name `scratch` is only a handle for the lookup, never an address.
int quantize_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    (void)hipGetLastError();
    return 6;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return 6;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

size_t rmsnorm_quantize_ws_bytes(int64_t rows) {
  return ((size_t)rows * 4 + 255) / 256 * 256 + kMaxPartials * sizeof(float);
}

template <typename T>
static int rmsnorm_quantize_t(const T* x, int64_t rows, int64_t cols, int64_t ld, const float* gamma, float eps,
                              uint8_t* codes, uint8_t* scales, float* gs, void* ws, hipStream_t st) {
  float* rinv = reinterpret_cast<float*>(ws);
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ((size_t)rows * 4 + 255) / 256 * 256);
  const uint32_t nbc = (uint32_t)(cols / kBlock);
  const uint32_t nblocks = (uint32_t)rows * nbc;
  int64_t g = (rows + 3) / 4;
  if (g > kMaxPartials) g = kMaxPartials;
  uint32_t qgrid = (nblocks + 255u) / 256u;
  if (qgrid > kQuantGrid) qgrid = kQuantGrid;
  if (qgrid < 1) qgrid = 1;
  const int s0 = launch_begin(KC_QUANTIZE, st);
  hipLaunchKernelGGL(rms_amax_kernel<T>, dim3((uint32_t)g), dim3(256), 0, st, x, rows, nbc, ld, gamma, eps, rinv,
                     partials);
  launch_end(s0, st);
  const int s1 = launch_begin(KC_QUANTIZE, st);
  hipLaunchKernelGGL((quantize_kernel<T, true>), dim3(qgrid), dim3(256), 0, st, x, nbc, nblocks, ld,
                     (const float*)partials, (uint32_t)g, gs, 0, codes, scales, (const float*)rinv, gamma);
  launch_end(s1, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int rmsnorm_quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, const float* gamma,
                            float eps, uint8_t* codes, uint8_t* scales, float* gs, void* ws, hipStream_t st) {
  if (x_dtype == 1)
    return rmsnorm_quantize_t(reinterpret_cast<const uint16_t*>(x), rows, cols, ld, gamma, eps, codes, scales, gs,
                              ws, st);
  return rmsnorm_quantize_t(reinterpret_cast<const float*>(x), rows, cols, ld, gamma, eps, codes, scales, gs, ws,
                            st);
}

int mlp_prologue_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                        uint8_t* scales, float* gs, const float* x_amax, uint32_t* zero, uint32_t nzero,
                        uint32_t* zero2, uint32_t nzero2, hipStream_t st) {
  const uint32_t nbc = (uint32_t)(cols / kBlock);
  const uint32_t nblocks = (uint32_t)rows * nbc;
  const uint32_t npart = x_amax ? kAmaxSlots : 0u;
  const uint32_t grid = nblocks > 0 ? (nblocks + 1023u) / 1024u : 1u;
  const int s0 = launch_begin(KC_QUANTIZE, st);
  if (x_dtype == 1)
    hipLaunchKernelGGL(quantize_small_kernel<uint16_t>, dim3(grid), dim3(1024), 0, st,
                       reinterpret_cast<const uint16_t*>(x), nbc, nblocks, ld, gs, codes, scales, zero, nzero, x_amax,
                       npart, zero2, nzero2);
  else
    hipLaunchKernelGGL(quantize_small_kernel<float>, dim3(grid), dim3(1024), 0, st, reinterpret_cast<const float*>(x),
                       nbc, nblocks, ld, gs, codes, scales, zero, nzero, x_amax, npart, zero2, nzero2);
  launch_end(s0, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int requant_f32_launch(const float* h, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                       float* gs, const float* partials, uint32_t npart, hipStream_t st, _Float16* h16) {
  return quantize_launch_t(h, rows, cols, cols, codes, scales, gs, 0, nullptr, partials, npart, st, h16);
}

}  // namespace nvfp4
