// NVFP4 x NVFP4 contractions on the CDNA4 matrix cores.
//
// C = A . B^T with A [M][K] (activations) and B [N][K] (a linear layer's
// weight), both NVFP4 (packed E2M1 codes + one E4M3 scale per 16 elements +
// a float32 global scale).  One launch covers the whole batch of M rows with
// a grid that grows with M (vllm.cpp issue, "Fix directions" 1).
//
// Why f16 matrix cores: NVFP4 carries an E4M3 (non power-of-two) scale per
// 16 elements, while the gfx950 block-scaled MFMA takes power-of-two E8M0
// scales per 32 elements.  code * scale has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16; each product of two such
// values is exact in the float32 accumulator's input, and only the float32
// accumulation rounds.
//
// Structure (per wave, wave64): the lane layout of v_mfma_f32_32x32x16_f16
// puts row (lane % 32) and eight consecutive K-slots (8 * (lane / 32) + j)
// of the A operand in each lane, and the same for the B operand's columns.
// The contraction is invariant under any permutation of K applied to both
// operands, so each lane streams its own row straight from global memory in
// the packed layout: for a 128-wide K chunk, lane half h reads 32 contiguous
// code bytes (64 elements) and the 4 scale bytes covering them, and feeds
// elements 64h + 8s .. 64h + 8s + 7 to MFMA step s (s = 0..7).  The packed
// bytes are expanded to f16 in registers (hardware E2M1 -> f16 convert, then
// an exact f16 multiply by the E4M3 scale), with the next chunk's loads in
// flight.  Weight rows are read in 64-byte runs per chunk; work-group tiles
// are remapped so that the tiles of one XCD share weight columns in its L2.
//
// Epilogues: float32/bf16 store scaled by gs_a * gs_b; or, with two weight
// operands (gate, up) sharing the one quantised activation (llama.cpp
// discussion, "What the patch does"), H = SiLU(gate) * up in float32 written
// to a workspace plus one partial max|H| per work-group, from which the
// requantisation kernel forms the global scale of H on the device.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gs;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_gs;
  const uint8_t* u_codes;
  const uint8_t* u_scales;
  const float* u_gs;
  int64_t M, N, K;
  void* c;
  int64_t ldc;
  int c_bf16;
  float* h;
  float* partials;
  const int32_t* a_rows;
  const int32_t* off;
  int E;
  uint32_t m_tiles;  // dense: ceil(M/BM); grouped: static bound on the expert tiles
};

// Packed operand data of one 32-row fragment for one 128-wide K chunk.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Frag {
  u32x4 c0, c1;  // 32 code bytes: 64 elements
  uint32_t s;    // 4 scale bytes
};

__device__ __forceinline__ Frag load_frag(const uint8_t* codes_row, const uint8_t* scales_row, int64_t kc) {
  Frag f;
  const u32x4* cp = reinterpret_cast<const u32x4*>(codes_row + (kc >> 1));
  f.c0 = cp[0];
  f.c1 = cp[1];
  f.s = *reinterpret_cast<const uint32_t*>(scales_row + (kc >> 4));
  return f;
}

template <int S>
__device__ __forceinline__ uint32_t frag_word(const Frag& f) {
  if constexpr (S == 0) return f.c0[0];
  else if constexpr (S == 1) return f.c0[1];
  else if constexpr (S == 2) return f.c0[2];
  else if constexpr (S == 3) return f.c0[3];
  else if constexpr (S == 4) return f.c1[0];
  else if constexpr (S == 5) return f.c1[1];
  else if constexpr (S == 6) return f.c1[2];
  else return f.c1[3];
}

template <int S>
__device__ __forceinline__ f16x8 frag_expand(const Frag& f) {
  return expand8(frag_word<S>(f), (f.s >> (8 * (S >> 1))) & 0xFFu);
}

template <int TM, int TN, bool DUAL>
struct Bufs {
  Frag a[TM];
  Frag b[TN];
  Frag u[DUAL ? TN : 1];
};

template <int TM, int TN, bool DUAL, int S>
__device__ __forceinline__ void mfma_step(const Bufs<TM, TN, DUAL>& f, f32x16 (&acc)[TM][TN],
                                          f32x16 (&accu)[TM][TN]) {
  f16x8 av[TM], bv[TN], uv[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) av[i] = frag_expand<S>(f.a[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    bv[j] = frag_expand<S>(f.b[j]);
    if constexpr (DUAL) uv[j] = frag_expand<S>(f.u[j]);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      if constexpr (DUAL) accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], uv[j], accu[i][j], 0, 0, 0);
    }
}

template <int TM, int TN, bool DUAL>
__device__ __forceinline__ void mfma_chunk(const Bufs<TM, TN, DUAL>& f, f32x16 (&acc)[TM][TN],
                                           f32x16 (&accu)[TM][TN]) {
  mfma_step<TM, TN, DUAL, 0>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 1>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 2>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 3>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 4>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 5>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 6>(f, acc, accu);
  mfma_step<TM, TN, DUAL, 7>(f, acc, accu);
}

enum { EPI_STORE = 0, EPI_GLU = 1 };

template <int WM, int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI>
__global__ void __launch_bounds__(WM * WN * 64) gemm_kernel(GemmArgs p) {
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  __shared__ float red[WM * WN];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int r32 = lane & 31, hh = lane >> 5;

  // ---- tile ---------------------------------------------------------------
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t n_tile = t / p.m_tiles;
  const uint32_t mt = t - n_tile * p.m_tiles;
  int64_t m0, m_end;
  int e = 0;
  if constexpr (GROUPED) {
    // Map the m-tile index onto (expert, tile within the expert) from the
    // device-resident offsets; tiles past the last expert have no work.
    uint32_t cum = 0;
    m0 = -1;
    m_end = 0;
    for (int x = 0; x < p.E; ++x) {
      const int64_t s0 = p.off[x], s1 = p.off[x + 1];
      const uint32_t nt = (uint32_t)((s1 - s0 + BM - 1) / BM);
      if (mt < cum + nt) {
        e = x;
        m0 = s0 + (int64_t)(mt - cum) * BM;
        m_end = s1;
        break;
      }
      cum += nt;
    }
    if (m0 < 0) {
      if constexpr (EPI == EPI_GLU) {
        if (threadIdx.x == 0) p.partials[blockIdx.x] = 0.f;
      }
      return;
    }
  } else {
    m0 = (int64_t)mt * BM;
    m_end = p.M;
  }
  const int64_t n0 = (int64_t)n_tile * BN;
  const int64_t K = p.K;
  const int64_t kb = K >> 1, ks = K >> 4;
  const int64_t wstride_c = GROUPED ? (int64_t)e * p.N * kb : 0;
  const int64_t wstride_s = GROUPED ? (int64_t)e * p.N * ks : 0;

  // ---- per-lane row pointers (rows past the end are clamped; never stored) ----
  const uint8_t* a_c[TM];
  const uint8_t* a_s[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t m = m0 + (wm * TM + i) * 32 + r32;
    if (m > m_end - 1) m = m_end - 1;
    const int64_t src = (GROUPED && p.a_rows) ? (int64_t)p.a_rows[m] : m;
    a_c[i] = p.a_codes + src * kb + 32 * hh;
    a_s[i] = p.a_scales + src * ks + 4 * hh;
  }
  const uint8_t* b_c[TN];
  const uint8_t* b_s[TN];
  const uint8_t* u_c[TN];
  const uint8_t* u_s[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int64_t n = n0 + (wn * TN + j) * 32 + r32;
    if (n > p.N - 1) n = p.N - 1;
    b_c[j] = p.b_codes + wstride_c + n * kb + 32 * hh;
    b_s[j] = p.b_scales + wstride_s + n * ks + 4 * hh;
    if constexpr (DUAL) {
      u_c[j] = p.u_codes + wstride_c + n * kb + 32 * hh;
      u_s[j] = p.u_scales + wstride_s + n * ks + 4 * hh;
    }
  }

  f32x16 acc[TM][TN];
  f32x16 accu[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[i][j][r] = 0.f;
        accu[i][j][r] = 0.f;
      }

  auto load_all = [&](Bufs<TM, TN, DUAL>& f, int64_t kc) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = load_frag(a_c[i], a_s[i], kc);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      f.b[j] = load_frag(b_c[j], b_s[j], kc);
      if constexpr (DUAL) f.u[j] = load_frag(u_c[j], u_s[j], kc);
    }
  };

  // ---- main loop: two register buffers, the next chunk's loads in flight ----
  Bufs<TM, TN, DUAL> f0, f1;
  load_all(f0, 0);
  int64_t kc = 0;
  for (; kc + 256 <= K; kc += 256) {
    load_all(f1, kc + 128);
    mfma_chunk<TM, TN, DUAL>(f0, acc, accu);
    if (kc + 256 < K) load_all(f0, kc + 256);
    mfma_chunk<TM, TN, DUAL>(f1, acc, accu);
  }
  if (kc < K) mfma_chunk<TM, TN, DUAL>(f0, acc, accu);

  // ---- epilogue ---------------------------------------------------------------
  const float alpha = p.a_gs[0] * p.b_gs[GROUPED ? e : 0];
  float alpha_u = 0.f;
  if constexpr (DUAL) alpha_u = p.a_gs[0] * p.u_gs[GROUPED ? e : 0];
  float hmax = 0.f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + (wn * TN + j) * 32 + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + (wm * TM + i) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < m_end && col < p.N) {
          if constexpr (EPI == EPI_GLU) {
            const float hv = silu_mul(acc[i][j][r] * alpha, accu[i][j][r] * alpha_u);
            p.h[row * p.N + col] = hv;
            hmax = fmaxf(hmax, fabsf(hv));
          } else {
            const float v = acc[i][j][r] * alpha;
            if (p.c_bf16)
              reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] = (uint16_t)f32_to_bf16_bits(v);
            else
              reinterpret_cast<float*>(p.c)[row * p.ldc + col] = v;
          }
        }
      }
    }
  if constexpr (EPI == EPI_GLU) {
    hmax = block_max(hmax, red);
    if (threadIdx.x == 0) p.partials[blockIdx.x] = hmax;
  }
}

// ---- launch configurations ------------------------------------------------------
// Small batches (M <= 32): one 32-row MFMA tile, four waves side by side in N.
// Larger batches: 2x2 waves of 64x64 (x2 with the gate/up pair).
template <int WM, int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI>
static int launch_cfg(const GemmArgs& a_in, uint32_t m_tiles, hipStream_t st) {
  constexpr int BN = WN * TN * 32;
  GemmArgs a = a_in;
  a.m_tiles = m_tiles;
  const uint32_t n_tiles = (uint32_t)((a.N + BN - 1) / BN);
  const uint32_t grid = m_tiles * n_tiles;
  hipLaunchKernelGGL((gemm_kernel<WM, WN, TM, TN, DUAL, GROUPED, EPI>), dim3(grid), dim3(WM * WN * 64), 0, st, a);
  count_launch();
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

static uint32_t tiles(int64_t n, int64_t b) { return (uint32_t)((n + b - 1) / b); }

static GemmArgs base_args(Operand a, Operand b, int64_t M, int64_t N, int64_t K) {
  GemmArgs g{};
  g.a_codes = a.codes; g.a_scales = a.scales; g.a_gs = a.gscale;
  g.b_codes = b.codes; g.b_scales = b.scales; g.b_gs = b.gscale;
  g.M = M; g.N = N; g.K = K;
  return g;
}

int gemm_launch(Operand a, Operand b, int64_t M, int64_t N, int64_t K, void* c, int c_bf16, int64_t ldc,
                hipStream_t st) {
  GemmArgs g = base_args(a, b, M, N, K);
  g.c = c; g.ldc = ldc; g.c_bf16 = c_bf16;
  if (M <= 32) return launch_cfg<1, 4, 1, 1, false, false, EPI_STORE>(g, tiles(M, 32), st);
  return launch_cfg<2, 2, 2, 2, false, false, EPI_STORE>(g, tiles(M, 128), st);
}

size_t glu_partials_needed(int64_t M, int64_t N) {
  if (M <= 32) return (size_t)tiles(M, 32) * tiles(N, 128);
  return (size_t)tiles(M, 128) * tiles(N, 128);
}

int gemm_glu_launch(Operand a, Operand gt, Operand up, int64_t M, int64_t N, int64_t K, float* h,
                    float* partials, uint32_t* npart, hipStream_t st) {
  GemmArgs g = base_args(a, gt, M, N, K);
  g.u_codes = up.codes; g.u_scales = up.scales; g.u_gs = up.gscale;
  g.h = h; g.partials = partials;
  *npart = (uint32_t)glu_partials_needed(M, N);
  if (M <= 32) return launch_cfg<1, 4, 1, 1, true, false, EPI_GLU>(g, tiles(M, 32), st);
  return launch_cfg<2, 2, 2, 2, true, false, EPI_GLU>(g, tiles(M, 128), st);
}

// Static bound on the number of 128-row expert tiles: sum_e ceil(n_e/128) <= M/128 + E.
static uint32_t grouped_m_tiles(int64_t M, int E) { return tiles(M, 128) + (uint32_t)E; }

size_t grouped_glu_partials_needed(int64_t M, int64_t N, int E) {
  return (size_t)grouped_m_tiles(M, E) * tiles(N, 128);
}

int grouped_gemm_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand w,
                        int64_t N, int64_t K, void* c, int c_bf16, int64_t ldc, hipStream_t st) {
  GemmArgs g = base_args(a, w, M, N, K);
  g.c = c; g.ldc = ldc; g.c_bf16 = c_bf16;
  g.a_rows = a_rows; g.off = off; g.E = E;
  return launch_cfg<2, 2, 2, 2, false, true, EPI_STORE>(g, grouped_m_tiles(M, E), st);
}

int grouped_glu_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt,
                       Operand up, int64_t N, int64_t K, float* h, float* partials, uint32_t* npart,
                       hipStream_t st) {
  GemmArgs g = base_args(a, gt, M, N, K);
  g.u_codes = up.codes; g.u_scales = up.scales; g.u_gs = up.gscale;
  g.h = h; g.partials = partials;
  g.a_rows = a_rows; g.off = off; g.E = E;
  *npart = (uint32_t)grouped_glu_partials_needed(M, N, E);
  return launch_cfg<2, 2, 2, 2, true, true, EPI_GLU>(g, grouped_m_tiles(M, E), st);
}

}  // namespace nvfp4
