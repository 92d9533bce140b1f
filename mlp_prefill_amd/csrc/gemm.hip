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
// values is exact, and only the float32 accumulation rounds.
//
// Data flow.  The activation operand is expanded once per call to f16
// (code * scale, exact) by expand_kernel -- a cheap pass over T x K that can
// also gather rows (expert slots).  The GEMM kernel then streams the packed
// weights: v_mfma_f32_32x32x16_f16 holds, in each lane, row (lane % 32) and
// eight consecutive K-slots 8 * (lane / 32) + j of an operand.  The
// contraction is invariant under any permutation of K applied to both
// operands, so each lane reads its own rows contiguously: for a 128-wide K
// chunk, lane half h of a weight fragment reads 32 code bytes (64 elements)
// and the 4 scale bytes covering them, and feeds elements 64h + 8s .. +7 to
// MFMA step s (s = 0..7); the activation fragment for step s is the 16 bytes
// of f16 at the same K positions.
//
// Each 128-wide K chunk of the work-group's activation tile (f16) and weight
// tile (packed codes and scales) is copied from global memory straight into
// LDS by the LDS DMA path, double-buffered: the copy of chunk c+1 is in
// flight while chunk c is consumed.  Weight fragments are read from LDS
// packed and expanded in registers (hardware E2M1 -> f16 convert and an
// exact f16 multiply by the E4M3 scale) one step ahead of the MFMAs that
// consume them, so the vector ALU work co-issues with the matrix core.
//
// The waves of a work-group sit side by side along N and share the staged
// activation rows; each expands only its own weight columns, so no
// expansion is duplicated.  Work-group tiles are remapped so that the tiles
// of one XCD share weight columns in its L2.
//
// Epilogues: float32/bf16 store scaled by gs_a * gs_b (or unscaled split-K
// partials reduced by splitk_reduce_kernel in a fixed order); or, with two
// weight operands (gate, up) sharing the one activation (llama.cpp
// discussion, "What the patch does"), H = SiLU(gate) * up in float32 written
// to a workspace plus one partial max|H| per work-group, from which the
// requantisation kernel forms the global scale of H on the device.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const _Float16* a;      // expanded activations, f16 [rows][K] (slot order when grouped)
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
  float* split_out;       // [splits][M][N] float32 partial sums (splits > 1)
  const int32_t* off;
  int E;
  uint32_t m_tiles;       // dense: ceil(M/BM); grouped: static bound on the expert tiles
  uint32_t n_tiles;
  uint32_t splits;
  uint32_t chunks_per_split;
};

// ---- expansion of the activation operand ------------------------------------------
// out[r][k] = code * scale (f16, exact) of row src(r) = rows ? rows[r] : r.
__global__ void __launch_bounds__(256) expand_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const int32_t* __restrict__ rows, uint32_t nbc,
                                                     uint32_t nblocks, _Float16* __restrict__ out) {
  for (uint32_t b = blockIdx.x * 256u + threadIdx.x; b < nblocks; b += gridDim.x * 256u) {
    const uint32_t r = b / nbc, cb = b - r * nbc;
    const int64_t src = rows ? (int64_t)rows[r] : (int64_t)r;
    const uint2 c = *reinterpret_cast<const uint2*>(codes + (src * nbc + cb) * 8);
    const uint32_t s = scales[src * nbc + cb];
    const f16x8 lo = expand8(c.x, s), hi = expand8(c.y, s);
    f16x8* o = reinterpret_cast<f16x8*>(out + ((int64_t)r * nbc + cb) * 16);
    o[0] = lo;
    o[1] = hi;
  }
}

// ---- packed weight fragments --------------------------------------------------------
struct Frag {
  u32x4 c0, c1;  // 32 code bytes: 64 elements
  uint32_t s;    // 4 scale bytes
};

template <int S>
__device__ __forceinline__ f16x8 frag_expand(const Frag& f) {
  const uint32_t w = (S < 4) ? f.c0[S & 3] : f.c1[S & 3];
  return expand8(w, (f.s >> (8 * (S >> 1))) & 0xFFu);
}

template <int TN, bool DUAL>
struct BPack {
  Frag b[TN];
  Frag u[DUAL ? TN : 1];
};

template <int TN, bool DUAL>
struct BExp {
  f16x8 b[TN];
  f16x8 u[DUAL ? TN : 1];
};

template <int TN, bool DUAL, int S>
__device__ __forceinline__ void expand_b(const BPack<TN, DUAL>& f, BExp<TN, DUAL>& e) {
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    e.b[j] = frag_expand<S>(f.b[j]);
    if constexpr (DUAL) e.u[j] = frag_expand<S>(f.u[j]);
  }
}

enum { EPI_STORE = 0, EPI_GLU = 1 };

// Per-chunk LDS staging (one 128-wide K chunk):
//   activations: BM rows x 16 slots of 16 B (f16); row r keeps K segment g
//                (8 elements) in slot g ^ (r % 16);
//   weight codes: NB rows x 4 units of 16 B (64 B = 128 codes); row r keeps
//                unit u in slot u ^ ((r / 4) % 4);
//   weight scales: NB rows x 8 B.
// NB = BN (or 2 BN with the gate/up pair).  All global loads are row
// contiguous: 16 lanes cover one activation row (256 B), 4 lanes one weight
// row (64 B), one lane the 8 scale bytes of a weight row.  The swizzles keep
// the fragment reads (32 rows at the same K offset) free of bank conflicts.
template <int WN, int TM, int TN, bool DUAL>
struct Cfg {
  static constexpr int BM = TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int NB = BN * (DUAL ? 2 : 1);   // weight rows per work-group
  static constexpr int NT = WN * 64;
  static constexpr int SA = BM * 16 / NT;           // 16-B activation units per thread
  static constexpr int SB = NB * 4 / NT;            // 16-B weight-code units per thread
  static constexpr int SD = NB * 2 / NT;            // 4-B scale units per thread
  static constexpr int LDS_A = BM * 16;             // f16x8 units
  static constexpr int LDS_B = NB * 4;              // u32x4 units
  static_assert(SA * NT == BM * 16 && SB * NT == NB * 4 && SD * NT == NB * 2, "tile must divide the thread count");
};

template <int WN, int TM, int TN, bool DUAL>
struct Ctx {
  using C = Cfg<WN, TM, TN, DUAL>;
  const _Float16* a_src[C::SA];  // global source of each staged 16-B unit (chunk 0 of this split)
  const uint8_t* b_src[C::SB];
  const uint8_t* s_src[C::SD];
  f16x8 ring[2][TM];             // activation fragments of the current and next step
  int lds_row[TM];               // LDS unit index of this lane's activation rows (row * 16)
  int lds_swz;                   // row % 16 of this lane's activation rows
  f32x16 acc[TM][TN];
  f32x16 accu[DUAL ? TM : 1][DUAL ? TN : 1];
};

struct Lds {
  f16x8* a;
  u32x4* b;
  uint2* s;
};

// Copy one K chunk of the work-group's activation and weight tiles straight
// from global memory into LDS buffer `l` (LDS DMA: no registers, no LDS store
// instructions).  Lane l of a wave writes the 16 (or 4) bytes at LDS unit
// base + l, so each unit's global source is chosen to realise the swizzled
// layout described above.
template <int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void stage_dma(const Ctx<WN, TM, TN, DUAL>& x, const Lds& l, int64_t chunk) {
  using C = Cfg<WN, TM, TN, DUAL>;
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS DMA builtin exists only in the device pass
  const int wbase = (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int u = 0; u < C::SA; ++u)
    __builtin_amdgcn_global_load_lds(x.a_src[u] + chunk * 128, l.a + u * C::NT + wbase, 16, 0, 0);
#pragma unroll
  for (int u = 0; u < C::SB; ++u)
    __builtin_amdgcn_global_load_lds(x.b_src[u] + chunk * 64, l.b + u * C::NT + wbase, 16, 0, 0);
#pragma unroll
  for (int u = 0; u < C::SD; ++u)
    __builtin_amdgcn_global_load_lds(x.s_src[u] + chunk * 8, reinterpret_cast<uint32_t*>(l.s) + u * C::NT + wbase,
                                     4, 0, 0);
#endif
}

// Packed weight fragment of LDS row `row` for this lane's K half.
__device__ __forceinline__ Frag read_frag(const Lds& l, int row, int hh) {
  Frag f;
  const int sw = (row >> 2) & 3;
  f.c0 = l.b[row * 4 + ((2 * hh) ^ sw)];
  f.c1 = l.b[row * 4 + ((2 * hh + 1) ^ sw)];
  const uint2 s8 = l.s[row];
  f.s = hh ? s8.y : s8.x;
  return f;
}

template <int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void read_b(const Lds& l, BPack<TN, DUAL>& f) {
  using C = Cfg<WN, TM, TN, DUAL>;
  const int lane = threadIdx.x & 63, wn = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int row = (wn * TN + j) * 32 + r32;
    f.b[j] = read_frag(l, row, hh);
    if constexpr (DUAL) f.u[j] = read_frag(l, row + C::BN, hh);
  }
}

// Activation fragments of step S (K elements 64h + 8S .. +7 of the chunk).
template <int S, int SLOT, int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void read_a(Ctx<WN, TM, TN, DUAL>& x, const Lds& l) {
  const int hh = (threadIdx.x & 63) >> 5;
  const int slot = ((hh << 3) + S) ^ x.lds_swz;
#pragma unroll
  for (int i = 0; i < TM; ++i) x.ring[SLOT][i] = l.a[x.lds_row[i] + slot];
}

// Scheduling of one step: the LDS reads of the next step's activation
// fragments go first (their latency hides behind this step's MFMAs), then one
// MFMA alternates with a few VALU instructions (weight expansion of the next
// step), so the vector ALU work co-issues with the matrix core.
template <int NDS, int NMFMA, int NVALU>
__device__ __forceinline__ void interleave_hint() {
  if constexpr (NDS > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);  // then a few VALU
  }
}

// Step S of a chunk: MFMAs on ring[S%2] x e_cur, while the weights of step
// S+1 are expanded into e_nxt and the activations of step S+1 are read.
template <int S, int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void pipe_step(Ctx<WN, TM, TN, DUAL>& x, const Lds& l, const BPack<TN, DUAL>& f,
                                          BExp<TN, DUAL>& e_cur, BExp<TN, DUAL>& e_nxt) {
  constexpr int NMFMA = TM * TN * (DUAL ? 2 : 1);
  constexpr int NVALU = TN * (DUAL ? 2 : 1) * 9;
  if constexpr (S < 7) {
    read_a<S + 1, (S + 1) & 1>(x, l);
    expand_b<TN, DUAL, S + 1>(f, e_nxt);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      x.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S & 1][i], e_cur.b[j], x.acc[i][j], 0, 0, 0);
      if constexpr (DUAL)
        x.accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S & 1][i], e_cur.u[j], x.accu[i][j], 0, 0, 0);
    }
  interleave_hint<(S < 7 ? TM : 0), NMFMA, (S < 7 ? (NVALU + NMFMA - 1) / NMFMA : 0)>();
}

template <int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void run_chunk(Ctx<WN, TM, TN, DUAL>& x, const Lds& l) {
  BPack<TN, DUAL> f;
  BExp<TN, DUAL> e0, e1;
  read_b<WN, TM, TN, DUAL>(l, f);
  read_a<0, 0>(x, l);
  expand_b<TN, DUAL, 0>(f, e0);
  pipe_step<0>(x, l, f, e0, e1);
  pipe_step<1>(x, l, f, e1, e0);
  pipe_step<2>(x, l, f, e0, e1);
  pipe_step<3>(x, l, f, e1, e0);
  pipe_step<4>(x, l, f, e0, e1);
  pipe_step<5>(x, l, f, e1, e0);
  pipe_step<6>(x, l, f, e0, e1);
  pipe_step<7>(x, l, f, e1, e0);
}

// Tile shape of the large-batch kernels (rows per wave) and the number of
// work-groups the register budget must leave room for on one CU.
#ifndef NVFP4_GLU_TM
#define NVFP4_GLU_TM 2
#endif
#ifndef NVFP4_STORE_TM
#define NVFP4_STORE_TM 2
#endif
#ifndef NVFP4_MIN_WG_PER_CU
#define NVFP4_MIN_WG_PER_CU 2
#endif

template <int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI>
__global__ void __launch_bounds__(WN * 64, NVFP4_MIN_WG_PER_CU) gemm_kernel(GemmArgs p) {
  using C = Cfg<WN, TM, TN, DUAL>;
  constexpr int BM = C::BM;
  constexpr int BN = C::BN;
  __shared__ float red[WN];
  __shared__ f16x8 lds_a0[C::LDS_A];
  __shared__ f16x8 lds_a1[C::LDS_A];
  __shared__ u32x4 lds_b0[C::LDS_B];
  __shared__ u32x4 lds_b1[C::LDS_B];
  __shared__ uint2 lds_s0[C::NB];
  __shared__ uint2 lds_s1[C::NB];
  const int lane = threadIdx.x & 63;
  const int wn = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;

  // ---- tile: consecutive ids share (split, n_tile) and walk the m tiles ------
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t mt = t % p.m_tiles;
  const uint32_t rest = t / p.m_tiles;
  const uint32_t split = rest % p.splits;
  const uint32_t n_tile = rest / p.splits;
  int64_t m0, m_end;
  int e = 0;
  if constexpr (GROUPED) {
    // (expert, tile within the expert) from the device-resident offsets;
    // tiles past the last expert have no work.
    uint32_t cum = 0;
    m0 = -1;
    m_end = 0;
    for (int xe = 0; xe < p.E; ++xe) {
      const int64_t s0 = p.off[xe], s1 = p.off[xe + 1];
      const uint32_t nt = (uint32_t)((s1 - s0 + BM - 1) / BM);
      if (mt < cum + nt) {
        e = xe;
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
  const int64_t nchunks_total = K >> 7;
  const int64_t c_begin = (int64_t)split * p.chunks_per_split;
  int64_t nch = nchunks_total - c_begin;
  if (nch > (int64_t)p.chunks_per_split) nch = p.chunks_per_split;
  const int64_t wstride_c = GROUPED ? (int64_t)e * p.N * kb : 0;
  const int64_t wstride_s = GROUPED ? (int64_t)e * p.N * ks : 0;

  // ---- staging sources (rows past the end are clamped; never stored) ----------
  Ctx<WN, TM, TN, DUAL> x;
#pragma unroll
  for (int u = 0; u < C::SA; ++u) {
    const int pu = u * C::NT + threadIdx.x;
    const int row = pu >> 4, slot = pu & 15;
    int64_t m = m0 + row;
    if (m > m_end - 1) m = m_end - 1;
    x.a_src[u] = p.a + m * K + c_begin * 128 + ((slot ^ (row & 15)) << 3);
  }
  auto wrow = [&](int rho, const uint8_t*& codes, const uint8_t*& scales) {
    const bool up = DUAL && rho >= BN;
    int64_t n = n0 + (up ? rho - BN : rho);
    if (n > p.N - 1) n = p.N - 1;
    codes = (up ? p.u_codes : p.b_codes) + wstride_c + n * kb + c_begin * 64;
    scales = (up ? p.u_scales : p.b_scales) + wstride_s + n * ks + c_begin * 8;
  };
#pragma unroll
  for (int u = 0; u < C::SB; ++u) {
    const int pu = u * C::NT + threadIdx.x;      // LDS unit: row pu/4, slot pu%4
    const int row = pu >> 2, slot = pu & 3;
    const uint8_t *cd, *sc;
    wrow(row, cd, sc);
    x.b_src[u] = cd + ((slot ^ ((row >> 2) & 3)) << 4);
  }
#pragma unroll
  for (int u = 0; u < C::SD; ++u) {
    const int pu = u * C::NT + threadIdx.x;      // LDS dword: row pu/2, half pu%2
    const uint8_t *cd, *sc;
    wrow(pu >> 1, cd, sc);
    x.s_src[u] = sc + ((pu & 1) << 2);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) x.lds_row[i] = (i * 32 + r32) * 16;
  x.lds_swz = r32 & 15;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x.acc[i][j][r] = 0.f;
        if constexpr (DUAL) x.accu[i][j][r] = 0.f;
      }

  // ---- main loop: chunk c+1 streams into the other LDS buffer (DMA) while
  // chunk c runs; one barrier per chunk -----------------------------------------
  const Lds l0{lds_a0, lds_b0, lds_s0}, l1{lds_a1, lds_b1, lds_s1};
  stage_dma(x, l0, 0);
  __builtin_amdgcn_s_waitcnt(0);     // vmcnt(0): this wave's copies have landed
  __builtin_amdgcn_s_barrier();
  for (int64_t c = 0; c < nch; c += 2) {
    if (c + 1 < nch) stage_dma(x, l1, c + 1);
    run_chunk(x, l0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    if (c + 1 >= nch) break;
    if (c + 2 < nch) stage_dma(x, l0, c + 2);
    run_chunk(x, l1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  }

  // ---- epilogue ---------------------------------------------------------------------
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
        const int64_t row = m0 + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < m_end && col < p.N) {
          if constexpr (EPI == EPI_GLU) {
            const float hv = silu_mul(x.acc[i][j][r] * alpha, x.accu[DUAL ? i : 0][DUAL ? j : 0][r] * alpha_u);
            p.h[row * p.N + col] = hv;
            hmax = fmaxf(hmax, fabsf(hv));
          } else {
            if (p.splits > 1) {
              p.split_out[((int64_t)split * p.M + row) * p.N + col] = x.acc[i][j][r];
            } else {
              const float v = x.acc[i][j][r] * alpha;
              if (p.c_bf16)
                reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] = (uint16_t)f32_to_bf16_bits(v);
              else
                reinterpret_cast<float*>(p.c)[row * p.ldc + col] = v;
            }
          }
        }
      }
    }
  if constexpr (EPI == EPI_GLU) {
    hmax = block_max(hmax, red);
    if (threadIdx.x == 0) p.partials[blockIdx.x] = hmax;
  }
}

// out[m][n] = (sum over splits, in split order) * gs_a * gs_b[expert of slot m].
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, uint32_t splits,
                                                            int64_t M, int64_t N, const float* a_gs,
                                                            const float* b_gs, const int32_t* off, int E,
                                                            void* out, int out_bf16, int64_t ldo) {
  const int64_t total = M * N;
  const float ga = a_gs[0];
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / N, n = idx - m * N;
    float acc = 0.f;
    for (uint32_t s = 0; s < splits; ++s) acc += part[(int64_t)s * total + idx];
    int e = 0;
    if (off) {
      while (e < E - 1 && off[e + 1] <= m) ++e;
    }
    const float v = acc * (ga * b_gs[e]);
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[m * ldo + n] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(out)[m * ldo + n] = v;
  }
}

// ---- launch configurations ----------------------------------------------------------
// Large batches: four waves side by side in N, each 128 rows x 32 columns
// (x2 with the gate/up pair).  Small batches (M <= 32): 32-row tiles, two
// waves per work-group to spread the weight stream over more work-groups.
struct Plan {
  bool small;
  uint32_t m_tiles, n_tiles, splits, chunks_per_split;
};

static uint32_t cdiv(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

static Plan plan_store(int64_t M, int64_t N, int64_t K, int E, bool grouped) {
  Plan pl{};
  pl.small = !grouped && M <= 32;
  const int64_t bm = pl.small ? 32 : 32 * NVFP4_STORE_TM;
  const int64_t bn = pl.small ? 64 : 128;
  pl.m_tiles = grouped ? cdiv(M, 32 * NVFP4_STORE_TM) + (uint32_t)E : cdiv(M, bm);
  pl.n_tiles = cdiv(N, bn);
  const uint32_t chunks = (uint32_t)(K / 128);
  // Split K until there are >= ~3 work-groups per CU, keeping >= 8 chunks per split.
  const uint32_t tiles = pl.m_tiles * pl.n_tiles;
  uint32_t s = 1;
  while (s < 8 && tiles * s < 768 && chunks / (s + 1) >= 8) ++s;
  pl.chunks_per_split = cdiv(chunks, s);
  pl.splits = cdiv(chunks, pl.chunks_per_split);
  return pl;
}

template <int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI>
static void launch_cfg(const GemmArgs& g, hipStream_t st) {
  const uint32_t grid = g.m_tiles * g.n_tiles * g.splits;
  const int slot = launch_begin(EPI == EPI_GLU ? KC_GEMM_GLU : KC_GEMM_STORE, st);
  hipLaunchKernelGGL((gemm_kernel<WN, TM, TN, DUAL, GROUPED, EPI>), dim3(grid), dim3(WN * 64), 0, st, g);
  launch_end(slot, st);
}

static void launch_expand(const uint8_t* codes, const uint8_t* scales, const int32_t* rows, int64_t nrows,
                          int64_t cols, _Float16* out, hipStream_t st) {
  const uint32_t nbc = (uint32_t)(cols / 16);
  const uint32_t nblocks = (uint32_t)nrows * nbc;
  uint32_t grid = (nblocks + 255u) / 256u;
  if (grid > 4096u) grid = 4096u;
  if (grid < 1u) grid = 1u;
  const int slot = launch_begin(KC_EXPAND, st);
  hipLaunchKernelGGL(expand_kernel, dim3(grid), dim3(256), 0, st, codes, scales, rows, nbc, nblocks, out);
  launch_end(slot, st);
}

static void launch_reduce(const float* part, uint32_t splits, int64_t M, int64_t N, const float* a_gs,
                          const float* b_gs, const int32_t* off, int E, void* out, int bf16, int64_t ldo,
                          hipStream_t st) {
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const int slot = launch_begin(KC_REDUCE, st);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, part, splits, M, N, a_gs,
                     b_gs, off, E, out, bf16, ldo);
  launch_end(slot, st);
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static GemmArgs base_args(const _Float16* a16, const float* a_gs, Operand b, int64_t M, int64_t N, int64_t K) {
  GemmArgs g{};
  g.a = a16;
  g.a_gs = a_gs;
  g.b_codes = b.codes;
  g.b_scales = b.scales;
  g.b_gs = b.gscale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.splits = 1;
  return g;
}

// Store-epilogue GEMM (dense or grouped).  Workspace: [A f16 M x K][split partials].
size_t store_ws_bytes(int64_t M, int64_t N, int64_t K, int E, bool grouped) {
  const Plan pl = plan_store(M, N, K, E, grouped);
  return align256((size_t)M * K * 2) + align256((size_t)pl.splits * M * N * 4);
}

int store_launch(Operand a, const int32_t* rows, const int32_t* off, int E, int64_t M, Operand w, int64_t N,
                 int64_t K, void* c, int c_bf16, int64_t ldc, void* ws, hipStream_t st) {
  const bool grouped = off != nullptr;
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)M * K * 2));
  launch_expand(a.codes, a.scales, rows, M, K, a16, st);
  const Plan pl = plan_store(M, N, K, E, grouped);
  GemmArgs g = base_args(a16, a.gscale, w, M, N, K);
  g.c = c;
  g.ldc = ldc;
  g.c_bf16 = c_bf16;
  g.splits = pl.splits;
  g.chunks_per_split = pl.chunks_per_split;
  g.split_out = part;
  g.off = off;
  g.E = E;
  g.m_tiles = pl.m_tiles;
  g.n_tiles = pl.n_tiles;
  if (grouped) launch_cfg<4, NVFP4_STORE_TM, 1, false, true, EPI_STORE>(g, st);
  else if (pl.small) launch_cfg<2, 1, 1, false, false, EPI_STORE>(g, st);
  else launch_cfg<4, NVFP4_STORE_TM, 1, false, false, EPI_STORE>(g, st);
  // The reduction always runs (over zero rows when K was not split), so the
  // number of launches never depends on the shape.
  launch_reduce(part, pl.splits, pl.splits > 1 ? M : 0, N, a.gscale, w.gscale, off, E, c, c_bf16, ldc, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

// GLU GEMM.  Workspace: [H float32 M x N][A f16 M x K][partials].
static uint32_t glu_parts(int64_t M, int64_t N, int E, bool grouped) {
  if (grouped) return (cdiv(M, 32 * NVFP4_GLU_TM) + (uint32_t)E) * cdiv(N, 128);
  if (M <= 32) return cdiv(M, 32) * cdiv(N, 64);
  return cdiv(M, 32 * NVFP4_GLU_TM) * cdiv(N, 128);
}

size_t glu_ws_bytes(int64_t M, int64_t N, int64_t K, int E, bool grouped) {
  return align256((size_t)M * N * 4) + align256((size_t)M * K * 2) + align256((size_t)glu_parts(M, N, E, grouped) * 4);
}

int glu_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt, Operand up,
               int64_t N, int64_t K, uint8_t* hq_codes, uint8_t* hq_scales, float* hq_gs, void* ws,
               hipStream_t st) {
  const bool grouped = off != nullptr;
  float* h = reinterpret_cast<float*>(ws);
  _Float16* a16 = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(ws) + align256((size_t)M * N * 4));
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a16) + align256((size_t)M * K * 2));
  launch_expand(a.codes, a.scales, a_rows, M, K, a16, st);
  GemmArgs g = base_args(a16, a.gscale, gt, M, N, K);
  g.u_codes = up.codes;
  g.u_scales = up.scales;
  g.u_gs = up.gscale;
  g.h = h;
  g.partials = partials;
  g.off = off;
  g.E = E;
  g.chunks_per_split = (uint32_t)(K / 128);
  if (grouped) {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM) + (uint32_t)E;
    g.n_tiles = cdiv(N, 128);
    launch_cfg<4, NVFP4_GLU_TM, 1, true, true, EPI_GLU>(g, st);
  } else if (M <= 32) {
    g.m_tiles = cdiv(M, 32);
    g.n_tiles = cdiv(N, 64);
    launch_cfg<2, 1, 1, true, false, EPI_GLU>(g, st);
  } else {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM);
    g.n_tiles = cdiv(N, 128);
    launch_cfg<4, NVFP4_GLU_TM, 1, true, false, EPI_GLU>(g, st);
  }
  if (hipGetLastError() != hipSuccess) return 7;
  return requant_f32_launch(h, M, N, hq_codes, hq_scales, hq_gs, partials, glu_parts(M, N, E, grouped), st);
}

}  // namespace nvfp4
