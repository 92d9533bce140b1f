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
#include <atomic>
#include <type_traits>

namespace nvfp4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const _Float16* a;      // expanded activations, f16 [rows][K] (slot order when grouped)
  const uint8_t* a_codes; // the activation itself, NVFP4 [M][K] (the weight streams expand it in registers)
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
  float* split_out;       // [splits][M][N] float32 partial sums (splits > 1)
  const int32_t* off;
  int E;
  uint32_t m_tiles;       // dense: ceil(M/BM); grouped: static bound on the expert tiles
  uint32_t n_tiles;
  uint32_t splits;
  uint32_t chunks_per_split;
  int force_split;        // store epilogue: write split_out even when splits == 1
  uint8_t* q_codes;       // EPI_GLUQ output [M][N] NVFP4 and its given global scale
  uint8_t* q_scales;
  const float* q_gs;
  _Float16* q16;          // EPI_GLUQ (nullable): the f16 copy of the quantised output, code * scale
  // Split-K finished inside the weight streams (store epilogue, split_out
  // written): one ticket per column group, cleared by an earlier launch; the
  // wave (or work-group) of a group that arrives last adds the group's partial
  // sums in split order and stores the outputs.  amax_slots (nullable, cleared
  // too): max |stored output| of each group folded into slot group % kAmaxSlots.
  uint32_t* tickets;
  float* amax_slots;
  // Optional tile-contiguous copies of the weights (gate / up) that the
  // large-batch kernels stage from instead of the row-major codes and scales.
  const uint8_t* b_tiled;
  const uint8_t* u_tiled;
  // Expert-grouped gather (nullable): slot s stages activation row a_gather[s]
  // of the f16 copy at `a` ([a_gather_rows][K]) instead of row s.
  const int32_t* a_gather;
  int64_t a_gather_rows;
};

// Partial sums shared between the work-groups of one launch go through the
// device-coherent level (agent-scope accesses: the stores write through the
// XCD's L2, the loads miss in it), so no L2 write-back or invalidation is
// needed between them -- agent-scope fences per wave cost about 25 ns each,
// serialised, which is most of a decode call at thousands of waves.  The
// ordering that a fence would give comes from the hardware: a writer waits
// until its stores are acknowledged (vmcnt) before it takes its ticket, and
// the last arriver issues its loads only after its ticket returned.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every store of this wave acknowledged (and no memory access moved across)
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// Output (t, c) = sum * gs_a * gs_b stored (float32 or bf16); returns |stored value|.
__device__ __forceinline__ float store_output(const GemmArgs& p, int64_t t, int64_t c, float sum) {
  const float v = sum * (p.a_gs[0] * p.b_gs[0]);
  if (p.c_bf16) {
    const uint32_t b = f32_to_bf16_bits(v);
    reinterpret_cast<uint16_t*>(p.c)[t * p.ldc + c] = (uint16_t)b;
    return fabsf(__uint_as_float(b << 16));
  }
  reinterpret_cast<float*>(p.c)[t * p.ldc + c] = v;
  return fabsf(v);
}

// Output (t, c) of a split-K store: the partial sums in split order (the
// order and arithmetic of the reduction kernels), scaled by gs_a * gs_b and
// stored; returns |stored value|.  Loads go eight splits at a time.
__device__ __forceinline__ float finish_output(const GemmArgs& p, int64_t t, int64_t c) {
  const int64_t plane = p.M * p.N, idx = t * p.N + c;
  float acc = 0.f;
  uint32_t s = 0;
  for (; s + 8u <= p.splits; s += 8u) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_coherent(p.split_out + (int64_t)(s + k) * plane + idx);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += v[k];
  }
  for (; s < p.splits; ++s) acc += load_coherent(p.split_out + (int64_t)s * plane + idx);
  return store_output(p, t, c, acc);
}

// Ticket of a column group after this caller's partial sums are stored and
// acknowledged (one lane per wave, or one thread per work-group); true for the
// arrival that completes the group.  No waiting: the others just leave.
__device__ __forceinline__ bool last_arrival(uint32_t* ticket, uint32_t count) {
  return __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == count - 1u;
}

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

// ---- tile-contiguous weight copy ----------------------------------------------------
// One work-group per block (e, g, c): 128 rows x 128 K of a weight [E][N][K].
// Its 512 code units (16 bytes, 32 codes) go where the large-batch kernels'
// staging puts them in LDS -- unit u of row r at r * 4 + (u ^ ((r / 4) % 4)) --
// and its 128 rows of 8 scale bytes follow in row order, so that staging a
// chunk of a column tile is a run of whole 1 KiB pieces.  Rows past N are
// zero.  A permutation of the weight's bytes: no value changes.
__global__ void __launch_bounds__(256) tile_weight_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales, int64_t N, int64_t K,
                                                          int64_t G, uint8_t* __restrict__ out) {
  const int64_t Cn = K / kTileK;
  const int64_t blk = blockIdx.x;
  const int64_t c = blk % Cn, eg = blk / Cn, g = eg % G, e = eg / G;
  const int64_t kb = K / 2, ks = K / 16;
  uint8_t* dst = out + blk * kTileBlock;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = (int)threadIdx.x + 256 * j;
    const int r = q >> 2, u = (q & 3) ^ ((r >> 2) & 3);
    const int64_t n = g * kTileRows + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) v = *reinterpret_cast<const uint4*>(codes + (e * N + n) * kb + c * 64 + u * 16);
    *reinterpret_cast<uint4*>(dst + q * 16) = v;
  }
  if (threadIdx.x < kTileRows) {
    const int64_t n = g * kTileRows + threadIdx.x;
    uint2 v = make_uint2(0u, 0u);
    if (n < N) v = *reinterpret_cast<const uint2*>(scales + (e * N + n) * ks + c * 8);
    *reinterpret_cast<uint2*>(dst + 8192 + threadIdx.x * 8) = v;
  }
}

size_t tile_weight_bytes(int64_t E, int64_t N, int64_t K) {
  return (size_t)(E * ((N + kTileRows - 1) / kTileRows) * (K / kTileK) * kTileBlock);
}

int tile_weight_launch(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N, int64_t K, uint8_t* out,
                       hipStream_t st) {
  const int64_t G = (N + kTileRows - 1) / kTileRows;
  const int64_t blocks = E * G * (K / kTileK);
  if (blocks <= 0) return 0;
  const int slot = launch_begin(KC_EXPAND, st);
  hipLaunchKernelGGL(tile_weight_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, codes, scales, N, K, G, out);
  launch_end(slot, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
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

// EPI_GLUQ: the GLU output quantised in the epilogue with a given global
// scale (no float32 H, no requantisation launch).
enum { EPI_STORE = 0, EPI_GLU = 1, EPI_GLUQ = 2 };

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
  // Staging sources: buffer descriptors (wave-uniform, based at this tile's
  // first row and this split's first chunk) and each lane's byte offset of
  // every staged unit; a chunk adds a scalar offset.
  i32x4 ra, rb, ru, rsb, rsu;
  uint32_t wstep, sstep;         // bytes between consecutive chunks of the weight codes / scales
  uint32_t a_off[C::SA];
  uint32_t b_off[C::SB];
  uint32_t s_off[C::SD];
  f16x8 ring[4][TM];             // activation fragments, slot = step % 4
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
// from global memory into one LDS buffer (LDS DMA: no registers, no LDS
// store instructions).  Lane l of a wave writes the 16 (or 4) bytes at LDS
// unit base + l, so each unit's global source is chosen to realise the
// swizzled layout described above.
//
// The copies are buffer loads with the LDS bit, issued from inline assembly:
// lane offsets are fixed, the chunk offset is a scalar operand and M0 (the
// wave's LDS destination) a scalar, so a chunk costs no vector ALU work.  The
// compiler does not see these copies, so it neither waits for them nor moves
// LDS reads across the explicit waits (vmcnt + barrier, below) that order
// them.  Nothing else in these kernels uses M0 (gfx950 LDS instructions do not
// read it and no register is indexed dynamically), so clobbering it is safe.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// Raw buffer descriptor over `bytes` bytes at p (gfx9 family: dword3
// 0x00020000, stride 0), made wave-uniform.
__device__ __forceinline__ i32x4 buf_desc(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)(size_t)p;
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xFFFFu));
  d[2] = __builtin_amdgcn_readfirstlane(n);
  d[3] = 0x00020000;
  return d;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// (soff and lds are wave-uniform and made scalar here; the offset goes
// through a scratch SGPR because a constant would otherwise be printed as a
// literal, which the instruction does not accept.)
__device__ __forceinline__ void dma_b128(const i32x4& r, uint32_t voff, uint32_t soff, uint32_t lds) {
  soff = __builtin_amdgcn_readfirstlane(soff);
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t t;
  asm volatile("s_mov_b32 m0, %[l]\n\ts_mov_b32 %[t], %[so]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[vo], %[r], %[t] offen lds"
               : [t] "=&s"(t) : [vo] "v"(voff), [r] "s"(r), [so] "s"(soff), [l] "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const i32x4& r, uint32_t voff, uint32_t soff, uint32_t lds) {
  soff = __builtin_amdgcn_readfirstlane(soff);
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t t;
  asm volatile("s_mov_b32 m0, %[l]\n\ts_mov_b32 %[t], %[so]\n\ts_nop 0\n\tbuffer_load_dword %[vo], %[r], %[t] offen lds"
               : [t] "=&s"(t) : [vo] "v"(voff), [r] "s"(r), [so] "s"(soff), [l] "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// la / lb / ls: this wave's LDS byte address in the buffer's activation,
// weight-code and scale arrays.
template <int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void stage_dma(const Ctx<WN, TM, TN, DUAL>& x, uint32_t la, uint32_t lb, uint32_t ls,
                                          int64_t chunk) {
  using C = Cfg<WN, TM, TN, DUAL>;
  const uint32_t ca = (uint32_t)chunk * 256u, cb = (uint32_t)chunk * x.wstep, cs = (uint32_t)chunk * x.sstep;
#pragma unroll
  for (int u = 0; u < C::SA; ++u) dma_b128(x.ra, x.a_off[u], ca, la + u * C::NT * 16);
#pragma unroll
  for (int u = 0; u < C::SB; ++u)   // units 0 .. 2TN-1 hold gate rows, the rest up rows
    dma_b128((DUAL && u >= 2 * TN) ? x.ru : x.rb, x.b_off[u], cb, lb + u * C::NT * 16);
#pragma unroll
  for (int u = 0; u < C::SD; ++u)   // units 0 .. TN-1 hold gate rows
    dma_b32((DUAL && u >= TN) ? x.rsu : x.rsb, x.s_off[u], cs, ls + u * C::NT * 4);
}

// Wait until at most `later` chunks' copies of this wave are in flight (all
// older ones have landed in LDS), then synchronise the work-group: after it,
// every wave's share of those chunks is visible and every wave has finished
// reading the buffer the next copy overwrites.
template <int PER, int MAXLATER>
__device__ __forceinline__ void ring_wait(int64_t later) {
  if (MAXLATER >= 2 && later >= 2)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(2 * PER) : "memory");
  else if (MAXLATER >= 1 && later >= 1)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(PER) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
  __builtin_amdgcn_sched_barrier(0);
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
    read_a<S + 1, (S + 1) % 4>(x, l);
    expand_b<TN, DUAL, S + 1>(f, e_nxt);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      x.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S % 4][i], e_cur.b[j], x.acc[i][j], 0, 0, 0);
      if constexpr (DUAL)
        x.accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S % 4][i], e_cur.u[j], x.accu[i][j], 0, 0, 0);
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

// ---- the cross-chunk pipeline (two LDS buffers) ---------------------------------------
// Step S of chunk c (buffer lc; chunk c+1 lives in ln): the MFMAs of step S
// use activation slot S%4 and the expanded weights e_cur, while the
// activations of step S+2 are read (from ln for S >= 6) and the weights of
// step S+1 are expanded (chunk c+1's first step for S = 7).  At S = 6 the
// work-group synchronises once: chunk c+1's copy has landed (vmcnt) and
// every wave has finished reading lc (lgkmcnt: the reads for steps 6 and 7
// were issued at steps 4 and 5), so the copy of chunk c+2 goes into lc and
// chunk c+1's packed weights are read from ln.  No step waits on a chunk
// boundary.  Reads of ln past the last chunk fetch stale data that is never
// used.
template <int S, int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void xstep(Ctx<WN, TM, TN, DUAL>& x, const Lds& lc, const Lds& ln,
                                      const BPack<TN, DUAL>& fc, BPack<TN, DUAL>& fn, BExp<TN, DUAL>& e_cur,
                                      BExp<TN, DUAL>& e_nxt, bool refill, int64_t chunk2, uint32_t da, uint32_t db,
                                      uint32_t ds) {
  constexpr int NMFMA = TM * TN * (DUAL ? 2 : 1);
  constexpr int NVALU = TN * (DUAL ? 2 : 1) * 9;
  constexpr int NDS = TM + (S == 6 ? 3 * TN * (DUAL ? 2 : 1) : 0);
  // Gate/up: the wave issues steps 2-5 at raised priority and returns to the
  // normal one before the chunk barrier, so the SIMD's arbiter favours a wave
  // in the middle of its MFMA steps over one leaving or arriving at the
  // barrier (same box: gate/up 310.8 -> 308.5 us; steps 0-5 305.4 against
  // 311.0 on another; the store kernel measured slower with it).
  if constexpr (DUAL && S == 2) __builtin_amdgcn_s_setprio(1);
  if constexpr (DUAL && S == 6) __builtin_amdgcn_s_setprio(0);
  if constexpr (S == 6) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (refill) stage_dma(x, da, db, ds, chunk2);
    read_b<WN, TM, TN, DUAL>(ln, fn);
  }
  if constexpr (S + 2 < 8) read_a<S + 2, (S + 2) % 4>(x, lc);
  else read_a<S - 6, (S + 2) % 4>(x, ln);
  if constexpr (S + 1 < 8) expand_b<TN, DUAL, S + 1>(fc, e_nxt);
  else expand_b<TN, DUAL, 0>(fn, e_nxt);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      x.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S % 4][i], e_cur.b[j], x.acc[i][j], 0, 0, 0);
      if constexpr (DUAL)
        x.accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x.ring[S % 4][i], e_cur.u[j], x.accu[i][j], 0, 0, 0);
    }
  interleave_hint<NDS, NMFMA, (NVALU + NMFMA - 1) / NMFMA>();
}

template <int WN, int TM, int TN, bool DUAL>
__device__ __forceinline__ void xchunk(Ctx<WN, TM, TN, DUAL>& x, const Lds& lc, const Lds& ln,
                                       const BPack<TN, DUAL>& fc, BPack<TN, DUAL>& fn, BExp<TN, DUAL>& e0,
                                       BExp<TN, DUAL>& e1, bool refill, int64_t chunk2, uint32_t da, uint32_t db,
                                       uint32_t ds) {
  xstep<0>(x, lc, ln, fc, fn, e0, e1, refill, chunk2, da, db, ds);
  xstep<1>(x, lc, ln, fc, fn, e1, e0, refill, chunk2, da, db, ds);
  xstep<2>(x, lc, ln, fc, fn, e0, e1, refill, chunk2, da, db, ds);
  xstep<3>(x, lc, ln, fc, fn, e1, e0, refill, chunk2, da, db, ds);
  xstep<4>(x, lc, ln, fc, fn, e0, e1, refill, chunk2, da, db, ds);
  xstep<5>(x, lc, ln, fc, fn, e1, e0, refill, chunk2, da, db, ds);
  xstep<6>(x, lc, ln, fc, fn, e0, e1, refill, chunk2, da, db, ds);
  xstep<7>(x, lc, ln, fc, fn, e1, e0, refill, chunk2, da, db, ds);
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
// Work-groups the split-K plan of the store epilogue aims for: about two
// rounds of the 512 resident work-groups.  The 1024-token down projection
// (320 tiles) then takes 4 splits; with tiled weights 4 measured faster than
// 3 (10.47 -> 10.21 ms of down projection per long-prefill step, same box)
// and 5 or 6 slower.
#ifndef NVFP4_SPLIT_TARGET
#define NVFP4_SPLIT_TARGET 1000
#endif
// Waves per work-group of the large-batch kernels (side by side in N).
#ifndef NVFP4_GLU_WN
#define NVFP4_GLU_WN 4
#endif
#ifndef NVFP4_STORE_WN
#define NVFP4_STORE_WN 4
#endif
// 32-column sub-tiles per wave of the store-epilogue kernels: two give every
// activation fragment read from LDS two MFMAs, as the gate/up pair does.
#ifndef NVFP4_STORE_TN
#define NVFP4_STORE_TN 2
#endif
#ifndef NVFP4_GROUPED_STORE_TN
#define NVFP4_GROUPED_STORE_TN 2
#endif
// LDS buffers of the chunk ring (2 to 4).
#ifndef NVFP4_GLU_STAGES
#define NVFP4_GLU_STAGES 2
#endif
#ifndef NVFP4_STORE_STAGES
#define NVFP4_STORE_STAGES 2
#endif
#ifndef NVFP4_GLU_MINWG
#define NVFP4_GLU_MINWG NVFP4_MIN_WG_PER_CU
#endif
#ifndef NVFP4_STORE_MINWG
#define NVFP4_STORE_MINWG NVFP4_MIN_WG_PER_CU
#endif

constexpr uint32_t kGroupGm = 8;   // m tiles per super-tile of the expert-grouped tile order
// m tiles per super-tile of the dense, unsplit tile order (0: all m tiles of
// one n tile, then the next n tile).  With 4, the 64 work-groups resident on
// one XCD cover 4 m tiles x 16 n tiles instead of 16 x 4, which reads fewer
// activation tiles past its L2.
#ifndef NVFP4_DENSE_GROUP_M
#define NVFP4_DENSE_GROUP_M 4
#endif

// Work-groups of the dense large-batch kernels are persistent: work-group b
// takes the tiles v = b, b + grid, b + 2 grid, ... of the launch's tile order
// (grid = the work-groups the chip holds at once), and with the two-buffer
// pipeline and a register epilogue it issues the copies of its next tile's
// first two chunks before it writes the current tile's outputs, so that their
// latency hides behind the epilogue instead of following a new work-group's
// start.  Every tile's arithmetic and its order are those it has on a
// work-group of its own.  Measured on the 1024-token gate/up (4.25 tiles per
// work-group): 300-303 against 307 us.  The expert-grouped kernels keep one
// work-group per tile: with 18 tiles per work-group the work-groups of an XCD
// drift apart over the fixed stride, its tiles in flight spread out, and the
// 64-expert layer measured 1.93 against 1.89-1.90 ms.  0: one work-group per
// tile everywhere.
#ifndef NVFP4_PERSIST
#define NVFP4_PERSIST 1
#endif
#ifndef NVFP4_PERSIST_GROUPED
#define NVFP4_PERSIST_GROUPED 0
#endif

// A tile of the launch: K split, first row and row end (the expert's end for
// expert groups; m0 < 0: a tile past the last expert, no work), first column,
// expert.
struct TileLoc {
  int64_t m0, m_end, n0;
  uint32_t split;
  int e;
};

// Tile order: K splits slowest, then super-tiles of kGm m tiles x all n tiles
// (m fastest inside), so that the work-groups resident on one XCD work on one
// K range and share both activation rows and weight columns in its L2 (for
// expert groups the gathered activations of all experts do not fit the
// MALL); kGm = 0: m fastest, then n.  Virtual tile v is dealt to the XCD that
// runs work-group v % 8 (xcd_remap).  Expert groups: the launch covers a
// static bound on the m tiles, but only the experts' own m tiles (their row
// counts rounded up to BM, read from the device-resident offsets) enter the
// order, so that every XCD gets an equal share of the tiles that have work;
// virtual tiles past them have none (m0 < 0).
template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ TileLoc locate_tile(const GemmArgs& p, uint32_t v, uint32_t vtotal) {
  TileLoc L;
  L.e = 0;
  L.m0 = -1;
  L.m_end = 0;
  L.split = 0;
  L.n0 = 0;
  uint32_t m_tiles = p.m_tiles;
  const int lane = threadIdx.x & 63;
  if constexpr (GROUPED) {
    // the experts' m tiles: the lanes of each wave take 64 experts at a time
    uint32_t real = 0;
    for (int g0 = 0; g0 < p.E; g0 += 64) {
      const int xe = g0 + lane;
      const int32_t s0 = xe < p.E ? p.off[xe] : 0;
      const int32_t s1 = xe < p.E ? p.off[xe + 1] : 0;
      real += (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_sum_u32((uint32_t)((s1 - s0 + BM - 1) / BM)));
    }
    m_tiles = real < p.m_tiles ? real : p.m_tiles;
    vtotal = m_tiles * p.n_tiles * p.splits;
    if (v >= vtotal) return L;
  }
  const uint32_t t = xcd_remap(v, vtotal);
  uint32_t mt, n_tile;
  constexpr uint32_t kGm = GROUPED ? kGroupGm : (uint32_t)NVFP4_DENSE_GROUP_M;
  const uint32_t per_split = m_tiles * p.n_tiles;
  L.split = t / per_split;
  const uint32_t u = t - L.split * per_split;
  if (kGm > 0) {
    const uint32_t span = kGm * p.n_tiles;
    const uint32_t sup = u / span, r = u - sup * span;
    const uint32_t gm = (sup + 1) * kGm <= m_tiles ? kGm : m_tiles - sup * kGm;
    mt = sup * kGm + r % gm;
    n_tile = r / gm;
  } else {
    mt = u % m_tiles;
    n_tile = u / m_tiles;
  }
  L.n0 = (int64_t)n_tile * BN;
  if constexpr (GROUPED) {
    // (expert, tile within the expert): the lanes add up the experts' tile
    // counts with a wave prefix sum, and the first expert whose running count
    // passes the tile wins
    uint32_t cum = 0;
    for (int g0 = 0; g0 < p.E; g0 += 64) {
      const int xe = g0 + lane;
      const int32_t s0 = xe < p.E ? p.off[xe] : 0;
      const int32_t s1 = xe < p.E ? p.off[xe + 1] : 0;
      const uint32_t nt = (uint32_t)((s1 - s0 + BM - 1) / BM);
      uint32_t incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t w = __shfl_up(incl, d, 64);
        if (lane >= d) incl += w;
      }
      const uint32_t group = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
      if (mt < cum + group) {                      // wave-uniform
        const uint64_t hit = __ballot(cum + incl > mt);
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
        L.e = g0 + l;
        const uint32_t before = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(incl - nt, l, 64));
        L.m0 = (int64_t)__builtin_amdgcn_readfirstlane(__shfl(s0, l, 64)) + (int64_t)(mt - cum - before) * BM;
        L.m_end = (int64_t)__builtin_amdgcn_readfirstlane(__shfl(s1, l, 64));
        break;
      }
      cum += group;
    }
  } else {
    L.m0 = (int64_t)mt * BM;
    L.m_end = p.M;
  }
  return L;
}

// Staging sources of one tile (from chunk c_begin of its K split), in two
// parts: the buffer descriptors (wave-uniform; rebuilt wherever a tile's
// copies are issued, so that no descriptor is carried around the tile loop,
// which would move it out of the scalar registers the copies need), and each
// lane's byte offset of every unit it copies.  Rows past the end are clamped
// (staged, never stored).
template <int WN, int TM, int TN, bool DUAL, bool GROUPED>
__device__ __forceinline__ void tile_desc(Ctx<WN, TM, TN, DUAL>& x, const GemmArgs& p, const TileLoc& L,
                                          int64_t c_begin) {
  using C = Cfg<WN, TM, TN, DUAL>;
  constexpr int BM = C::BM;
  constexpr int BN = C::BN;
  const int64_t m0 = L.m0, m_end = L.m_end, n0 = L.n0;
  const int64_t K = p.K;
  const int64_t kb = K >> 1, ks = K >> 4;
  const int64_t wstride_c = GROUPED ? (int64_t)L.e * p.N * kb : 0;
  const int64_t wstride_s = GROUPED ? (int64_t)L.e * p.N * ks : 0;
  // uniform: the weights come from their tile-contiguous copies (both of the pair)
  const bool tiled = p.b_tiled != nullptr && (!DUAL || p.u_tiled != nullptr);
  const int64_t a_rows = (m_end < m0 + BM ? m_end : m0 + BM) - m0;
  x.ra = buf_desc(p.a + m0 * K + c_begin * 128, a_rows * K * 2 - c_begin * 256);
  if constexpr (GROUPED) {
    if (p.a_gather != nullptr)   // uniform: the slots' rows are staged from the token copy directly
      x.ra = buf_desc(p.a + c_begin * 128, p.a_gather_rows * K * 2 - c_begin * 256);
  }
  if (tiled) {
    // blocks (e, g, c): this tile's first group g0 = n0 / 128, from chunk c_begin on
    const int64_t G = (p.N + kTileRows - 1) / kTileRows, Cn = K / kTileK;
    const int64_t first = ((GROUPED ? (int64_t)L.e * G : 0) + n0 / kTileRows) * Cn + c_begin;
    const int64_t bytes = ((G - n0 / kTileRows) * Cn - c_begin) * kTileBlock;
    x.rb = buf_desc(p.b_tiled + first * kTileBlock, bytes);
    x.rsb = buf_desc(p.b_tiled + first * kTileBlock + 8192, bytes - 8192);
    if constexpr (DUAL) {
      x.ru = buf_desc(p.u_tiled + first * kTileBlock, bytes);
      x.rsu = buf_desc(p.u_tiled + first * kTileBlock + 8192, bytes - 8192);
    } else {
      x.ru = x.rb;
      x.rsu = x.rsb;
    }
    x.wstep = x.sstep = (uint32_t)kTileBlock;
  } else {
    const int64_t b_rows = (p.N < n0 + BN ? p.N : n0 + BN) - n0;
    x.rb = buf_desc(p.b_codes + wstride_c + n0 * kb + c_begin * 64, b_rows * kb - c_begin * 64);
    x.rsb = buf_desc(p.b_scales + wstride_s + n0 * ks + c_begin * 8, b_rows * ks - c_begin * 8);
    if constexpr (DUAL) {
      x.ru = buf_desc(p.u_codes + wstride_c + n0 * kb + c_begin * 64, b_rows * kb - c_begin * 64);
      x.rsu = buf_desc(p.u_scales + wstride_s + n0 * ks + c_begin * 8, b_rows * ks - c_begin * 8);
    } else {
      x.ru = x.rb;
      x.rsu = x.rsb;
    }
    x.wstep = 64u;
    x.sstep = 8u;
  }
}

template <int WN, int TM, int TN, bool DUAL, bool GROUPED>
__device__ __forceinline__ void tile_offsets(Ctx<WN, TM, TN, DUAL>& x, const GemmArgs& p, const TileLoc& L) {
  using C = Cfg<WN, TM, TN, DUAL>;
  constexpr int BN = C::BN;
  const int64_t m0 = L.m0, m_end = L.m_end, n0 = L.n0;
  const int64_t K = p.K;
  const int64_t kb = K >> 1, ks = K >> 4;
  const bool tiled = p.b_tiled != nullptr && (!DUAL || p.u_tiled != nullptr);
  const bool gather = GROUPED && p.a_gather != nullptr;   // uniform
#pragma unroll
  for (int u = 0; u < C::SA; ++u) {
    const int pu = u * C::NT + threadIdx.x;
    const int row = pu >> 4, slot = pu & 15;
    int64_t m = m0 + row;
    if (m > m_end - 1) m = m_end - 1;
    const int64_t src = gather ? (int64_t)p.a_gather[m] : m - m0;
    x.a_off[u] = (uint32_t)((src * K + ((slot ^ (row & 15)) << 3)) * 2);
  }
  auto wrow = [&](int rho) -> int64_t {          // row of this tile's gate (or up) matrix, clamped
    int64_t n = n0 + ((DUAL && rho >= BN) ? rho - BN : rho);
    if (n > p.N - 1) n = p.N - 1;
    return n - n0;
  };
  // tiled: row rho of the tile (gate rows first with the pair) is row rho % 128
  // of group min(g0 + (rho mod BN) / 128, G - 1); a block holds the LDS order of
  // its 128 rows, so LDS unit (dword) q of a group is byte 16 q (8192 + 4 q)
  const int64_t tgrp_last = tiled ? (p.N + kTileRows - 1) / kTileRows - 1 - n0 / kTileRows : 0;
  auto tgrp = [&](int rho) -> int64_t {          // group of tile row rho, relative to g0, clamped
    const int64_t g = ((DUAL && rho >= BN) ? rho - BN : rho) / kTileRows;
    return (g < tgrp_last ? g : tgrp_last) * (K / kTileK) * kTileBlock;
  };
#pragma unroll
  for (int u = 0; u < C::SB; ++u) {
    const int pu = u * C::NT + threadIdx.x;      // LDS unit: row pu/4, slot pu%4
    const int row = pu >> 2, slot = pu & 3;
    x.b_off[u] = tiled ? (uint32_t)(tgrp(row) + (int64_t)(pu & 511) * 16)
                       : (uint32_t)(wrow(row) * kb + ((slot ^ ((row >> 2) & 3)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::SD; ++u) {
    const int pu = u * C::NT + threadIdx.x;      // LDS dword: row pu/2, half pu%2
    x.s_off[u] = tiled ? (uint32_t)(tgrp(pu >> 1) + (int64_t)(pu & 255) * 4)
                       : (uint32_t)(wrow(pu >> 1) * ks + ((pu & 1) << 2));
  }
}

template <int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI, int NS, int MINWG>
__global__ void __launch_bounds__(WN * 64, MINWG) gemm_kernel(GemmArgs p) {
  using C = Cfg<WN, TM, TN, DUAL>;
  constexpr int BM = C::BM;
  constexpr int BN = C::BN;
  static_assert(BN % kTileRows == 0 && C::NB * 4 % 512 == 0, "whole 128-row groups of the tiled weights per tile");
  __shared__ float red[WN];
  __shared__ f16x8 lds_a[NS][C::LDS_A];
  __shared__ u32x4 lds_b[NS][C::LDS_B];
  __shared__ uint2 lds_s[NS][C::NB];
  const int lane = threadIdx.x & 63;
  const int wn = threadIdx.x >> 6;
  const int r32 = lane & 31, hh = lane >> 5;
  // the next tile's first copies go out before this tile's epilogue (two
  // buffers, and an epilogue that does not use them)
  constexpr bool kAhead = NS == 2 && EPI != EPI_GLUQ;
  const uint32_t vtotal = p.m_tiles * p.n_tiles * p.splits;
  const int64_t nchunks_total = p.K >> 7;
  auto chunks_of = [&](uint32_t split) -> int64_t {   // chunks of a K split
    const int64_t n = nchunks_total - (int64_t)split * p.chunks_per_split;
    return n < (int64_t)p.chunks_per_split ? n : (int64_t)p.chunks_per_split;
  };

  Ctx<WN, TM, TN, DUAL> x;
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
  const uint32_t wb = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 64u;
  auto la = [&](int st) { return lds_addr(lds_a[st]) + wb * 16u; };
  auto lb = [&](int st) { return lds_addr(lds_b[st]) + wb * 16u; };
  auto ls = [&](int st) { return lds_addr(lds_s[st]) + wb * 4u; };
  constexpr int PER0 = C::SA + C::SB + C::SD;      // copies per wave per chunk

  TileLoc cur = locate_tile<BM, BN, GROUPED>(p, blockIdx.x, vtotal);
  bool staged = false;                             // cur's first copies already issued
  for (uint32_t v = blockIdx.x; v < vtotal; v += gridDim.x) {
    const uint32_t vn = v + gridDim.x;
    if (cur.m0 < 0) {                              // (uniform) a tile past the last expert
      if constexpr (EPI == EPI_GLU) {
        if (threadIdx.x == 0) p.partials[v] = 0.f;
      }
      if (vn < vtotal) cur = locate_tile<BM, BN, GROUPED>(p, vn, vtotal);
      continue;
    }
    const int64_t m0 = cur.m0, m_end = cur.m_end, n0 = cur.n0;
    const uint32_t split = cur.split;
    const int e = cur.e;
    const int64_t nch = chunks_of(split);
    tile_desc<WN, TM, TN, DUAL, GROUPED>(x, p, cur, (int64_t)split * p.chunks_per_split);
    if (!staged) {
      // every wave is past its last reads of the stage buffers (earlier tile)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
      __builtin_amdgcn_sched_barrier(0);
      tile_offsets<WN, TM, TN, DUAL, GROUPED>(x, p, cur);
    }

    // ---- main loop ----------------------------------------------------------------
    if constexpr (NS == 2) {
      // Two buffers, pipelined across chunk boundaries (xstep above).
      const Lds l0{lds_a[0], lds_b[0], lds_s[0]}, l1{lds_a[1], lds_b[1], lds_s[1]};
      BPack<TN, DUAL> f0, f1;
      BExp<TN, DUAL> e0, e1;
      // both buffers' copies in flight before the first wait (chunk 0 landed:
      // at most chunk 1's copies still outstanding); copies issued ahead of the
      // previous tile's epilogue wait for everything that epilogue stored too
      if (!staged) {
        stage_dma(x, la(0), lb(0), ls(0), 0);
        if (nch > 1) {
          stage_dma(x, la(1), lb(1), ls(1), 1);
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(PER0) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
        }
      } else {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
      }
      __builtin_amdgcn_sched_barrier(0);
      read_b<WN, TM, TN, DUAL>(l0, f0);
      read_a<0, 0>(x, l0);
      read_a<1, 1>(x, l0);
      expand_b<TN, DUAL, 0>(f0, e0);
      // Chunk pairs in one loop body (no exit between them, so the
      // accumulators keep their registers across the back edge), then the odd
      // last chunk.
      int64_t c = 0;
      for (; c + 1 < nch; c += 2) {
        xchunk(x, l0, l1, f0, f1, e0, e1, c + 2 < nch, c + 2, la(0), lb(0), ls(0));
        xchunk(x, l1, l0, f1, f0, e0, e1, c + 3 < nch, c + 3, la(1), lb(1), ls(1));
      }
      if (c < nch) xchunk(x, l0, l1, f0, f1, e0, e1, false, c + 2, la(0), lb(0), ls(0));
    } else {
      // NS-buffer ring: the copies of chunks c+1 .. c+NS-2 stay in flight while
      // chunk c is consumed; the buffer of chunk c-1 is refilled with chunk
      // c+NS-1 right after the barrier that ends its last reads.
      static_assert(NS >= 3 && NS <= 4, "ring of 3 or 4 buffers");
      constexpr int PER = PER0;
      static_assert((NS - 2) * PER <= 63, "vmcnt range");
#pragma unroll
      for (int st = 0; st < NS - 1; ++st)
        if (st < nch) stage_dma(x, la(st), lb(st), ls(st), st);
      int sc = 0;                                      // buffer of chunk c
      for (int64_t c = 0; c < nch; ++c) {
        const int64_t later = (nch - 1 - c) < (NS - 2) ? (nch - 1 - c) : (NS - 2);
        ring_wait<PER, NS - 2>(later);
        const int sf = sc == 0 ? NS - 1 : sc - 1;      // buffer of chunk c-1
        if (c + NS - 1 < nch) stage_dma(x, la(sf), lb(sf), ls(sf), c + NS - 1);
        run_chunk(x, Lds{lds_a[sc], lds_b[sc], lds_s[sc]});
        sc = sc == NS - 1 ? 0 : sc + 1;
      }
    }

    // ---- the next tile's first copies -------------------------------------------------
    staged = false;
    if (vn < vtotal) {
      cur = locate_tile<BM, BN, GROUPED>(p, vn, vtotal);
      if constexpr (kAhead) {
        if (cur.m0 >= 0) {
          // every wave is past its reads of both buffers (the last chunk's
          // reads of the other buffer fetch data that is never used)
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
          __builtin_amdgcn_sched_barrier(0);
          tile_desc<WN, TM, TN, DUAL, GROUPED>(x, p, cur, (int64_t)cur.split * p.chunks_per_split);
          tile_offsets<WN, TM, TN, DUAL, GROUPED>(x, p, cur);
          stage_dma(x, la(0), lb(0), ls(0), 0);
          if (chunks_of(cur.split) > 1) stage_dma(x, la(1), lb(1), ls(1), 1);
          staged = true;
        }
      }
    }

    // ---- epilogue ---------------------------------------------------------------------
    if constexpr (EPI == EPI_GLUQ) {
      // SiLU(gate) * up of the whole tile goes to LDS (the stage buffers are
      // free once every wave is past the main loop), then each thread quantises
      // whole 16-column blocks of it with the given global scale.  Columns are
      // XOR-swizzled in units of four floats by the row, so the two row halves
      // of an MFMA fragment store to different banks.
      static_assert(DUAL, "quantising GLU epilogue: gate/up pair");
      static_assert(BM * C::BN * 4 <= (int)sizeof(lds_b), "GLU tile must fit the stage buffers");
      float* tile = reinterpret_cast<float*>(&lds_b[0][0]);
      const float alpha = p.a_gs[0] * p.b_gs[GROUPED ? e : 0];
      const float alpha_u = p.a_gs[0] * p.u_gs[GROUPED ? e : 0];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = (wn * TN + j) * 32 + r32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            tile[row * C::BN + (col ^ ((row & 7) << 2))] = silu_mul(x.acc[i][j][r] * alpha, x.accu[i][j][r] * alpha_u);
          }
        }
      __syncthreads();
      const float gs = p.q_gs[0];
      constexpr int NBC = C::BN / 16;
      for (int q = threadIdx.x; q < BM * NBC; q += C::NT) {
        const int row = q / NBC, cb = q - row * NBC;
        const int64_t grow = m0 + row, gcol = n0 + cb * 16;
        if (grow >= m_end || gcol >= p.N) continue;
        float vv[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 t4 = *reinterpret_cast<const float4*>(tile + row * C::BN + ((cb * 16 + 4 * g4) ^ ((row & 7) << 2)));
          vv[4 * g4] = t4.x; vv[4 * g4 + 1] = t4.y; vv[4 * g4 + 2] = t4.z; vv[4 * g4 + 3] = t4.w;
        }
        uint32_t w0, w1;
        const uint32_t sc = quantize_block16(vv, gs, w0, w1);
        *reinterpret_cast<uint2*>(p.q_codes + grow * (p.N / 2) + gcol / 2) = make_uint2(w0, w1);
        p.q_scales[grow * (p.N / 16) + gcol / 16] = (uint8_t)sc;
        if (p.q16 != nullptr) {
          f16x8* o = reinterpret_cast<f16x8*>(p.q16 + grow * p.N + gcol);
          o[0] = expand8(w0, sc);
          o[1] = expand8(w1, sc);
        }
      }
    } else {
      // Register epilogue.  Output (row, col) of this lane: row = urow + 4 hh,
      // col = ucol + r32 with urow, ucol the same for the whole wave, so each
      // store is a wave-uniform address (scalar arithmetic) plus this lane's
      // fixed offset; tiles inside the matrix skip the bounds checks.
      const float alpha = p.a_gs[0] * p.b_gs[GROUPED ? e : 0];
      float alpha_u = 0.f;
      if constexpr (DUAL) alpha_u = p.a_gs[0] * p.u_gs[GROUPED ? e : 0];
      float hmax = 0.f;
      const int wnu = __builtin_amdgcn_readfirstlane(wn);
      const bool full = m0 + BM <= m_end && n0 + BN <= p.N;   // uniform
      // KIND 0: SiLU(gate) * up, float32 H; 1: split-K partial sums; 2: float32
      // output * alpha; 3: bf16 output * alpha
      auto emit = [&](auto kind, auto check) {
        constexpr int KIND = decltype(kind)::value;
        constexpr bool CHECK = decltype(check)::value;
        constexpr int ESZ = KIND == 3 ? 2 : 4;
        char* out;
        int64_t ld;
        if constexpr (KIND == 0) {
          out = reinterpret_cast<char*>(p.h);
          ld = p.N;
        } else if constexpr (KIND == 1) {
          out = reinterpret_cast<char*>(p.split_out + (int64_t)split * p.M * p.N);
          ld = p.N;
        } else {
          out = reinterpret_cast<char*>(p.c);
          ld = p.ldc;
        }
        const uint32_t lane_off = (uint32_t)(((int64_t)(4 * hh) * ld + r32) * ESZ);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int64_t ucol = n0 + (int64_t)(wnu * TN + j) * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t urow = m0 + i * 32 + 8 * (r >> 2) + (r & 3);
              float val;
              if constexpr (KIND == 0) {
                val = silu_mul(x.acc[i][j][r] * alpha, x.accu[DUAL ? i : 0][DUAL ? j : 0][r] * alpha_u);
                if (!CHECK || (urow + 4 * hh < m_end && ucol + r32 < p.N)) hmax = fmaxf(hmax, fabsf(val));
              } else if constexpr (KIND == 1) {
                val = x.acc[i][j][r];
              } else {
                val = x.acc[i][j][r] * alpha;
              }
              if (!CHECK || (urow + 4 * hh < m_end && ucol + r32 < p.N)) {
                char* a = out + (urow * ld + ucol) * ESZ + lane_off;
                if constexpr (KIND == 3)
                  *reinterpret_cast<uint16_t*>(a) = (uint16_t)f32_to_bf16_bits(val);
                else
                  *reinterpret_cast<float*>(a) = val;
              }
            }
          }
      };
      auto emit_kind = [&](auto kind) {
        if (full) emit(kind, std::false_type{});
        else emit(kind, std::true_type{});
      };
      if constexpr (EPI == EPI_GLU) emit_kind(std::integral_constant<int, 0>{});
      else if (p.splits > 1 || p.force_split) emit_kind(std::integral_constant<int, 1>{});
      else if (p.c_bf16) emit_kind(std::integral_constant<int, 3>{});
      else emit_kind(std::integral_constant<int, 2>{});
      if constexpr (EPI == EPI_GLU) {
        hmax = block_max(hmax, red);
        if (threadIdx.x == 0) p.partials[v] = hmax;
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x.acc[i][j][r] = 0.f;
          if constexpr (DUAL) x.accu[i][j][r] = 0.f;
        }
  }
}

// ---- small batches (M <= 32): the contraction is a weight stream -------------------
// A work-group is kSkWaves waves on the same 32 weight rows (x2 with the
// gate/up pair); each wave takes its own slice of the work-group's K range and
// the slices' sums are added through LDS in wave order (deterministic).
// Packed weights and the f16 activation fragments go from global memory
// straight into registers kSkDepth chunks ahead of their MFMAs -- no LDS
// staging and no barrier in the main loop -- so each wave keeps several KiB of
// loads in flight, which is what a weight stream needs to approach the HBM
// bandwidth.  The MFMA tile is 32 rows, so any M <= 32 costs the same.
constexpr int kSkWaves = 4;
constexpr int kSkDepth = 2;

template <bool DUAL>
struct SkSlot {
  Frag b, u;
  f16x8 a[8];
};

// Raw buffer resource over `bytes` bytes at p (gfx9 family: dword3 0x00020000).
// Reads past the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

__device__ __forceinline__ f16x8 frag_expand_rt(const Frag& f, int s) {
  const uint32_t w = (s < 4) ? f.c0[s & 3] : f.c1[s & 3];
  return expand8(w, (f.s >> (8 * (s >> 1))) & 0xFFu);
}

template <bool DUAL, int EPI>
__global__ void __launch_bounds__(kSkWaves * 64) skinny_kernel(GemmArgs p) {
  constexpr int NM = DUAL ? 2 : 1;
  __shared__ float red[kSkWaves * NM * 16 * 64];
  __shared__ float redmax[kSkWaves];
  __shared__ float tq[EPI == EPI_GLUQ ? 32 * 33 : 1];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps the loop scalar
  const int r32 = lane & 31, hh = lane >> 5;
  const uint32_t n_tile = blockIdx.x % p.n_tiles;
  const uint32_t split = blockIdx.x / p.n_tiles;
  const int64_t n0 = (int64_t)n_tile * 32;
  const int64_t K = p.K, kb = K >> 1, ks = K >> 4;
  const int64_t total = K >> 7;
  const int64_t cs0 = (int64_t)split * p.chunks_per_split;
  int64_t cs1 = cs0 + p.chunks_per_split;
  if (cs1 > total) cs1 = total;
  const int64_t len = cs1 > cs0 ? cs1 - cs0 : 0;
  const int64_t c0 = cs0 + (len * w) / kSkWaves;
  const int64_t n = cs0 + (len * (w + 1)) / kSkWaves - c0;   // chunks of this wave (wave-uniform, may be 0)

  // Buffer loads (one wave-uniform resource per operand, based at this tile's
  // first row): 32-bit lane offsets, the chunk offset in the scalar operand.
  // They are intrinsic calls, which the compiler keeps where they are written,
  // so the register ring below stays a software pipeline.
  const int64_t nrow = (p.N - n0) < 32 ? (p.N - n0) : 32;
  const int32_t wr = r32 < nrow ? r32 : (int32_t)nrow - 1;
  const int32_t arow = r32 < p.M ? r32 : (int32_t)p.M - 1;   // rows past M: finite, never stored
  const int64_t cbase = n0 * kb + c0 * 64, sbase = n0 * ks + c0 * 8;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b_codes + cbase, nrow * kb - c0 * 64);
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(p.b_scales + sbase, nrow * ks - c0 * 8);
  __amdgpu_buffer_rsrc_t ru = rb, rus = rbs;
  if constexpr (DUAL) {
    ru = make_rsrc(p.u_codes + cbase, nrow * kb - c0 * 64);
    rus = make_rsrc(p.u_scales + sbase, nrow * ks - c0 * 8);
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + c0 * 128, (int64_t)p.M * K * 2 - c0 * 256);
  const int32_t vo_c = wr * (int32_t)kb + hh * 32;
  const int32_t vo_s = wr * (int32_t)ks + hh * 4;
  const int32_t vo_a = arow * (int32_t)K * 2 + hh * 128;

  auto load = [&](int64_t c, SkSlot<DUAL>& sl) {
    const int32_t cc = (int32_t)c * 64, csc = (int32_t)c * 8, ca = (int32_t)c * 256;
    sl.b.c0 = __builtin_amdgcn_raw_buffer_load_b128(rb, vo_c, cc, 0);
    sl.b.c1 = __builtin_amdgcn_raw_buffer_load_b128(rb, vo_c + 16, cc, 0);
    sl.b.s = __builtin_amdgcn_raw_buffer_load_b32(rbs, vo_s, csc, 0);
    if constexpr (DUAL) {
      sl.u.c0 = __builtin_amdgcn_raw_buffer_load_b128(ru, vo_c, cc, 0);
      sl.u.c1 = __builtin_amdgcn_raw_buffer_load_b128(ru, vo_c + 16, cc, 0);
      sl.u.s = __builtin_amdgcn_raw_buffer_load_b32(rus, vo_s, csc, 0);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, vo_a + 16 * s, ca, 0);
      sl.a[s] = __builtin_bit_cast(f16x8, v);
    }
  };

  f32x16 acc, accu;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = 0.f;
    accu[r] = 0.f;
  }
  auto compute = [&](const SkSlot<DUAL>& sl) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sl.a[s], frag_expand_rt(sl.b, s), acc, 0, 0, 0);
      if constexpr (DUAL)
        accu = __builtin_amdgcn_mfma_f32_32x32x16_f16(sl.a[s], frag_expand_rt(sl.u, s), accu, 0, 0, 0);
    }
  };

  // Every load is unconditional (chunk indices clamped to the wave's last
  // chunk: the tail re-reads it from L2) so that the loads stay in issue order
  // and each MFMA waits only for the loads of its own chunk.
  if (n > 0) {
    const int64_t last = n - 1;
    SkSlot<DUAL> ring[kSkDepth];
#pragma unroll
    for (int d = 0; d < kSkDepth; ++d) {
      load(d < last ? d : last, ring[d]);
      __builtin_amdgcn_sched_barrier(0);   // slots issue in order: slot 0 is the oldest
    }
    for (int64_t c = 0; c < n; c += kSkDepth) {
#pragma unroll
      for (int d = 0; d < kSkDepth; ++d) {
        if (c + d < n) compute(ring[d]);
        __builtin_amdgcn_sched_barrier(0);   // keep the refill after the MFMAs that read the slot
        const int64_t nx = c + d + kSkDepth;
        load(nx < last ? nx : last, ring[d]);
        __builtin_amdgcn_sched_barrier(0);   // and before the next slot's MFMAs
      }
    }
  }

  // ---- add the waves' partial tiles (wave order), then the epilogue ----------------
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    red[((w * NM) * 16 + r) * 64 + lane] = acc[r];
    if constexpr (DUAL) red[((w * NM + 1) * 16 + r) * 64 + lane] = accu[r];
  }
  __syncthreads();
  const float alpha = p.a_gs[0] * p.b_gs[0];
  float alpha_u = 0.f;
  if constexpr (DUAL) alpha_u = p.a_gs[0] * p.u_gs[0];
  float hmax = 0.f;
#pragma unroll
  for (int i = 0; i < 1024 / (kSkWaves * 64); ++i) {
    const int e = (int)threadIdx.x + i * kSkWaves * 64;
    const int r = e >> 6, l = e & 63;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kSkWaves; ++w2) {
      g += red[((w2 * NM) * 16 + r) * 64 + l];
      if constexpr (DUAL) u += red[((w2 * NM + 1) * 16 + r) * 64 + l];
    }
    const int64_t row = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    const int64_t col = n0 + (l & 31);
    if constexpr (EPI == EPI_GLUQ) {
      tq[row * 33 + (l & 31)] = silu_mul(g * alpha, u * alpha_u);
      continue;
    }
    if (row < p.M && col < p.N) {
      if constexpr (EPI == EPI_GLU) {
        const float hv = silu_mul(g * alpha, u * alpha_u);
        p.h[row * p.N + col] = hv;
        hmax = fmaxf(hmax, fabsf(hv));
      } else if (p.splits > 1 || p.force_split) {
        p.split_out[((int64_t)split * p.M + row) * p.N + col] = g;
      } else {
        const float v = g * alpha;
        if (p.c_bf16)
          reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] = (uint16_t)f32_to_bf16_bits(v);
        else
          reinterpret_cast<float*>(p.c)[row * p.ldc + col] = v;
      }
    }
  }
  if constexpr (EPI == EPI_GLU) {
    hmax = block_max(hmax, redmax);
    if (threadIdx.x == 0) p.partials[blockIdx.x] = hmax;
  }
  if constexpr (EPI == EPI_GLUQ) {
    // the 32 x 32 tile (rows past M are computed, never stored): threads
    // 0..63 quantise its two 16-column blocks per row
    __syncthreads();
    const int row = (int)threadIdx.x >> 1, half = (int)threadIdx.x & 1;
    const int64_t gcol = n0 + 16 * half;
    if (threadIdx.x < 64 && row < p.M && gcol < p.N) {
      float v[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = tq[row * 33 + 16 * half + c];
      uint32_t w0, w1;
      const uint32_t sc = quantize_block16(v, p.q_gs[0], w0, w1);
      *reinterpret_cast<uint2*>(p.q_codes + row * (p.N / 2) + gcol / 2) = make_uint2(w0, w1);
      p.q_scales[row * (p.N / 16) + gcol / 16] = (uint8_t)sc;
    }
  }
}

// ---- weight stream for one or two tokens ---------------------------------------------
// At T <= 2 the contraction is a matrix-vector product bound by reading the
// weights once.  Reading them at full HBM speed needs long contiguous runs
// per wave instruction: the MFMA fragment layout (32 weight rows x 32 bytes
// per instruction) streams at about half the rate of a layout where a wave
// reads one row at a time.  So here the lanes run along K: K is cut into
// units of 1024 elements (64 blocks of 16), a split takes BPL consecutive
// units, and lane l takes block l of each of them (BPL blocks 64 apart, 8
// code bytes and one scale byte each), so one load instruction of the wave
// reads 512 contiguous code bytes.  The activation (f16, expanded once per
// call) follows the same layout and stays in registers for the whole wave.
//
// Each block's 16 products code * x are summed by v_dot2_f32_f16 on the
// plain code values (the converter's scale is 1, so they are exact in f16;
// each product is exact in float32), then multiplied once by the block's
// E4M3 scale.  The scale is decoded through f16: the bits (s << 7) are
// dec(s) * 2^-8 for every E4M3 code, and the final * 256 restores it
// exactly.  Lane partial sums are added across the wave in a fixed butterfly
// order.
//
// A wave owns a few consecutive output columns (weight rows) of one split
// and walks them in groups of RP columns (with the gate/up pair, RP gate rows
// and the same RP up rows), the loads of the next DEPTH-1 groups in flight
// while a group is computed.  The results per token stay in registers until
// the epilogue: the GLU output and its max (one partial per wave), the GLU
// output quantised in 16-column blocks with a given scale (the work-group's
// four waves hold consecutive columns and gather them in LDS), or the
// store / split-K partial store.
#ifndef NVFP4_GV_DEPTH
#define NVFP4_GV_DEPTH 2
#endif
#ifndef NVFP4_GV_MAXT
#define NVFP4_GV_MAXT 2
#endif
// Output columns per wave (4, 8 or 16): fewer columns give more waves and
// more weight bytes in flight per CU.
#ifndef NVFP4_GV_COLS
#define NVFP4_GV_COLS 4
#endif
constexpr int kGvCols = NVFP4_GV_COLS;
static_assert(kGvCols == 4 || kGvCols == 8 || kGvCols == 16, "a work-group must cover whole 16-column blocks");

__device__ __forceinline__ float e4m3_over_256(uint32_t s) {
  return (float)bitcast<_Float16>((uint16_t)(s << 7));
}

// Sum over the 64 lanes of a wave in a fixed order with DPP row shifts and
// row broadcasts (16-lane prefix sums, then rows 0+1 and 2+3, then all);
// lane 63 ends with the total, which is returned to every lane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// WGK (store epilogue, at most kGvWgkSplits K splits): the work-group is one
// column group's K splits, wave w taking split w, and the splits' partial
// sums are added through LDS, in split order, by the work-group's first wave
// (the arithmetic of the reduction kernels): one barrier instead of partial
// sums stored to and read back from memory across work-groups.
constexpr int kGvWgkSplits = 12;

template <int T, int BPL, bool DUAL, int EPI, bool WGK = false>
__global__ void __launch_bounds__(WGK ? 64 * kGvWgkSplits : 256) gemv_kernel(GemmArgs p) {
  static_assert(!WGK || (!DUAL && EPI == EPI_STORE), "split-K in one work-group: store epilogue");
  constexpr int PER = BPL * (DUAL ? 2 : 1);
  constexpr int RP0 = (8 / PER) > 0 ? (8 / PER) : 1;
  constexpr int RP = RP0 < kGvCols ? RP0 : kGvCols;       // columns per group
  constexpr int NR = DUAL ? 2 * RP : RP;                  // weight rows per group
  constexpr int G = kGvCols / RP;                         // groups per wave
  constexpr int D = NVFP4_GV_DEPTH < G ? NVFP4_GV_DEPTH : G;
  static_assert(kGvCols % RP == 0, "groups must tile the wave's columns");
  __shared__ float hq[EPI == EPI_GLUQ && kGvCols < 16 ? T * 4 * kGvCols : 1];
  __shared__ float wgk[WGK ? kGvWgkSplits * T * kGvCols : 1];
  const int lane = threadIdx.x & 63;
  const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t N = p.N, K = p.K, M = p.M;
  const int64_t wps = (N + kGvCols - 1) / kGvCols;       // waves per split
  // WGK: one work-group per column group, one wave per split (no wave past the end)
  const int64_t wave = WGK ? (int64_t)wi * wps + blockIdx.x : (int64_t)blockIdx.x * 4 + wi;
  // Only the store epilogue can have waves past the end (the gate/up pair
  // has N % 128 == 0 and one split, so its work-groups are full); the
  // quantising epilogue's barrier below is never skipped by any wave.
  if (!WGK && wave >= wps * (int64_t)p.splits) return;
  const int64_t split = wave / wps;
  const int64_t n0 = (wave - split * wps) * kGvCols;
  // block b of this lane is block 64 b + lane of the split
  const int64_t e0 = split * BPL * 1024 + (int64_t)lane * 16;          // K element of this lane's block 0
  constexpr int64_t EB = 1024;                                          // K elements between its blocks
  const int64_t kb = K >> 1, ks = K >> 4;

  struct Slot {
    uint2 c[NR][BPL];
    uint32_t s[NR][BPL];
  };
  // Weight loads are buffer-load intrinsics over one row (a wave-uniform
  // resource): the compiler keeps them where they are written and does not
  // merge the scale bytes into wider loads whose unpacking would wait for
  // them at once, so the loads of later groups stay in flight.
  const int32_t vo_c = (int32_t)(e0 / 2), vo_s = (int32_t)(e0 / 16);
  auto load = [&](int g, Slot& sl) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int q = r % RP;
      int64_t row = n0 + g * RP + q;
      row = row < N ? row : N - 1;                          // columns past N: valid rows, never stored
      const bool up = DUAL && r >= RP;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc((up ? p.u_codes : p.b_codes) + row * kb, kb);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc((up ? p.u_scales : p.b_scales) + row * ks, ks);
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        // the resources span one row: a block past K (last unit partial) reads
        // past them and gets zero, with no memory traffic
        sl.c[r][b] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, vo_c + (int32_t)(EB / 2) * b, 0, 0));
        sl.s[r][b] = __builtin_amdgcn_raw_buffer_load_b8(rs, vo_s + (int32_t)(EB / 16) * b, 0, 0);
      }
    }
  };

  float res[T][kGvCols];
  float resu[DUAL ? T : 1][DUAL ? kGvCols : 1];
  Slot ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(d, ring[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the weight loads of the first groups are in flight before the activation is read
  // activation blocks of this lane, expanded here from the NVFP4 activation
  // into the f16 pairs the dot products take (code * scale, exact; the
  // converter is given 2^8 and the pair of E4M3 scale bits (s << 7), which is
  // dec(s) * 2^-8, so the product is code * dec(s)); tokens past M are zero
  f16x2 xp[T][BPL][8];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      if (t < M && e0 + EB * b < K) {                    // blocks past K (last unit partial): zero
        const uint2 cw = *reinterpret_cast<const uint2*>(p.a_codes + t * (K >> 1) + (e0 + EB * b) / 2);
        const uint32_t sh = (uint32_t)p.a_scales[t * (K >> 4) + (e0 + EB * b) / 16] << 7;
        const f16x2 sc = bitcast<f16x2>(sh | (sh << 16));
        xp[t][b][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.x, 256.0f, 0) * sc;
        xp[t][b][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.x, 256.0f, 1) * sc;
        xp[t][b][2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.x, 256.0f, 2) * sc;
        xp[t][b][3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.x, 256.0f, 3) * sc;
        xp[t][b][4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.y, 256.0f, 0) * sc;
        xp[t][b][5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.y, 256.0f, 1) * sc;
        xp[t][b][6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.y, 256.0f, 2) * sc;
        xp[t][b][7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw.y, 256.0f, 3) * sc;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xp[t][b][i] = (f16x2){(_Float16)0.f, (_Float16)0.f};
      }
    }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    Slot& sl = ring[g % D];
    float acc[NR][T];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const uint32_t w0 = sl.c[r][b].x, w1 = sl.c[r][b].y;
        const f16x2 cp[8] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2),
                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3)};
        const float sc = e4m3_over_256(sl.s[r][b]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) d = __builtin_amdgcn_fdot2(cp[i], xp[t][b][i], d, false);
          acc[r][t] = fmaf(d, sc, acc[r][t]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (g + D < G) load(g + D, sl);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < RP; ++q)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        res[t][g * RP + q] = wave_sum_dpp(acc[q][t]) * 256.f;
        if constexpr (DUAL) resu[t][g * RP + q] = wave_sum_dpp(acc[RP + q][t]) * 256.f;
      }
  }

  // ---- epilogue: lane t < M writes token t's 16 columns ----------------------------
  float v[kGvCols], vu[DUAL ? kGvCols : 1];
#pragma unroll
  for (int c = 0; c < kGvCols; ++c) {
    v[c] = res[0][c];
    if constexpr (DUAL) vu[c] = resu[0][c];
  }
#pragma unroll
  for (int t = 1; t < T; ++t)
    if (lane == t) {
#pragma unroll
      for (int c = 0; c < kGvCols; ++c) {
        v[c] = res[t][c];
        if constexpr (DUAL) vu[c] = resu[t][c];
      }
    }
  const bool active = lane < M && lane < T;
  if constexpr (DUAL) {
    const float alpha = p.a_gs[0] * p.b_gs[0], alpha_u = p.a_gs[0] * p.u_gs[0];
    float hmax = 0.f;
#pragma unroll
    for (int c = 0; c < kGvCols; ++c) {
      v[c] = silu_mul(v[c] * alpha, vu[c] * alpha_u);
      hmax = fmaxf(hmax, active ? fabsf(v[c]) : 0.f);
    }
    if constexpr (EPI == EPI_GLU) {
      if (active) {
        float4* dst = reinterpret_cast<float4*>(p.h + lane * N + n0);   // N % 128 == 0: 16-B aligned
#pragma unroll
        for (int c = 0; c < kGvCols / 4; ++c) dst[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
      }
      hmax = wave_max(hmax);
      if (lane == 0) p.partials[wave] = hmax;
    } else if constexpr (kGvCols == 16) {
      if (active) {
        uint32_t w0, w1;
        const uint32_t sc = quantize_block16(v, p.q_gs[0], w0, w1);
        *reinterpret_cast<uint2*>(p.q_codes + lane * (N / 2) + n0 / 2) = make_uint2(w0, w1);
        p.q_scales[lane * (N / 16) + n0 / 16] = (uint8_t)sc;
      }
    } else {
      // the work-group's 4 waves hold 4 * kGvCols consecutive columns: gather
      // them per token, then one thread per (16-column block, token) quantises
      constexpr int WC = 4 * kGvCols;
      if (active) {
#pragma unroll
        for (int c = 0; c < kGvCols; ++c) hq[lane * WC + wi * kGvCols + c] = v[c];
      }
      __syncthreads();
      const int tid = (int)threadIdx.x;
      const int blk = tid % (WC / 16), t = tid / (WC / 16);
      if (t < T && t < M) {
        float b16[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) b16[c] = hq[t * WC + blk * 16 + c];
        const int64_t c0 = (int64_t)blockIdx.x * WC + blk * 16;
        uint32_t w0, w1;
        const uint32_t sc = quantize_block16(b16, p.q_gs[0], w0, w1);
        *reinterpret_cast<uint2*>(p.q_codes + t * (N / 2) + c0 / 2) = make_uint2(w0, w1);
        p.q_scales[t * (N / 16) + c0 / 16] = (uint8_t)sc;
      }
    }
  } else if constexpr (WGK) {
    // each split's sums to LDS, then the first wave adds them in split order
    // (lane = token * kGvCols + column) and stores the outputs
    if (active) {
#pragma unroll
      for (int c = 0; c < kGvCols; ++c) wgk[(wi * T + lane) * kGvCols + c] = v[c];
    }
    __syncthreads();
    if (wi == 0) {
      const int64_t t = lane / kGvCols, c = lane % kGvCols;
      float am = 0.f;
      if (t < M && t < T && n0 + c < N) {
        float acc = 0.f;
        for (uint32_t sp = 0; sp < p.splits; ++sp) acc += wgk[(sp * T + t) * kGvCols + c];
        am = store_output(p, t, n0 + c, acc);
      }
      if (p.amax_slots != nullptr) {
        am = wave_max(am);
        if (lane == 0)
          atomicMax(reinterpret_cast<unsigned int*>(p.amax_slots + (n0 / kGvCols) % kAmaxSlots), __float_as_uint(am));
      }
    }
  } else {
    const bool part = p.splits > 1 || p.force_split;
    if (active) {
      if (part) {
        float* dst = p.split_out + (split * M + lane) * N + n0;
#pragma unroll
        for (int c = 0; c < kGvCols; ++c) {
          if (n0 + c >= N) continue;
          if (p.tickets != nullptr) store_coherent(dst + c, v[c]);
          else dst[c] = v[c];
        }
      } else {
        const float alpha = p.a_gs[0] * p.b_gs[0];
#pragma unroll
        for (int c = 0; c < kGvCols; ++c) {
          if (n0 + c >= N) continue;
          const float o = v[c] * alpha;
          if (p.c_bf16)
            reinterpret_cast<uint16_t*>(p.c)[lane * p.ldc + n0 + c] = (uint16_t)f32_to_bf16_bits(o);
          else
            reinterpret_cast<float*>(p.c)[lane * p.ldc + n0 + c] = o;
        }
      }
    }
    if (part && p.tickets != nullptr) {
      // split-K finish: the wave of this column group that arrives last adds
      // every split's partial sums (lane = token * kGvCols + column)
      stores_done();
      const int64_t grp = n0 / kGvCols;
      uint32_t last = 0;
      if (lane == 0) last = last_arrival(p.tickets + grp, p.splits) ? 1u : 0u;
      last = (uint32_t)__builtin_amdgcn_readfirstlane((int)last);
      if (last) {
        const int64_t t = lane / kGvCols, c = n0 + lane % kGvCols;
        float am = 0.f;
        if (t < M && t < T && c < N) am = finish_output(p, t, c);
        if (p.amax_slots != nullptr) {
          am = wave_max(am);
          if (lane == 0)
            atomicMax(reinterpret_cast<unsigned int*>(p.amax_slots + grp % kAmaxSlots), __float_as_uint(am));
        }
      }
    }
  }
}

// ---- weight stream for 3 to 16 tokens on the 16x16x32 matrix core -----------------------
// v_mfma_f32_16x16x32_f16 takes, in lane l, row l % 16 of the 16-row operand
// A and K positions 8 * (l / 16) .. +7; the same lanes hold column l % 16 of
// B at those K positions; lane l receives D[4 * (l / 16) + r][l % 16] in entry
// r.  Here A holds the tokens (MT = 8 rows staged for 3-8 tokens, 16 for
// 9-16; rows past M repeat the last token: computed, never stored) and B
// sixteen weight rows, so one instruction takes 16 rows x 32 K positions of
// the weights for every token at once, at the full matrix-core rate (the
// 4x4x4 instruction runs at a fraction of it).
//
// A wave is one work item: a column tile (16 output columns of the gate/up
// pair, i.e. 16 gate rows and the same 16 up rows; or 32 output columns of
// one weight) and one split of K.  Its K range is cut into stages of 256
// elements; each stage of the tile's 32 weight rows (128 code bytes and 16
// scale bytes per row) and of the tokens is copied from global memory straight
// into the wave's own LDS ring by the LDS DMA path, kTlDepth stages ahead.
// Every copy instruction moves whole 128-byte lines of a few rows (the
// row-contiguous pattern a weight stream needs to run near the HBM rate), and
// copies in flight hold no registers, so a CU keeps ~100 KiB of weights in
// flight.  The wave reads a landed stage back in fragment layout and expands
// it in registers (code * scale, exact in f16, as in the large-batch kernels).
//
// Within a stage, lane quarter g = l / 16 takes K elements 64g .. 64g+63 of
// each row and step s (0..7) feeds elements 64g + 8s .. +7 of them to the
// matrix core: one permutation of K applied to both operands leaves every
// dot product as it is.  An LDS row is eight 16-byte units, unit u of row r
// stored at position u ^ (r & 7), so the 8 lanes that read the same unit of 8
// consecutive rows hit 8 different bank groups.
//
// The splits of a column tile store their partial sums (device-coherent
// stores, as in the other weight streams); the wave that arrives last on the
// tile's ticket (cleared by an earlier launch) adds them in split order and
// runs the epilogue.  An unsplit tile runs it directly.  Without tickets (the
// store epilogue of a separate call) the partial sums go to the reduction
// launch.
// Ring depth, waves per work-group and the target number of stages per split
// of K: measured at 3-8 tokens on the 5120 / 17408 MLP, a shallow ring with
// one-wave work-groups (about 13 waves per CU, bounded by LDS) beats deeper
// rings with fewer waves, and 8-stage splits beat shorter ones.
#ifndef NVFP4_TL_DEPTH
#define NVFP4_TL_DEPTH 2
#endif
#ifndef NVFP4_TL_WAVES
#define NVFP4_TL_WAVES 1
#endif
#ifndef NVFP4_TL_SPS
#define NVFP4_TL_SPS 8
#endif
constexpr int kTlDepth = NVFP4_TL_DEPTH;
constexpr int kTlWaves = NVFP4_TL_WAVES;
constexpr int kTlMaxT = 16;
constexpr int kTlStageK = 256;
// Bytes of one stage in LDS for MT (8 or 16) token rows: weight codes (32 rows
// x 8 units), weight scales (32 rows x 16), token codes (MT rows x 8 units),
// token scales (16 slots x 16); and the copies per stage (4 + 2 for the
// weights, MT/8 + 1 for the tokens).
template <int MT>
struct TlCfg {
  static_assert(MT == 8 || MT == 16, "8 or 16 token rows");
  static constexpr int Bc = 0, Bs = 4096, Ac = 4608, As = Ac + MT * 128, Stage = As + 256;
  static constexpr int Dma = 6 + MT / 8 + 1;
};

// Wait until at most `ahead` stages' copies (DMA copies each) of this wave are
// in flight.
template <int DMA>
__device__ __forceinline__ void tl_wait(int64_t ahead) {
  static_assert(DMA * (kTlDepth - 1) <= 63, "vmcnt range");
  switch (ahead) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * DMA) : "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(4 * DMA) : "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(5 * DMA) : "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(6 * DMA) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(7 * DMA) : "memory"); break;
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int MT, bool DUAL, int EPI>
__global__ void __launch_bounds__(kTlWaves * 64) tile_kernel(GemmArgs p) {
  static_assert(kTlDepth >= 1 && kTlDepth <= 8, "ring depth");
  using L = TlCfg<MT>;
  constexpr int kTlBc = L::Bc, kTlBs = L::Bs, kTlAc = L::Ac, kTlAs = L::As, kTlStage = L::Stage;
  __shared__ __align__(16) uint8_t lds[kTlWaves * kTlDepth * kTlStage];
  constexpr int CW = DUAL ? 16 : 32;                      // output columns per tile
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t N = p.N, K = p.K, M = p.M;
  const int64_t ntile = (N + CW - 1) / CW;
  const int64_t item = (int64_t)blockIdx.x * kTlWaves + w;
  if (item >= ntile * (int64_t)p.splits) return;         // no barrier below: a wave may leave
  const int64_t split = item / ntile, ct = item - split * ntile;
  const int64_t n0 = ct * CW;
  const int64_t st0 = split * (int64_t)p.chunks_per_split;   // first stage of this split
  const int64_t nst_all = K / kTlStageK;
  const int64_t nst = (nst_all - st0) < (int64_t)p.chunks_per_split ? (nst_all - st0) : (int64_t)p.chunks_per_split;
  const int64_t kb = K >> 1, ks = K >> 4;

  // Buffer resources based at the tile's first weight row (rows past N read
  // row N-1: valid memory, never stored) and at the first token.
  const int64_t nrow = (N - n0) < (DUAL ? 16 : 32) ? (N - n0) : (DUAL ? 16 : 32);
  // With the tile-contiguous copies the resources cover this tile's 128-row
  // group g (rows 128g .. 128g+127, all chunks): its 16 or 32 rows of one
  // 128-K chunk are 1 or 2 KiB of consecutive code units there (rows past N
  // are zero in the copy).
  const bool tiled = p.b_tiled != nullptr && (!DUAL || p.u_tiled != nullptr);   // uniform
  const int64_t tgroup = (n0 / kTileRows) * (K / kTileK) * kTileBlock, tbytes = (K / kTileK) * kTileBlock;
  const i32x4 rb = tiled ? buf_desc(p.b_tiled + tgroup, tbytes) : buf_desc(p.b_codes + n0 * kb, nrow * kb);
  const i32x4 rbs = tiled ? rb : buf_desc(p.b_scales + n0 * ks, nrow * ks);
  i32x4 ru = rb, rus = rbs;
  if constexpr (DUAL) {
    ru = tiled ? buf_desc(p.u_tiled + tgroup, tbytes) : buf_desc(p.u_codes + n0 * kb, nrow * kb);
    rus = tiled ? ru : buf_desc(p.u_scales + n0 * ks, nrow * ks);
  }
  const i32x4 ra = buf_desc(p.a_codes, M * kb);
  const i32x4 ras = buf_desc(p.a_scales, M * ks);

  // Lane offsets of the copies (fixed for the whole loop; the stage goes in the
  // scalar offset).  Code copy d writes LDS units 64d + l: row 8d + l/8 of the
  // tile (with the gate/up pair, copies 2 and 3 hold the up rows), swizzled
  // unit l % 8, i.e. source unit (l % 8) ^ (l / 8).  Scale copy e writes row
  // 16e + l/4 (the up rows for e = 1 with the pair), 4-byte piece l % 4.
  //
  // Tiled: code copy d takes 1 KiB (16 rows x 4 units, already in the staged
  // order) of chunk half d % 2 of the stage, rows 16 (d / 2) .. (the up rows
  // for d >= 2 with the pair) into stage bytes (d % 2) * 2048 + (d / 2) * 1024;
  // scale copy e takes 16 rows x 8 bytes of both chunk halves of one matrix
  // (lanes 0-31 the first, 32-63 the second) into e * 256, or with one weight
  // all 32 rows of chunk half e.
  const uint32_t su = (uint32_t)((lane & 7) ^ (lane >> 3));
  const int64_t lr0 = n0 % kTileRows;               // the tile's first row within its group
  uint32_t vb[4], vs[2], db[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    int64_t r = DUAL ? 8 * (d & 1) + (lane >> 3) : 8 * d + (lane >> 3);
    r = r < nrow ? r : nrow - 1;
    vb[d] = tiled ? (uint32_t)((d & 1) * kTileBlock + (lr0 + (DUAL ? 0 : 16 * (d >> 1))) * 64 + lane * 16)
                  : (uint32_t)(r * kb) + su * 16u;
    db[d] = tiled ? (uint32_t)((d & 1) * 2048 + (d >> 1) * 1024) : (uint32_t)(d * 1024);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    int64_t r = DUAL ? (lane >> 2) : 16 * e + (lane >> 2);
    r = r < nrow ? r : nrow - 1;
    vs[e] = tiled ? (DUAL ? (uint32_t)(8192 + (lane >> 5) * kTileBlock + lr0 * 8 + (lane & 31) * 4)
                          : (uint32_t)(8192 + e * kTileBlock + lr0 * 8 + lane * 4))
                  : (uint32_t)(r * ks) + (uint32_t)(lane & 3) * 4u;
  }
  const uint32_t sc_step = tiled ? (uint32_t)(2 * kTileBlock) : 128u, ss_step = tiled ? (uint32_t)(2 * kTileBlock) : 16u;
  // token copy d writes token rows 8d .. 8d+7 the same way (rows past M read
  // the last token); the scale copy fills 16 token slots
  uint32_t va[MT / 8];
#pragma unroll
  for (int d = 0; d < MT / 8; ++d) {
    const int64_t tc = (8 * d + (lane >> 3)) < M ? (8 * d + (lane >> 3)) : M - 1;
    va[d] = (uint32_t)(tc * kb) + su * 16u;
  }
  const int64_t tsc = (lane >> 2) < M ? (lane >> 2) : M - 1;
  const uint32_t vas = (uint32_t)(tsc * ks) + (uint32_t)(lane & 3) * 4u;

  const uint32_t ring = (uint32_t)w * (kTlDepth * kTlStage);   // this wave's ring (byte offset in lds)
  const uint32_t ring_addr = lds_addr(lds) + ring;
  auto issue = [&](int64_t stg, uint32_t buf) {
    const uint32_t sw = (uint32_t)stg * sc_step, sws = (uint32_t)stg * ss_step;   // weight codes / scales
    const uint32_t sc = (uint32_t)stg * 128u, ss = (uint32_t)stg * 16u;           // tokens
    const uint32_t b = ring_addr + buf * kTlStage;
#pragma unroll
    for (int d = 0; d < 4; ++d) dma_b128((DUAL && d >= 2) ? ru : rb, vb[d], sw, b + kTlBc + db[d]);
#pragma unroll
    for (int e = 0; e < 2; ++e) dma_b32((DUAL && e >= 1) ? rus : rbs, vs[e], sws, b + kTlBs + e * 256);
#pragma unroll
    for (int d = 0; d < MT / 8; ++d) dma_b128(ra, va[d], sc, b + kTlAc + d * 1024);
    dma_b32(ras, vas, ss, b + kTlAs);
  };

  // Fragment offsets of this lane within a stage: row t of each 16-row tile
  // (t = l % 16), quarter g = l / 16 (units 2g and 2g+1, scale piece g).
  // Tiled: quarter g is chunk half g / 2, units 2 (g % 2) and 2 (g % 2) + 1 of
  // its 64-byte row piece, stored at unit ^ ((row / 4) % 4); scale piece g % 2
  // of the row's 8 bytes of that half.
  const int t = lane & 15, g = lane >> 4;
  uint32_t ob[2][2], obs[2], oa[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ob[j][h] = tiled ? kTlBc + (uint32_t)((g >> 1) * 2048 + (16 * j + t) * 64 + ((2 * (g & 1) + h) ^ ((t >> 2) & 3)) * 16)
                       : kTlBc + (uint32_t)((16 * j + t) * 8 + ((2 * g + h) ^ (t & 7))) * 16u;
    obs[j] = tiled ? (DUAL ? kTlBs + (uint32_t)((2 * j + (g >> 1)) * 128 + t * 8 + 4 * (g & 1))
                           : kTlBs + (uint32_t)((g >> 1) * 256 + (16 * j + t) * 8 + 4 * (g & 1)))
                   : kTlBs + (uint32_t)(16 * j + t) * 16u + 4u * g;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) oa[h] = kTlAc + (uint32_t)((MT == 16 ? t : (t & 7)) * 8 + ((2 * g + h) ^ (t & 7))) * 16u;
  const uint32_t oas = kTlAs + (uint32_t)t * 16u + 4u * g;

#pragma unroll
  for (int d = 0; d < kTlDepth; ++d)
    if (d < nst) issue(st0 + d, (uint32_t)d);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = 0; i < nst; ++i) {
    const int64_t left = nst - 1 - i;
    tl_wait<L::Dma>(left < kTlDepth - 1 ? left : kTlDepth - 1);
    const uint32_t buf = (uint32_t)(i % kTlDepth);
    const uint8_t* sb = lds + ring + buf * kTlStage;
    u32x4 bc[2][2], ac[2];
    uint32_t bs[2], as;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) bc[j][h] = *reinterpret_cast<const u32x4*>(sb + ob[j][h]);
      bs[j] = *reinterpret_cast<const uint32_t*>(sb + obs[j]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) ac[h] = *reinterpret_cast<const u32x4*>(sb + oa[h]);
    as = *reinterpret_cast<const uint32_t*>(sb + oas);
    // the reads above have returned before the buffer is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (i + kTlDepth < nst) issue(st0 + i + kTlDepth, buf);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int h = s >> 2, wd = s & 3, sh = 8 * (s >> 1);
      const f16x8 a = expand8(ac[h][wd], (as >> sh) & 0xFFu);
      const f16x8 b0 = expand8(bc[0][h][wd], (bs[0] >> sh) & 0xFFu);
      const f16x8 b1 = expand8(bc[1][h][wd], (bs[1] >> sh) & 0xFFu);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b1, acc1, 0, 0, 0);
    }
  }

  // ---- epilogue: lane (t, g) holds tokens 4g + r (r = 0..3) of tile column t ----------
  if constexpr (DUAL) {
    const int64_t c = n0 + t;                    // N % 16 == 0: every column exists
    float gv[4], uv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      gv[r] = acc0[r];
      uv[r] = acc1[r];
    }
    if (p.splits > 1) {
      // partial sums [splits][M][2N]: gate at column c, up at N + c
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = 4 * g + r;
        if (tok < M) {
          float* dst = p.split_out + (split * M + tok) * 2 * N + c;
          store_coherent(dst, gv[r]);
          store_coherent(dst + N, uv[r]);
        }
      }
      stores_done();
      uint32_t last = 0;
      if (lane == 0) last = last_arrival(p.tickets + ct, p.splits) ? 1u : 0u;
      if (!__builtin_amdgcn_readfirstlane((int)last)) return;
      // eight splits' loads in flight at a time, added in split order
      const int64_t plane = M * 2 * N;
#pragma unroll
      for (int r = 0; r < 4; ++r) gv[r] = uv[r] = 0.f;
      for (uint32_t s0 = 0; s0 < p.splits; s0 += 8u) {
        float lg[4][8], lu[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t tok = (4 * g + r) < M ? 4 * g + r : M - 1;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t s2 = s0 + k < p.splits ? s0 + k : p.splits - 1;
            const float* src = p.split_out + (int64_t)s2 * plane + tok * 2 * N + c;
            lg[r][k] = load_coherent(src);
            lu[r][k] = load_coherent(src + N);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (s0 + k < p.splits) {
              gv[r] += lg[r][k];
              uv[r] += lu[r][k];
            }
      }
    }
    const float alpha = p.a_gs[0] * p.b_gs[0], alpha_u = p.a_gs[0] * p.u_gs[0];
    if constexpr (EPI == EPI_GLU) {
      float hmax = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = 4 * g + r;
        if (tok < M) {
          const float hv = silu_mul(gv[r] * alpha, uv[r] * alpha_u);
          p.h[tok * N + c] = hv;
          hmax = fmaxf(hmax, fabsf(hv));
        }
      }
      hmax = wave_max(hmax);
      if (lane == 0) p.partials[ct] = hmax;
    } else {
      // the tile's 16 columns are one block per token: gather each token's
      // row in the wave's (drained) ring, then lane tok < M quantises it
      float* hq = reinterpret_cast<float*>(lds + ring);
#pragma unroll
      for (int r = 0; r < 4; ++r) hq[(4 * g + r) * 16 + t] = silu_mul(gv[r] * alpha, uv[r] * alpha_u);
      __builtin_amdgcn_wave_barrier();
      if (lane < M) {
        float b16[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) b16[k] = hq[lane * 16 + k];
        uint32_t w0, w1;
        const uint32_t sc = quantize_block16(b16, p.q_gs[0], w0, w1);
        *reinterpret_cast<uint2*>(p.q_codes + lane * (N / 2) + n0 / 2) = make_uint2(w0, w1);
        p.q_scales[lane * (N / 16) + n0 / 16] = (uint8_t)sc;
      }
    }
  } else {
    const bool part = p.splits > 1 || p.force_split;
    const float alpha = p.a_gs[0] * p.b_gs[0];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = 4 * g + r, c = n0 + 16 * j + t;
        if (tok >= M || c >= N) continue;
        const float v = j ? acc1[r] : acc0[r];
        if (part) {
          float* dst = p.split_out + (split * M + tok) * N + c;
          if (p.tickets != nullptr) store_coherent(dst, v);
          else *dst = v;
        } else if (p.c_bf16) {
          reinterpret_cast<uint16_t*>(p.c)[tok * p.ldc + c] = (uint16_t)f32_to_bf16_bits(v * alpha);
        } else {
          reinterpret_cast<float*>(p.c)[tok * p.ldc + c] = v * alpha;
        }
      }
    if (part && p.tickets != nullptr) {
      stores_done();
      uint32_t last = 0;
      if (lane == 0) last = last_arrival(p.tickets + ct, p.splits) ? 1u : 0u;
      if (!__builtin_amdgcn_readfirstlane((int)last)) return;
      // the tile's M x 32 outputs (NQ per lane), their partial sums added in
      // split order as finish_output does, with SB splits' loads of all NQ in
      // flight at a time
      constexpr int NQ = MT * CW / 64, SB = 64 / NQ;
      const int64_t plane = M * N;
      float sum[NQ];
      int64_t idx[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        sum[q] = 0.f;
        const int o = lane + 64 * q;
        const int64_t tok = o / CW < M ? o / CW : M - 1, c = n0 + o % CW < N ? n0 + o % CW : N - 1;
        idx[q] = tok * N + c;
      }
      for (uint32_t s0 = 0; s0 < p.splits; s0 += SB) {
        float l[NQ][SB];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int k = 0; k < SB; ++k) {
            const uint32_t s2 = s0 + k < p.splits ? s0 + k : p.splits - 1;
            l[q][k] = load_coherent(p.split_out + (int64_t)s2 * plane + idx[q]);
          }
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int k = 0; k < SB; ++k)
            if (s0 + k < p.splits) sum[q] += l[q][k];
      }
      float am = 0.f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int o = lane + 64 * q;
        const int64_t tok = o / CW, c = n0 + o % CW;
        if (tok < M && c < N) am = fmaxf(am, store_output(p, tok, c, sum[q]));
      }
      if (p.amax_slots != nullptr) {
        am = wave_max(am);
        if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(p.amax_slots + ct % kAmaxSlots), __float_as_uint(am));
      }
    }
  }
}

// Words cleared before a launch whose work items take tickets.
__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

// Output amax: each work-group writes the largest |stored value| it produced
// (after the bf16 rounding for bf16 outputs: rounding is monotone, so the max
// of the rounded values is the rounded max) to its own slot; with an amax
// output the reduction runs exactly kAmaxSlots work-groups, so the max over
// the slots is max |C|.  No atomics (thousands of work-groups taking turns on
// one word cost tens of microseconds) and nothing to clear.
__device__ __forceinline__ void fold_amax(float m, float* amax) {
  __shared__ float red[4];
  m = block_max(m, red);
  if (threadIdx.x == 0) amax[blockIdx.x] = m;
}

__device__ __forceinline__ float stored_abs(float v, int bf16) {
  return bf16 ? __uint_as_float(f32_to_bf16_bits(fabsf(v)) << 16) : fabsf(v);
}

// Expert of slot m: the last e with off[e] <= m (binary search over the
// non-decreasing offsets; empty experts share their offset with the next one).
__device__ __forceinline__ int expert_of(const int32_t* off, int E, int64_t m) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// out[m][n] = (sum over splits, in split order) * gs_a * gs_b[expert of slot m].
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, uint32_t splits,
                                                            int64_t M, int64_t N, const float* a_gs,
                                                            const float* b_gs, const int32_t* off, int E,
                                                            void* out, int out_bf16, int64_t ldo, float* amax) {
  const int64_t total = M * N;
  const float ga = a_gs[0];
  float vmax = 0.f;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / N, n = idx - m * N;
    // loads in batches of eight, added in split order
    float acc = 0.f;
    uint32_t s = 0;
    for (; s + 8u <= splits; s += 8u) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = part[(int64_t)(s + k) * total + idx];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += v[k];
    }
    for (; s < splits; ++s) acc += part[(int64_t)s * total + idx];
    const int e = off ? expert_of(off, E, m) : 0;
    const float v = acc * (ga * b_gs[e]);
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[m * ldo + n] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(out)[m * ldo + n] = v;
    vmax = fmaxf(vmax, stored_abs(v, out_bf16));
  }
  if (amax) fold_amax(vmax, amax);
}

// The same reduction with four consecutive outputs of one row per thread
// (N % 4 == 0): 16-byte loads of each split's partials, added in split order,
// so the sums are those of splitk_reduce_kernel bit for bit.
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(const float* __restrict__ part, uint32_t splits,
                                                             int64_t M, int64_t N, const float* a_gs,
                                                             const float* b_gs, const int32_t* off, int E,
                                                             void* out, int out_bf16, int64_t ldo, float* amax) {
  const int64_t total = M * N, total4 = total / 4;
  const float ga = a_gs[0];
  float vmax = 0.f;
  for (int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x; i4 < total4; i4 += (int64_t)gridDim.x * 256) {
    const int64_t idx = 4 * i4, m = idx / N, n = idx - m * N;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t s = 0;
    for (; s + 4u <= splits; s += 4u) {
      float4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const float4*>(part + (int64_t)(s + k) * total + idx);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc.x += v[k].x;
        acc.y += v[k].y;
        acc.z += v[k].z;
        acc.w += v[k].w;
      }
    }
    for (; s < splits; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)s * total + idx);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int e = off ? expert_of(off, E, m) : 0;
    const float sc = ga * b_gs[e];
    const float4 o = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    if (out_bf16) {
      const uint32_t lo = f32_to_bf16_bits(o.x) | (f32_to_bf16_bits(o.y) << 16);
      const uint32_t hi = f32_to_bf16_bits(o.z) | (f32_to_bf16_bits(o.w) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + m * ldo + n) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + m * ldo + n) = o;
    }
    vmax = fmaxf(fmaxf(vmax, stored_abs(o.x, out_bf16)), stored_abs(o.y, out_bf16));
    vmax = fmaxf(fmaxf(vmax, stored_abs(o.z, out_bf16)), stored_abs(o.w, out_bf16));
  }
  if (amax) fold_amax(vmax, amax);
}

// The same reduction, quantised: each thread takes whole 16-column blocks,
// adds the splits in split order, scales by gs_a * gs_b (the float32 values
// splitk_reduce_kernel would store) and quantises them with the given global
// scale.
__global__ void __launch_bounds__(256) splitk_reduce_quant_kernel(const float* __restrict__ part, uint32_t splits,
                                                                  int64_t M, int64_t N, const float* a_gs,
                                                                  const float* b_gs, const float* q_gs,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  const int64_t nbc = N / 16, total = M * nbc, plane = M * N;
  const float alpha = a_gs[0] * b_gs[0];
  const float gs = q_gs[0];
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < total; b += (int64_t)gridDim.x * 256) {
    const int64_t m = b / nbc, cb = b - m * nbc;
    const float* src = part + m * N + cb * 16;
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = 0.f;
    // loads of two splits in flight at a time, added in split order
    uint32_t sp = 0;
    for (; sp + 2u <= splits; sp += 2u) {
      float4 t4[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          t4[h][g4] = *reinterpret_cast<const float4*>(src + (int64_t)(sp + h) * plane + 4 * g4);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          v[4 * g4] += t4[h][g4].x;
          v[4 * g4 + 1] += t4[h][g4].y;
          v[4 * g4 + 2] += t4[h][g4].z;
          v[4 * g4 + 3] += t4[h][g4].w;
        }
    }
    for (; sp < splits; ++sp) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 t4 = *reinterpret_cast<const float4*>(src + (int64_t)sp * plane + 4 * g4);
        v[4 * g4] += t4.x;
        v[4 * g4 + 1] += t4.y;
        v[4 * g4 + 2] += t4.z;
        v[4 * g4 + 3] += t4.w;
      }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] *= alpha;
    uint32_t w0, w1;
    const uint32_t sc = quantize_block16(v, gs, w0, w1);
    *reinterpret_cast<uint2*>(codes + b * 8) = make_uint2(w0, w1);
    scales[b] = (uint8_t)sc;
  }
}

// ---- launch configurations ----------------------------------------------------------
// Large batches: four waves side by side in N, each 32 * TM rows x 32 columns
// of both the gate and the up matrix, or (store epilogue) 32 * TM rows x
// 32 * NVFP4_STORE_TN columns of one matrix.  Small batches (M <= 32): the weight-stream
// kernel, 32 weight rows per work-group, K split over its waves (and, for the
// store epilogue, over work-groups too).
struct Plan {
  bool small;
  int gv_bpl;   // > 0: the one/two-token weight stream with BPL units of K per split
  bool tl;      // the 3-16 token stream (chunks_per_split: stages of 256 per split)
  uint32_t m_tiles, n_tiles, splits, chunks_per_split;
};

static uint32_t cdiv(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

// The weight stream takes M <= NVFP4_GV_MAXT tokens and K >= 1024 (a multiple
// of 16; the last 1024-wide unit may be partial); a split covers BPL units (the
// largest divisor of the unit count up to 5, else 2 with a shorter last split).  The gate/up pair needs whole
// rows in one split (GLU epilogue), so there K <= 5120.
struct GvPlan {
  int bpl;          // 0: not applicable
  uint32_t splits;
};

static GvPlan plan_gemv(int64_t M, int64_t K, bool dual) {
  GvPlan pl{0, 0};
  if (M < 1 || M > NVFP4_GV_MAXT || K % 16 != 0 || K < 1024) return pl;
  const int64_t U = (K + 1023) / 1024;            // the last unit may be partial
  int bpl = 1;
  for (int b = 5; b >= 2; --b)
    if (U % b == 0) {
      bpl = b;
      break;
    }
  // No divisor up to 5 (U prime, e.g. 17 units for K = 17408): two units per
  // lane with a shorter last split beat one-unit splits (half the partial sums
  // and twice the bytes per row and wave; measured on the 5120 x 17408 down
  // projection at one token).
  if (!dual && bpl == 1 && U > 2) bpl = 2;
  const int64_t S = (U + bpl - 1) / bpl;          // the last split may hold fewer units
  if ((dual && S != 1) || S > 64) return pl;
  pl.bpl = bpl;
  pl.splits = (uint32_t)S;
  return pl;
}

// The 3-16 token stream: K a multiple of 256 (one stage); K is cut into
// splits of about NVFP4_TL_SPS stages, so that thousands of waves share the
// weights; with the gate/up pair N is a multiple of 16 (whole column tiles).
struct TlPlan {
  bool ok;
  uint32_t splits, sps;   // K splits, stages per split
};

static TlPlan plan_tile(int64_t M, int64_t N, int64_t K, bool dual) {
  TlPlan pl{false, 0, 0};
  if (M < 3 || M > kTlMaxT || K < kTlStageK || K % kTlStageK != 0 || (dual && N % 16 != 0)) return pl;
  const int64_t U = K / kTlStageK;
  const int64_t S0 = (U + NVFP4_TL_SPS - 1) / NVFP4_TL_SPS;
  pl.sps = cdiv(U, S0);
  pl.splits = cdiv(U, pl.sps);
  pl.ok = true;
  return pl;
}

static Plan plan_store(int64_t M, int64_t N, int64_t K, int E, bool grouped) {
  Plan pl{};
  if (!grouped) {
    const GvPlan gv = plan_gemv(M, K, false);
    if (gv.bpl > 0) {
      pl.small = true;
      pl.gv_bpl = gv.bpl;
      pl.m_tiles = 1;
      pl.n_tiles = cdiv(N, kGvCols);
      pl.splits = gv.splits;
      pl.chunks_per_split = 0;
      return pl;
    }
    const TlPlan tl = plan_tile(M, N, K, false);
    if (tl.ok) {
      pl.small = true;
      pl.tl = true;
      pl.m_tiles = 1;
      pl.n_tiles = cdiv(N, 32);
      pl.splits = tl.splits;
      pl.chunks_per_split = tl.sps;
      return pl;
    }
  }
  pl.small = !grouped && M <= 32;
  const uint32_t chunks = (uint32_t)(K / 128);
  uint32_t s = 1;
  if (pl.small) {
    // Weight stream: split K until there are >= 512 work-groups (>= 2 waves
    // per SIMD), keeping >= 4 chunks per wave.
    pl.m_tiles = 1;
    pl.n_tiles = cdiv(N, 32);
    while (s < 16 && pl.n_tiles * s < 512 && chunks / (s + 1) >= 4u * kSkWaves) ++s;
  } else {
    pl.m_tiles = grouped ? cdiv(M, 32 * NVFP4_STORE_TM) + (uint32_t)E : cdiv(M, 32 * NVFP4_STORE_TM);
    pl.n_tiles = cdiv(N, 32 * NVFP4_STORE_WN * (grouped ? NVFP4_GROUPED_STORE_TN : NVFP4_STORE_TN));
    // Split K until there are enough work-groups, keeping >= 8 chunks per split.
    const uint32_t tiles = pl.m_tiles * pl.n_tiles;
    while (s < 8 && tiles * s < NVFP4_SPLIT_TARGET && chunks / (s + 1) >= 8) ++s;
  }
  pl.chunks_per_split = cdiv(chunks, s);
  pl.splits = cdiv(chunks, pl.chunks_per_split);
  return pl;
}

template <bool DUAL, int EPI>
static void launch_skinny(const GemmArgs& g, hipStream_t st) {
  const uint32_t grid = g.n_tiles * g.splits;
  const int slot = launch_begin(EPI != EPI_STORE ? KC_GEMM_GLU : KC_GEMM_STORE, st);
  hipLaunchKernelGGL((skinny_kernel<DUAL, EPI>), dim3(grid), dim3(kSkWaves * 64), 0, st, g);
  launch_end(slot, st);
}

template <int T, bool DUAL, int EPI, bool WGK = false>
static void launch_gemv_t(const GemmArgs& g, int bpl, uint32_t grid, uint32_t block, hipStream_t st) {
  switch (bpl) {
    case 1: hipLaunchKernelGGL((gemv_kernel<T, 1, DUAL, EPI, WGK>), dim3(grid), dim3(block), 0, st, g); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<T, 2, DUAL, EPI, WGK>), dim3(grid), dim3(block), 0, st, g); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<T, 3, DUAL, EPI, WGK>), dim3(grid), dim3(block), 0, st, g); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<T, 4, DUAL, EPI, WGK>), dim3(grid), dim3(block), 0, st, g); break;
    default: hipLaunchKernelGGL((gemv_kernel<T, 5, DUAL, EPI, WGK>), dim3(grid), dim3(block), 0, st, g); break;
  }
}

// g.splits holds the K splits; one wave per kGvCols output columns per
// split.  The store epilogue with its split-K finished in the kernel (tickets
// given) takes one work-group per column group, its splits added in LDS.
template <bool DUAL, int EPI>
static void launch_gemv(const GemmArgs& g, int bpl, hipStream_t st) {
  const int slot = launch_begin(EPI != EPI_STORE ? KC_GEMM_GLU : KC_GEMM_STORE, st);
  if constexpr (!DUAL && EPI == EPI_STORE) {
    if (g.tickets != nullptr && g.splits > 1 && g.splits <= (uint32_t)kGvWgkSplits) {
      const uint32_t grid = cdiv(g.N, kGvCols), block = 64u * g.splits;
      if (g.M <= 1) launch_gemv_t<1, false, EPI_STORE, true>(g, bpl, grid, block, st);
      else launch_gemv_t<NVFP4_GV_MAXT, false, EPI_STORE, true>(g, bpl, grid, block, st);
      launch_end(slot, st);
      return;
    }
  }
  const uint32_t waves = cdiv(g.N, kGvCols) * g.splits;
  const uint32_t grid = cdiv(waves, 4);
  if (g.M <= 1) launch_gemv_t<1, DUAL, EPI>(g, bpl, grid, 256, st);
  else launch_gemv_t<NVFP4_GV_MAXT, DUAL, EPI>(g, bpl, grid, 256, st);
  launch_end(slot, st);
}

// g.splits holds the K splits and g.chunks_per_split the stages per split;
// one wave per column tile per split.
template <bool DUAL, int EPI>
static void launch_tile(const GemmArgs& g, hipStream_t st) {
  const uint32_t items = cdiv(g.N, DUAL ? 16 : 32) * g.splits;
  const int slot = launch_begin(EPI != EPI_STORE ? KC_GEMM_GLU : KC_GEMM_STORE, st);
  if (g.M <= 8)
    hipLaunchKernelGGL((tile_kernel<8, DUAL, EPI>), dim3(cdiv(items, kTlWaves)), dim3(kTlWaves * 64), 0, st, g);
  else
    hipLaunchKernelGGL((tile_kernel<16, DUAL, EPI>), dim3(cdiv(items, kTlWaves)), dim3(kTlWaves * 64), 0, st, g);
  launch_end(slot, st);
}

static void launch_clear(uint32_t* p, uint32_t n, int kc, hipStream_t st) {
  uint32_t grid = cdiv(n, 256);
  if (grid > 64u) grid = 64u;
  if (grid < 1u) grid = 1u;
  const int slot = launch_begin(kc, st);
  hipLaunchKernelGGL(clear_words_kernel, dim3(grid), dim3(256), 0, st, p, n);
  launch_end(slot, st);
}

// Compute units of the current device, read once per device.
static uint32_t cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return (uint32_t)n;
}

template <int WN, int TM, int TN, bool DUAL, bool GROUPED, int EPI>
static void launch_cfg(const GemmArgs& g, hipStream_t st) {
  const uint32_t tiles = g.m_tiles * g.n_tiles * g.splits;
  constexpr int MW0 = EPI != EPI_STORE ? NVFP4_GLU_MINWG : NVFP4_STORE_MINWG;
  uint32_t grid = tiles;
  if (NVFP4_PERSIST && (!GROUPED || NVFP4_PERSIST_GROUPED)) {
    // the work-groups the chip holds at once, a multiple of the 8 XCDs
    uint32_t resident = cu_count() * (uint32_t)MW0;
    if (resident > 8u) resident -= resident % 8u;
    if (grid > resident) grid = resident;
  }
  const int slot = launch_begin(EPI != EPI_STORE ? KC_GEMM_GLU : KC_GEMM_STORE, st);
  constexpr int NS = EPI != EPI_STORE ? NVFP4_GLU_STAGES : NVFP4_STORE_STAGES;
  constexpr int MW = EPI != EPI_STORE ? NVFP4_GLU_MINWG : NVFP4_STORE_MINWG;
  hipLaunchKernelGGL((gemm_kernel<WN, TM, TN, DUAL, GROUPED, EPI, NS, MW>), dim3(grid), dim3(WN * 64), 0, st, g);
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
                          float* amax, hipStream_t st) {
  const bool vec = N % 4 == 0;   // four outputs per thread (partials, rows and output rows 16-B aligned)
  int64_t blocks = (M * N / (vec ? 4 : 1) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (amax) blocks = kAmaxSlots;  // one partial maximum per slot (grid-stride over the outputs)
  const int slot = launch_begin(KC_REDUCE, st);
  if (vec)
    hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, part, splits, M, N, a_gs,
                       b_gs, off, E, out, bf16, ldo, amax);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, part, splits, M, N, a_gs,
                       b_gs, off, E, out, bf16, ldo, amax);
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
  g.b_tiled = b.tiled;
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
                 int64_t K, void* c, int c_bf16, int64_t ldc, float* c_amax, void* ws, hipStream_t st,
                 const _Float16* a16_given) {
  const bool grouped = off != nullptr;
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)M * K * 2));
  const Plan pl = plan_store(M, N, K, E, grouped);
  // the weight streams expand the activation themselves; a given copy needs no expansion
  if (a16_given != nullptr && (!grouped || rows == nullptr)) a16 = const_cast<_Float16*>(a16_given);
  else if (grouped || (pl.gv_bpl == 0 && !pl.tl)) launch_expand(a.codes, a.scales, rows, M, K, a16, st);
  GemmArgs g = base_args(a16, a.gscale, w, M, N, K);
  g.a_codes = a.codes;
  g.a_scales = a.scales;
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
  // With an output amax every output goes through the reduction (the
  // contraction writes partial sums even when K is not split), which takes the
  // amax of what it stores.
  g.force_split = c_amax != nullptr;
  if (grouped) launch_cfg<NVFP4_STORE_WN, NVFP4_STORE_TM, NVFP4_GROUPED_STORE_TN, false, true, EPI_STORE>(g, st);
  else if (pl.gv_bpl > 0) launch_gemv<false, EPI_STORE>(g, pl.gv_bpl, st);
  else if (pl.tl) launch_tile<false, EPI_STORE>(g, st);
  else if (pl.small) launch_skinny<false, EPI_STORE>(g, st);
  else launch_cfg<NVFP4_STORE_WN, NVFP4_STORE_TM, NVFP4_STORE_TN, false, false, EPI_STORE>(g, st);
  // The reduction always runs (over zero rows when K was not split), so the
  // number of launches never depends on the shape.
  launch_reduce(part, pl.splits, (pl.splits > 1 || c_amax) ? M : 0, N, a.gscale, w.gscale, off, E, c, c_bf16, ldc,
                c_amax, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

// GLU GEMM.  Workspace: [H float32 M x N][A f16 M x K][partials].
static uint32_t glu_parts(int64_t M, int64_t N, int64_t K, int E, bool grouped) {
  if (grouped) return (cdiv(M, 32 * NVFP4_GLU_TM) + (uint32_t)E) * cdiv(N, 32 * NVFP4_GLU_WN);
  if (plan_gemv(M, K, true).bpl > 0) return cdiv(N, kGvCols);   // one partial per wave
  if (plan_tile(M, N, K, true).ok) return cdiv(N, 16);          // one partial per column tile
  if (M <= 32) return cdiv(N, 32);
  return cdiv(M, 32 * NVFP4_GLU_TM) * cdiv(N, 32 * NVFP4_GLU_WN);
}

// The gate/up pair on the 3-16 token stream with K split: partial sums
// [splits][M][2N] (gate, then up, per token) and one ticket per column tile.
static size_t tile_dual_bytes(int64_t M, int64_t N, int64_t K) {
  const TlPlan tl = plan_tile(M, N, K, true);
  if (!tl.ok || tl.splits < 2) return 0;
  return align256((size_t)tl.splits * M * 2 * N * 4) + align256((size_t)cdiv(N, 16) * 4);
}

// Points g at the split partial sums and tickets in `w` (tile_dual_bytes of
// space) and clears the tickets; no-op when K is not split.
static void tile_dual_setup(GemmArgs& g, const TlPlan& tl, char* w, hipStream_t st) {
  g.splits = tl.splits;
  g.chunks_per_split = tl.sps;
  if (tl.splits < 2) return;
  g.split_out = reinterpret_cast<float*>(w);
  g.tickets = reinterpret_cast<uint32_t*>(w + align256((size_t)tl.splits * g.M * 2 * g.N * 4));
  launch_clear(g.tickets, cdiv(g.N, 16), KC_GEMM_GLU, st);
}

size_t glu_ws_bytes(int64_t M, int64_t N, int64_t K, int E, bool grouped, bool gather) {
  return align256((size_t)M * N * 4) + (gather ? 0 : align256((size_t)M * K * 2)) +
         align256((size_t)glu_parts(M, N, K, E, grouped) * 4) + (grouped ? 0 : tile_dual_bytes(M, N, K));
}

int glu_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt, Operand up,
               int64_t N, int64_t K, uint8_t* hq_codes, uint8_t* hq_scales, float* hq_gs, void* ws,
               hipStream_t st, const _Float16* a16_given, _Float16* hq16, int64_t gather_rows) {
  const bool grouped = off != nullptr;
  const bool gather = grouped && a16_given != nullptr;   // slot rows staged from the token copy via a_rows
  float* h = reinterpret_cast<float*>(ws);
  _Float16* a16 = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(ws) + align256((size_t)M * N * 4));
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a16) + (gather ? 0 : align256((size_t)M * K * 2)));
  const bool stream = !grouped && (plan_gemv(M, K, true).bpl > 0 || plan_tile(M, N, K, true).ok);
  if (a16_given != nullptr) a16 = const_cast<_Float16*>(a16_given);
  else if (!stream) launch_expand(a.codes, a.scales, a_rows, M, K, a16, st);   // the streams expand x~ themselves
  GemmArgs g = base_args(a16, a.gscale, gt, M, N, K);
  if (gather) {
    g.a_gather = a_rows;
    g.a_gather_rows = gather_rows;
  }
  g.a_codes = a.codes;
  g.a_scales = a.scales;
  g.u_codes = up.codes;
  g.u_scales = up.scales;
  g.u_gs = up.gscale;
  g.u_tiled = up.tiled;
  g.h = h;
  g.partials = partials;
  g.off = off;
  g.E = E;
  g.chunks_per_split = (uint32_t)(K / 128);
  if (grouped) {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM) + (uint32_t)E;
    g.n_tiles = cdiv(N, 32 * NVFP4_GLU_WN);
    launch_cfg<NVFP4_GLU_WN, NVFP4_GLU_TM, 1, true, true, EPI_GLU>(g, st);
  } else if (const GvPlan gv = plan_gemv(M, K, true); gv.bpl > 0) {
    launch_gemv<true, EPI_GLU>(g, gv.bpl, st);
  } else if (const TlPlan tl = plan_tile(M, N, K, true); tl.ok) {
    tile_dual_setup(g, tl, reinterpret_cast<char*>(partials) + align256((size_t)glu_parts(M, N, K, E, grouped) * 4), st);
    launch_tile<true, EPI_GLU>(g, st);
  } else if (M <= 32) {
    g.m_tiles = 1;
    g.n_tiles = cdiv(N, 32);
    launch_skinny<true, EPI_GLU>(g, st);
  } else {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM);
    g.n_tiles = cdiv(N, 32 * NVFP4_GLU_WN);
    launch_cfg<NVFP4_GLU_WN, NVFP4_GLU_TM, 1, true, false, EPI_GLU>(g, st);
  }
  if (hipGetLastError() != hipSuccess) return 7;
  return requant_f32_launch(h, M, N, hq_codes, hq_scales, hq_gs, partials, glu_parts(M, N, K, E, grouped), st, hq16);
}

size_t glu_static_ws_bytes(int64_t M, int64_t N, int64_t K, bool grouped, bool gather) {
  return (gather ? 0 : align256((size_t)M * K * 2)) + (grouped ? 0 : tile_dual_bytes(M, N, K));
}

int glu_static_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt,
                      Operand up, int64_t N, int64_t K, uint8_t* hq_codes, uint8_t* hq_scales, const float* hq_gs,
                      void* ws, hipStream_t st, const _Float16* a16_given, _Float16* hq16, int64_t gather_rows) {
  const bool gather = off != nullptr && a16_given != nullptr;   // slot rows staged from the token copy via a_rows
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  const bool stream = !off && (plan_gemv(M, K, true).bpl > 0 || plan_tile(M, N, K, true).ok);
  if (a16_given != nullptr) a16 = const_cast<_Float16*>(a16_given);
  else if (!stream) launch_expand(a.codes, a.scales, a_rows, M, K, a16, st);   // the streams expand x~ themselves
  GemmArgs g = base_args(a16, a.gscale, gt, M, N, K);
  if (gather) {
    g.a_gather = a_rows;
    g.a_gather_rows = gather_rows;
  }
  g.q16 = off != nullptr ? hq16 : nullptr;   // written by the expert-grouped contraction's epilogue
  g.a_codes = a.codes;
  g.a_scales = a.scales;
  g.u_codes = up.codes;
  g.u_scales = up.scales;
  g.u_gs = up.gscale;
  g.u_tiled = up.tiled;
  g.q_codes = hq_codes;
  g.q_scales = hq_scales;
  g.q_gs = hq_gs;
  g.chunks_per_split = (uint32_t)(K / 128);
  g.off = off;
  g.E = E;
  if (off) {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM) + (uint32_t)E;
    g.n_tiles = cdiv(N, 32 * NVFP4_GLU_WN);
    launch_cfg<NVFP4_GLU_WN, NVFP4_GLU_TM, 1, true, true, EPI_GLUQ>(g, st);
  } else if (const GvPlan gv = plan_gemv(M, K, true); gv.bpl > 0) {
    launch_gemv<true, EPI_GLUQ>(g, gv.bpl, st);
  } else if (const TlPlan tl = plan_tile(M, N, K, true); tl.ok) {
    tile_dual_setup(g, tl, reinterpret_cast<char*>(ws) + (a16_given != nullptr ? 0 : align256((size_t)M * K * 2)), st);
    launch_tile<true, EPI_GLUQ>(g, st);
  } else if (M <= 32) {
    g.m_tiles = 1;
    g.n_tiles = cdiv(N, 32);
    launch_skinny<true, EPI_GLUQ>(g, st);
  } else {
    g.m_tiles = cdiv(M, 32 * NVFP4_GLU_TM);
    g.n_tiles = cdiv(N, 32 * NVFP4_GLU_WN);
    launch_cfg<NVFP4_GLU_WN, NVFP4_GLU_TM, 1, true, false, EPI_GLUQ>(g, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int store_quant_launch(Operand a, int64_t M, Operand w, int64_t N, int64_t K, uint8_t* yq_codes, uint8_t* yq_scales,
                       const float* yq_gs, void* ws, hipStream_t st) {
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)M * K * 2));
  const Plan pl = plan_store(M, N, K, 1, false);
  if (pl.gv_bpl == 0 && !pl.tl) launch_expand(a.codes, a.scales, nullptr, M, K, a16, st);
  GemmArgs g = base_args(a16, a.gscale, w, M, N, K);
  g.a_codes = a.codes;
  g.a_scales = a.scales;
  g.splits = pl.splits;
  g.chunks_per_split = pl.chunks_per_split;
  g.split_out = part;
  g.force_split = 1;
  g.m_tiles = pl.m_tiles;
  g.n_tiles = pl.n_tiles;
  if (pl.gv_bpl > 0) launch_gemv<false, EPI_STORE>(g, pl.gv_bpl, st);
  else if (pl.tl) launch_tile<false, EPI_STORE>(g, st);
  else if (pl.small) launch_skinny<false, EPI_STORE>(g, st);
  else launch_cfg<NVFP4_STORE_WN, NVFP4_STORE_TM, NVFP4_STORE_TN, false, false, EPI_STORE>(g, st);
  int64_t blocks = (M * (N / 16) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const int slot = launch_begin(KC_REDUCE, st);
  hipLaunchKernelGGL(splitk_reduce_quant_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, part, pl.splits, M, N,
                     a.gscale, w.gscale, yq_gs, yq_codes, yq_scales);
  launch_end(slot, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

// ---- whole MLP ---------------------------------------------------------------------
// Decode path: both projections on the weight streams and x small enough for
// the one-work-group quantiser.
struct MlpDecodePlan {
  bool ok;
  GvPlan gu_gv;
  TlPlan gu_tl;
  Plan dn;
  uint32_t groups;      // column groups of the down projection (tickets)
  uint32_t gu_groups;   // column tiles of the gate/up pair when its K is split (tickets)
};

static MlpDecodePlan plan_mlp_decode(int64_t T, int64_t K, int64_t I) {
  MlpDecodePlan d{};
  if (T < 1 || T > kTlMaxT || T * (K / 16) > (int64_t)kSmallQuantBlocks) return d;
  d.gu_gv = plan_gemv(T, K, true);
  d.gu_tl = plan_tile(T, I, K, true);
  if (d.gu_gv.bpl == 0 && !d.gu_tl.ok) return d;
  d.dn = plan_store(T, K, I, 1, false);
  if (d.dn.gv_bpl == 0 && !d.dn.tl) return d;
  d.groups = d.dn.gv_bpl > 0 ? cdiv(K, kGvCols) : cdiv(K, 32);
  d.gu_groups = d.gu_tl.ok && d.gu_tl.splits > 1 ? cdiv(I, 16) : 0;
  d.ok = true;
  return d;
}

size_t moe_mlp_ws_bytes(int64_t T, int64_t K, int64_t I, int E, int64_t M) {
  return align256(quantize_ws_bytes(T, K, 0)) + align256((size_t)T * K * 2) + align256(glu_ws_bytes(M, I, K, E, true, true)) +
         align256(store_ws_bytes(M, K, I, E, true));
}

int moe_mlp_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                   const int32_t* a_rows, const int32_t* off, int64_t M, Operand wg, Operand wu, Operand wd,
                   uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
                   float* hq_gs, void* y, int y_bf16, int64_t ldy, void* ws, hipStream_t st) {
  char* w = reinterpret_cast<char*>(ws);
  const size_t q_bytes = align256(quantize_ws_bytes(T, K, 0));
  _Float16* x16 = reinterpret_cast<_Float16*>(w + q_bytes);
  char* wg_ws = w + q_bytes + align256((size_t)T * K * 2);
  char* wd_ws = wg_ws + align256(glu_ws_bytes(M, I, K, E, true, true));
  _Float16* h16 = reinterpret_cast<_Float16*>(wd_ws);   // the down projection's f16 slot
  int rc = quantize_launch(x, x_dtype, T, K, ld_x, xq_codes, xq_scales, xq_gs, 0, w, st, x16);
  if (rc) return rc;
  const Operand xq{xq_codes, xq_scales, xq_gs, nullptr};
  if ((rc = glu_launch(xq, a_rows, off, E, M, wg, wu, I, K, hq_codes, hq_scales, hq_gs, wg_ws, st, x16, h16, T)))
    return rc;
  const Operand hq{hq_codes, hq_scales, hq_gs, nullptr};
  return store_launch(hq, nullptr, off, E, M, wd, K, I, y, y_bf16, ldy, nullptr, wd_ws, st, h16);
}

size_t moe_mlp_static_ws_bytes(int64_t T, int64_t K, int64_t I, int E, int64_t M) {
  return align256((size_t)T * K * 2) + align256(glu_static_ws_bytes(M, I, K, true, true)) +
         align256(store_ws_bytes(M, K, I, E, true));
}

int moe_mlp_static_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                          const int32_t* a_rows, const int32_t* off, int64_t M, Operand wg, Operand wu, Operand wd,
                          uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
                          const float* hq_gs, void* y, int y_bf16, int64_t ldy, void* ws, hipStream_t st) {
  char* w = reinterpret_cast<char*>(ws);
  _Float16* x16 = reinterpret_cast<_Float16*>(w);
  char* wg_ws = w + align256((size_t)T * K * 2);
  char* wd_ws = wg_ws + align256(glu_static_ws_bytes(M, I, K, true, true));
  _Float16* h16 = reinterpret_cast<_Float16*>(wd_ws);   // the down projection's f16 slot
  int rc = quantize_launch(x, x_dtype, T, K, ld_x, xq_codes, xq_scales, xq_gs, 1, nullptr, st, x16);
  if (rc) return rc;
  const Operand xq{xq_codes, xq_scales, xq_gs, nullptr};
  if ((rc = glu_static_launch(xq, a_rows, off, E, M, wg, wu, I, K, hq_codes, hq_scales, hq_gs, wg_ws, st, x16, h16,
                              T)))
    return rc;
  const Operand hq{hq_codes, hq_scales, const_cast<float*>(hq_gs), nullptr};
  return store_launch(hq, nullptr, off, E, M, wd, K, I, y, y_bf16, ldy, nullptr, wd_ws, st, h16);
}

size_t mlp_ws_bytes(int64_t T, int64_t K, int64_t I) {
  const MlpDecodePlan d = plan_mlp_decode(T, K, I);
  if (d.ok)   // [H float32][|H| partials][down partial sums][tickets: down, gate/up][gate/up partial sums]
    return align256((size_t)T * I * 4) + align256((size_t)glu_parts(T, I, K, 1, false) * 4) +
           align256((size_t)d.dn.splits * T * K * 4) + align256((size_t)(d.groups + d.gu_groups) * 4) +
           (d.gu_groups ? align256((size_t)d.gu_tl.splits * T * 2 * I * 4) : 0);
  // [quantiser partial maxima][gate/up workspace][down workspace]
  return align256(quantize_ws_bytes(T, K, 0)) + align256(glu_ws_bytes(T, I, K, 1, false)) +
         align256(store_ws_bytes(T, K, I, 1, false));
}

int mlp_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, Operand wg, Operand wu,
               Operand wd, uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
               float* hq_gs, void* y, int y_bf16, int64_t ldy, const float* x_amax, float* y_amax, void* ws,
               hipStream_t st) {
  char* w = reinterpret_cast<char*>(ws);
  const MlpDecodePlan d = plan_mlp_decode(T, K, I);
  if (!d.ok) {
    // The separate calls' kernels, but each quantiser also writes the f16
    // operand copy the next contraction reads (into that contraction's
    // workspace), so neither contraction needs an expansion launch.
    const size_t q_bytes = align256(quantize_ws_bytes(T, K, 0));
    const size_t g_bytes = align256(glu_ws_bytes(T, I, K, 1, false));
    char* wg_ws = w + q_bytes;
    char* wd_ws = w + q_bytes + g_bytes;
    _Float16* x16 = reinterpret_cast<_Float16*>(wg_ws + align256((size_t)T * I * 4));   // the gate/up's a16 slot
    _Float16* h16 = reinterpret_cast<_Float16*>(wd_ws);                                // the down's a16 slot
    int rc = x_amax ? quantize_launch(x, x_dtype, T, K, ld_x, xq_codes, xq_scales, xq_gs, 2, const_cast<float*>(x_amax),
                                      st, x16)
                    : quantize_launch(x, x_dtype, T, K, ld_x, xq_codes, xq_scales, xq_gs, 0, w, st, x16);
    if (rc) return rc;
    const Operand xq{xq_codes, xq_scales, xq_gs};
    if ((rc = glu_launch(xq, nullptr, nullptr, 1, T, wg, wu, I, K, hq_codes, hq_scales, hq_gs, wg_ws, st, x16, h16)))
      return rc;
    const Operand hq{hq_codes, hq_scales, hq_gs};
    return store_launch(hq, nullptr, nullptr, 1, T, wd, K, I, y, y_bf16, ldy, y_amax, wd_ws, st, h16);
  }
  float* h = reinterpret_cast<float*>(w);
  w += align256((size_t)T * I * 4);
  float* partials = reinterpret_cast<float*>(w);
  const uint32_t npart = glu_parts(T, I, K, 1, false);
  w += align256((size_t)npart * 4);
  float* part = reinterpret_cast<float*>(w);
  w += align256((size_t)d.dn.splits * T * K * 4);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)(d.groups + d.gu_groups) * 4);
  float* gu_part = reinterpret_cast<float*>(w);

  // 1: quantise x; clear the tickets and the output-amax slots
  int rc = mlp_prologue_launch(x, x_dtype, T, K, ld_x, xq_codes, xq_scales, xq_gs, x_amax, tickets,
                               d.groups + d.gu_groups, reinterpret_cast<uint32_t*>(y_amax), y_amax ? kAmaxSlots : 0u,
                               st);
  if (rc) return rc;
  // 2: gate/up weight stream, SiLU*up epilogue, float32 H and its partial maxima
  GemmArgs g = base_args(nullptr, xq_gs, wg, T, I, K);
  g.a_codes = xq_codes;
  g.a_scales = xq_scales;
  g.u_codes = wu.codes;
  g.u_scales = wu.scales;
  g.u_gs = wu.gscale;
  g.u_tiled = wu.tiled;
  g.h = h;
  g.partials = partials;
  if (d.gu_gv.bpl > 0) {
    launch_gemv<true, EPI_GLU>(g, d.gu_gv.bpl, st);
  } else {
    g.splits = d.gu_tl.splits;
    g.chunks_per_split = d.gu_tl.sps;
    if (d.gu_groups) {
      g.split_out = gu_part;
      g.tickets = tickets + d.groups;
    }
    launch_tile<true, EPI_GLU>(g, st);
  }
  if (hipGetLastError() != hipSuccess) return 7;
  // 3: requantise H with its global scale
  if ((rc = requant_f32_launch(h, T, I, hq_codes, hq_scales, hq_gs, partials, npart, st))) return rc;
  // 4: down weight stream; the last-arriving wave (work-group) of each column
  // group adds the K splits and stores y (and its amax)
  GemmArgs dn = base_args(nullptr, hq_gs, wd, T, K, I);
  dn.a_codes = hq_codes;
  dn.a_scales = hq_scales;
  dn.c = y;
  dn.ldc = ldy;
  dn.c_bf16 = y_bf16;
  dn.splits = d.dn.splits;
  dn.split_out = part;
  dn.force_split = 1;
  dn.tickets = tickets;
  dn.amax_slots = y_amax;
  dn.m_tiles = d.dn.m_tiles;
  dn.n_tiles = d.dn.n_tiles;
  dn.chunks_per_split = d.dn.chunks_per_split;
  if (d.dn.gv_bpl > 0) launch_gemv<false, EPI_STORE>(dn, d.dn.gv_bpl, st);
  else launch_tile<false, EPI_STORE>(dn, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // namespace nvfp4
