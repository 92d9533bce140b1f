// Host-side launchers behind the C ABI (nvfp4_abi.hip).  Every launcher
// assumes its arguments were validated by the ABI layer and only enqueues
// kernels; it returns 0 or 7 (NVFP4_ERR_LAUNCH).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Largest number of partial maxima any amax reduction produces.
constexpr uint32_t kMaxPartials = 4096;
// Partial maxima of an output-amax epilogue (NVFP4_AMAX_SLOTS in the header).
constexpr uint32_t kAmaxSlots = 1024;

// Kernel classes of the timing window (same values as the public enum).
enum KernelClass {
  KC_QUANTIZE = 0, KC_EXPAND = 1, KC_GEMM_GLU = 2, KC_GEMM_STORE = 3, KC_REDUCE = 4, KC_ROUTE = 5, KC_COMBINE = 6,
  KC_COUNT = 7
};

// Limits of the expert routing.
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 4096;

// Every launch is bracketed by these two calls: launch_begin records the
// start event when a timing window for `kc` is open (returns its slot, else
// -1); launch_end records the matching end event and counts the launch.
int launch_begin(int kc, hipStream_t st);
void launch_end(int slot, hipStream_t st);

// ---- quantisation -----------------------------------------------------------
size_t quantize_ws_bytes(int64_t rows, int64_t cols, int gs_mode);
// x16 (nullable): also write the dequantised values code * scale as f16
// [rows][cols] (the operand copy a matrix-core contraction reads).
int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                    uint8_t* scales, float* gs, int gs_mode, void* ws, hipStream_t st, _Float16* x16 = nullptr);
// Allocation-free quantiser: bytes of the per-device scratch array, and its
// device address on the current device (0, or 6 when it cannot be looked up).
size_t quantize_scratch_bytes();
int quantize_scratch(void** out);
// Requantise a float32 [rows][cols] matrix whose amax is the max of
// `partials` (written by an earlier kernel on the same stream).
int requant_f32_launch(const float* h, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                       float* gs, const float* partials, uint32_t npart, hipStream_t st, _Float16* h16 = nullptr);

// First launch of the whole-MLP decode path: quantise x (at most 8192 blocks
// of 16) in one launch, with the amax reduced from x or taken from the
// kAmaxSlots partial maxima `x_amax` (nullable), and clear the words
// [zero, zero + nzero) and [zero2, zero2 + nzero2) for the launches that follow.
constexpr uint32_t kSmallQuantBlocks = 8192;
int mlp_prologue_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                        uint8_t* scales, float* gs, const float* x_amax, uint32_t* zero, uint32_t nzero,
                        uint32_t* zero2, uint32_t nzero2, hipStream_t st);

// RMSNorm fused into the quantiser: workspace = inverse rms per row, then the
// partial maxima.
size_t rmsnorm_quantize_ws_bytes(int64_t rows);
int rmsnorm_quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, const float* gamma,
                            float eps, uint8_t* codes, uint8_t* scales, float* gs, void* ws, hipStream_t st);

// ---- contractions -----------------------------------------------------------
struct Operand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  const uint8_t* tiled;   // optional tile-contiguous copy of a weight (tile_weight_launch), else nullptr
};

// Tile-contiguous copy of a weight [experts][N][K] for the large-batch
// contractions: blocks of 128 rows x 128 K (kTileBlock bytes: the 8 KiB of
// codes in the order the contraction stages them in LDS, then the 1 KiB of
// scales), block (e, g, c) at ((e * G + g) * K/128 + c) * kTileBlock with
// G = ceil(N / 128); rows past N are zero.
constexpr int64_t kTileRows = 128, kTileK = 128, kTileBlock = 9216;
size_t tile_weight_bytes(int64_t E, int64_t N, int64_t K);
int tile_weight_launch(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N, int64_t K, uint8_t* out,
                       hipStream_t st);

// Store-epilogue contraction C[M][N] = A . W^T * gs_a * gs_w (float32 or bf16),
// dense (off == nullptr) or expert-grouped (slot s reads activation row
// rows[s] or s; slots [off[e], off[e+1]) use expert e's weights, stride N*K).
// c_amax (nullable): kAmaxSlots float32 partial maxima of |C| as stored.
// Workspace: f16-expanded activations, then split-K partial sums.
size_t store_ws_bytes(int64_t M, int64_t N, int64_t K, int E, bool grouped);
// a16 (nullable): the f16 copy of the (dense) activation, already written by
// the quantiser -- no expansion launch.
int store_launch(Operand a, const int32_t* rows, const int32_t* off, int E, int64_t M, Operand w, int64_t N,
                 int64_t K, void* c, int c_bf16, int64_t ldc, float* c_amax, void* ws, hipStream_t st,
                 const _Float16* a16 = nullptr);

// H = SiLU(A . G^T * gs_a*gs_g) * (A . U^T * gs_a*gs_u) (float32, row-major
// [M][N], at the start of the workspace), then its NVFP4 requantisation with a
// global scale over all M rows.  Dense or grouped as above.  On the 3-16 token
// stream with K split, the workspace also holds the split partial sums and the
// column tiles' tickets, cleared by a launch of their own before the
// contraction.
size_t glu_ws_bytes(int64_t M, int64_t N, int64_t K, int E, bool grouped, bool gather = false);
// a16 (nullable): as for store_launch -- except expert-grouped, where it is
// the f16 copy of the whole activation [gather_rows][K] and slot s stages row
// a_rows[s] of it (no expansion launch, no f16 slot in the workspace:
// glu_ws_bytes(..., gather = true)); hq16 (nullable): the requantisation also
// writes the f16 copy of H~ there (for the down projection).
int glu_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt, Operand up,
               int64_t N, int64_t K, uint8_t* hq_codes, uint8_t* hq_scales, float* hq_gs, void* ws,
               hipStream_t st, const _Float16* a16 = nullptr, _Float16* hq16 = nullptr, int64_t gather_rows = 0);

// The same GLU output (dense, or expert-grouped when `off` is given)
// quantised in the contraction's epilogue with the given global scale *hq_gs
// (two launches: expansion or ticket clearing, contraction).  Workspace: the
// f16 copy of A, then (3-16 token stream, K split) partial sums and tickets.
// With a16 given (expert groups: the token copy, a_rows the slots' token rows,
// gather_rows its rows) no expansion runs and the workspace holds no f16 copy
// of A; hq16 (expert groups, nullable) receives the f16 copy of H~.
size_t glu_static_ws_bytes(int64_t M, int64_t N, int64_t K, bool grouped, bool gather = false);
int glu_static_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand gt,
                      Operand up, int64_t N, int64_t K, uint8_t* hq_codes, uint8_t* hq_scales, const float* hq_gs,
                      void* ws, hipStream_t st, const _Float16* a16 = nullptr, _Float16* hq16 = nullptr,
                      int64_t gather_rows = 0);

// C = A . W^T * gs_a * gs_w quantised to NVFP4 with the given global scale
// *yq_gs by the (always launched) fixed-order split reduction.  Workspace as
// store_ws_bytes.
int store_quant_launch(Operand a, int64_t M, Operand w, int64_t N, int64_t K, uint8_t* yq_codes, uint8_t* yq_scales,
                       const float* yq_gs, void* ws, hipStream_t st);

// Whole MLP: quantise x, gate/up + SiLU*up + requantisation, down projection.
// For decode batches (T <= 16 with both projections on the weight streams) four
// launches: quantise x (also clearing the split-K tickets), gate/up, requantise
// H, and the down projection; in each contraction whose K is split the wave
// that arrives last on a column group adds the partial sums (no reduction
// launch); otherwise the launch sequence of
// the separate calls.  x_amax (nullable): kAmaxSlots partial maxima of |x|
// (the previous layer's y_amax); y_amax (nullable): the same for y.
size_t mlp_ws_bytes(int64_t T, int64_t K, int64_t I);
int mlp_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, Operand wg, Operand wu,
               Operand wd, uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
               float* hq_gs, void* y, int y_bf16, int64_t ldy, const float* x_amax, float* y_amax, void* ws,
               hipStream_t st);

// Expert MLP over routed slots: quantise x [T][K] (also writing its f16 copy),
// expert-grouped gate/up + SiLU*up staging each slot's row of that copy,
// requantisation over all M slots (also writing the f16 copy of H~), and the
// expert-grouped down projection into y_slots [M][K] -- six launches (five
// with the one-launch quantiser), none of them an expansion.  Workspace: [quantiser partials][x f16][gate/up
// workspace without its f16 slot][down workspace, H~ f16 in its f16 slot].
size_t moe_mlp_ws_bytes(int64_t T, int64_t K, int64_t I, int E, int64_t M);
int moe_mlp_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                   const int32_t* a_rows, const int32_t* off, int64_t M, Operand wg, Operand wu, Operand wd,
                   uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
                   float* hq_gs, void* y, int y_bf16, int64_t ldy, void* ws, hipStream_t st);

// The same with given global scales (x~ with *xq_gs, H~ with *hq_gs): quantise
// x with its scale (also writing its f16 copy), expert-grouped gate/up with
// the quantising epilogue staging each slot's row of that copy (also writing
// the f16 copy of H~), expert-grouped down projection on that copy, split
// reduction -- four launches, none of them an expansion.  Workspace: [x f16]
// [gate/up workspace][down workspace, H~ f16 in its f16 slot].
size_t moe_mlp_static_ws_bytes(int64_t T, int64_t K, int64_t I, int E, int64_t M);
int moe_mlp_static_launch(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                          const int32_t* a_rows, const int32_t* off, int64_t M, Operand wg, Operand wu, Operand wd,
                          uint8_t* xq_codes, uint8_t* xq_scales, float* xq_gs, uint8_t* hq_codes, uint8_t* hq_scales,
                          const float* hq_gs, void* y, int y_bf16, int64_t ldy, void* ws, hipStream_t st);

// ---- expert routing and combine ----------------------------------------------
size_t route_ws_bytes(int64_t T, int E, int k);
int route_launch(const float* logits, int64_t T, int E, int k, int64_t ld, int32_t* group_offsets, int32_t* a_rows,
                 int32_t* slot_of, float* weights, void* ws, hipStream_t st);
int combine_launch(const void* ys, int ys_bf16, int64_t ld_s, const int32_t* slot_of, const float* weights, int64_t T,
                   int k, int64_t N, void* y, int y_bf16, int64_t ldy, hipStream_t st);

}  // namespace nvfp4
