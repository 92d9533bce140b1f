/*
 * nvfp4.h -- C ABI of libnvfp4.so: the batched T-token NVFP4 W4A4 MLP on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for the operations (web pages, cited by title and section):
 *  [vllm]  vllm.cpp issue "tp>1 prefill is host-bound: per-token fp4 GEMM +
 *          per-layer H2D activation staging" -- sections "Problem" and
 *          "Fix directions" (1: one launch set per batch with a grid that
 *          scales with T; 2: activations stay on the device across fp4
 *          layers; 3: activation packing done on the device).
 *  [llama] llama.cpp discussion "CUDA: NVFP4 prefill on Blackwell leaves
 *          ~1.45x performance on the table" -- section "What the patch does"
 *          (gate and up share one quantised activation; the GLU output is
 *          quantised straight into the next GEMM's activation format;
 *          aligned, pipelined tile loads) and "Verified" (MUL_MAT,
 *          MUL_MAT_ID).
 *  [dsv4]  nvfp4-megamoe-kernel "PERFORMANCE -- verified hot-path audit and
 *          prioritized fixes" -- section P0 (activation global scale
 *          amax / (6*448), amax clamped at 1e-8, kept on the device instead
 *          of being read back with .item()) and P8 item 5 (MoE runner with
 *          pre-allocated buffers, no host syncs, no dynamic shapes).
 *
 * NVFP4 layout (all calls).  A matrix [rows][cols] is
 *   codes  : rows * cols/2 bytes, row-major, row r at codes + r*cols/2;
 *            byte j of a row holds element 2j in bits 3:0 and element 2j+1
 *            in bits 7:4; each 4-bit code is E2M1 (sign, 2 exponent bits,
 *            1 mantissa bit; magnitudes 0 0.5 1 1.5 2 3 4 6);
 *   scales : rows * cols/16 bytes, row-major; byte b of a row is the E4M3
 *            (OCP "FN", max 448) scale of elements [16b, 16b+16);
 *   gscale : one float32 global scale (one per expert for expert stacks),
 *            device-resident; value = code * scale * gscale.
 *
 * Conventions (all calls).
 *  - Every pointer is a device pointer unless its comment says host.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  The library never synchronises, never copies between host
 *    and device, never allocates, and never reads device memory on the
 *    host: global scales are produced and consumed on the device only.
 *  - The caller owns every buffer.  The library keeps no pointer after a
 *    call returns; its only state is a process-wide launch counter, a
 *    per-device record of the device check, and the optional timing window
 *    (nvfp4_timing_begin / nvfp4_timing_end).
 *  - Workspace: ws == NULL with ws_bytes != NULL is a size query: the
 *    required size is stored in *ws_bytes and NVFP4_OK returned without
 *    launching anything.  Otherwise *ws_bytes is the size of ws (ws_bytes ==
 *    NULL means no workspace, size 0) and must be at least the required
 *    size.  The workspace needs no initialisation; its contents after a call
 *    are documented per call.
 *  - Errors are returned before any work is enqueued, from host-side
 *    validation: NULL pointers, shapes, alignment, workspace size, unknown
 *    enum values; NVFP4_ERR_DEVICE when no gfx950 device is current.
 *    NVFP4_ERR_LAUNCH reports a failed kernel launch.  Faults inside a
 *    kernel (for instance an out-of-range row index in a_rows, or buffers
 *    shorter than the stated shapes) are undefined behaviour.
 *  - Inputs must be finite; NaN or Inf inputs give unspecified outputs.
 *  - A zero-row call (T == 0, rows == 0, M == 0) is a successful no-op and
 *    writes nothing, not even a global scale.
 *  - Alignment: codes and scales base pointers 16-byte aligned, gscale
 *    4-byte aligned, float/bf16 inputs and outputs 16-byte aligned with row
 *    strides that keep every row 16-byte aligned.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; exactly these declarations are exported. */
#pragma GCC visibility push(default)

typedef struct nvfp4_tensor {
  uint8_t *codes;   /* packed E2M1 codes, see the layout above          */
  uint8_t *scales;  /* E4M3 block scales, one per 16 elements of a row  */
  float   *gscale;  /* device float32 global scale(s)                   */
  const uint8_t *tiled;  /* optional (NULL): the tile-contiguous copy of
                      a weight written by nvfp4_tile_weight, 256-byte
                      aligned; read only for weight operands          */
} nvfp4_tensor;

enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,       /* a required pointer is NULL                       */
  NVFP4_ERR_SHAPE = 2,      /* negative size, or a size not a required multiple */
  NVFP4_ERR_ALIGN = 3,      /* pointer or row stride misaligned                 */
  NVFP4_ERR_WORKSPACE = 4,  /* workspace smaller than required                  */
  NVFP4_ERR_ARG = 5,        /* unknown enum value or inconsistent argument      */
  NVFP4_ERR_DEVICE = 6,     /* no usable gfx950 device is current               */
  NVFP4_ERR_LAUNCH = 7      /* a kernel launch failed                           */
};

enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1 };

enum nvfp4_gs_mode {
  NVFP4_GS_COMPUTE = 0,   /* amax over the whole input on the device; writes *gscale        */
  NVFP4_GS_GIVEN = 1,     /* use the float32 already stored at *gscale                     */
  NVFP4_GS_FROM_AMAX = 2  /* the amax is given on the device (ws); writes *gscale from it   */
};

/* Output-amax epilogues write this many float32 partial maxima (4 KiB); the
 * largest of them is max |output|. */
#define NVFP4_AMAX_SLOTS 1024

enum nvfp4_epilogue {
  NVFP4_EPI_STORE = 0,             /* out = A~ . W~^T scaled, float32 or bf16         */
  NVFP4_EPI_SILU_MUL_REQUANT = 1,  /* out_q = NVFP4(SiLU(A~ . Wg~^T) * (A~ . Wu~^T))  */
  NVFP4_EPI_SILU_MUL_QUANT_GIVEN = 2 /* the same with the static global scale already
                                        stored at *out_q.gscale (read on the device) */
};

/*
 * nvfp4_quantize_act -- NVFP4-quantise x [rows][cols] on the device.
 * [dsv4] P0: gscale = RN32(max(max|x|, 1e-8) / (6*448)), computed on the
 * device over the whole tensor of this call and written to *out.gscale
 * (NVFP4_GS_COMPUTE), or read from *out.gscale (NVFP4_GS_GIVEN).  Then per
 * 16-element block: scale = E4M3 round-to-nearest-even of blockmax / (6 *
 * gscale), saturating at 448; codes = E2M1 round-to-nearest-even of x /
 * (scale * gscale), saturating at 6, sign bit = sign bit of x, magnitude 0
 * in a block whose scale is 0.  All rounding decisions are exact (ties to
 * even).  [vllm] Fix directions 3 (packing on the device); the same call
 * quantises weights (rows = output features) in a cold setup step.
 *   x       : float32 (x_dtype NVFP4_F32) or bf16 (NVFP4_BF16), row stride
 *             ld_x elements (ld_x >= cols)
 *   cols    : multiple of 16
 *   ws      : NVFP4_GS_COMPUTE needs a small workspace (block partial
 *             maxima, 16 KiB); NVFP4_GS_GIVEN needs none;
 *             NVFP4_GS_FROM_AMAX: ws points to NVFP4_AMAX_SLOTS float32
 *             whose largest is max|x| over the whole tensor (written on the
 *             device by an earlier call on the stream: the y_amax output of
 *             the nvfp4_mlp_down whose output is x), *ws_bytes >= 4096,
 *             16-byte aligned; gscale is formed from it exactly as COMPUTE
 *             would (the max is exact)
 * Two kernel launches (COMPUTE) or one (GIVEN, FROM_AMAX); a COMPUTE call on
 * at most 8192 blocks of 16 (rows * cols <= 131072, e.g. decode activations)
 * takes the amax, the global scale and the codes in one launch.  One launch
 * set per call, never one per row.
 */
int nvfp4_quantize_act(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                       nvfp4_tensor out, int gs_mode, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_quantize_act_noalloc -- nvfp4_quantize_act without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results, launches and errors as nvfp4_quantize_act, minus ws / ws_bytes
 * (so gs_mode is NVFP4_GS_COMPUTE or NVFP4_GS_GIVEN; NVFP4_GS_FROM_AMAX,
 * whose amax travels in ws, is NVFP4_ERR_ARG here): the
 * partial maxima of the amax pass go to a scratch array of 16 KiB (4096
 * float32) that the library holds in device memory, one copy per GPU, for the
 * life of the process.  The call allocates nothing.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads without ordering) race on it and give
 * unspecified results; calls ordered on one stream are safe.  The array needs
 * no initialisation (the amax pass writes every entry the quantise pass
 * reads).  Tensors of every size nvfp4_quantize_act accepts fit the array;
 * NVFP4_ERR_WORKSPACE would report one that did not.  NVFP4_ERR_DEVICE also
 * reports a failed lookup of the array's device address.
 */
int nvfp4_quantize_act_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               nvfp4_tensor out, int gs_mode, void *stream);

/*
 * nvfp4_rmsnorm_quantize_act -- NVFP4 quantisation of RMSNorm(x), fused:
 * y[r][c] = (x[r][c] * rinv[r]) * gamma[c] with rinv[r] = 1 / sqrt(mean over
 * the row of x^2 + eps), formed in float32 and never written; then exactly as
 * nvfp4_quantize_act (NVFP4_GS_COMPUTE) applied to y.  [dsv4] P8 item 2 (fold
 * the RMSNorm into the next NVFP4 linear's activation quantisation);
 * [llama] "What the patch does" (batched-row rms_norm).
 *   x     : float32 or bf16 (x_dtype) [rows][cols], row stride ld_x
 *   gamma : float32 [cols], device, 16-byte aligned
 *   eps   : finite, >= 0
 *   ws    : required; on return its first rows*4 bytes hold rinv (float32)
 * Two launches (row statistics and max|y|, then quantisation), independent
 * of rows.
 */
int nvfp4_rmsnorm_quantize_act(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               const float *gamma, float eps, nvfp4_tensor out, void *ws, size_t *ws_bytes,
                               void *stream);

/*
 * nvfp4_gemm -- C[M][N] = (A~ . B~^T) * gscale_a * gscale_b.
 * One NVFP4 x NVFP4 contraction, K-contiguous operands as a linear layer
 * stores them ([llama] "Verified", MUL_MAT).  One launch set per
 * call whatever M is ([vllm] Fix directions 1): expansion of a~ to f16
 * (exact), the contraction, and a fixed-order split-K reduction (over zero
 * rows when K is not split); with M <= 2 and K >= 1024, or 3 <= M <= 16 and
 * K a multiple of 256, the contraction is a weight stream that expands a~
 * itself, so two launches.
 * Accumulation in float32 (matrix cores, or dot products of exact f16
 * products on the one/two-token stream); every product is exact.
 *   a  : [M][K] NVFP4, b : [N][K] NVFP4 (one gscale each)
 *   K  : multiple of 128
 *   c  : float32 or bf16 (c_dtype), row stride ldc >= N elements
 *   c_amax : NULL, or NVFP4_AMAX_SLOTS device float32 (16-byte aligned)
 *        that receive partial maxima of |c| as stored (after the bf16
 *        rounding for bf16 outputs): the largest of them is max |c|, the
 *        amax the next NVFP4 linear's activation global scale needs ([dsv4]
 *        P0), produced in the output epilogue so that no pass re-reads c for
 *        it; pass the array to nvfp4_quantize_act as ws with
 *        NVFP4_GS_FROM_AMAX.  Every slot is written (no initialisation, no
 *        atomics).  With c_amax the reduction launch stores every output
 *        (the contraction writes partial sums even when K is not split); the
 *        launch count is unchanged.
 *   ws : required: the f16 copy of a~ (M*K*2 bytes) and the float32
 *        partial sums; contents unspecified on return
 */
int nvfp4_gemm(nvfp4_tensor a, nvfp4_tensor b, int64_t M, int64_t N, int64_t K,
               void *c, int c_dtype, int64_t ldc, float *c_amax, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_mlp_gu_act -- gate/up projections, SiLU(gate) * up, requantisation.
 * [llama] "What the patch does": gate and up read one shared quantised
 * activation x~; the GLU output H = SiLU(x~ . Wg~^T) * (x~ . Wu~^T)
 * (SiLU(g) = g / (1 + e^-g), float32) is quantised directly into the down
 * projection's NVFP4 input h_out, with a global scale computed on the device
 * over the whole [T][I] tensor of this call and written to *h_out.gscale.
 *   x      : [T][K] NVFP4;  w_gate, w_up : [I][K] NVFP4
 *   h_out  : [T][I] NVFP4 (codes, scales, gscale written)
 *   K, I   : multiples of 128
 *   ws     : required; on return its first T*I*4 bytes hold H in float32,
 *            row-major [T][I] (the value that was quantised); then room for
 *            the f16 copy of x~ (written on the matrix-core paths, unused by
 *            the weight streams) and the partial maxima of |H|
 * Three launches per call (expansion, contraction with the SiLU*up epilogue
 * and the |H| tile maxima, requantisation); two on the weight streams, which
 * expand x~ themselves (T <= 2 with 1024 <= K <= 5120, or 3 <= T <= 16 with
 * K a multiple of 256), except that at 3 <= T <= 16 a K above 2048 is split and
 * one launch clears the column tiles' arrival tickets first (three).  One
 * launch set per batch: the count never grows with T within a range.
 */
int nvfp4_mlp_gu_act(nvfp4_tensor x, nvfp4_tensor w_gate, nvfp4_tensor w_up,
                     int64_t T, int64_t K, int64_t I, nvfp4_tensor h_out,
                     void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_mlp_down -- Y[T][K] = (H~ . Wd~^T) * gscale_h * gscale_wd.
 * The down projection of the MLP ([vllm] "Problem": MlpDownFp4, here once
 * per batch).  y is float32 (parity) or bf16 (the next layer's activation,
 * kept on the device: [vllm] Fix directions 2).
 *   h  : [T][I] NVFP4;  w_down : [K][I] NVFP4;  I multiple of 128
 *   y  : row stride ldy >= K elements
 *   y_amax : NULL, or NVFP4_AMAX_SLOTS device float32 receiving partial
 *        maxima of |y| as stored, as c_amax of nvfp4_gemm: a chained layer's
 *        input amax, so the next nvfp4_quantize_act (NVFP4_GS_FROM_AMAX) is
 *        one launch
 *   ws : required, as for nvfp4_gemm (f16 copy of h~, split-K partials)
 * Three launches per call (two on the weight streams: T <= 2 with I >= 1024,
 * or 3 <= T <= 16 with I a multiple of 256, as for nvfp4_gemm).
 */
int nvfp4_mlp_down(nvfp4_tensor h, nvfp4_tensor w_down, int64_t T, int64_t I, int64_t K,
                   void *y, int y_dtype, int64_t ldy, float *y_amax, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_mlp -- one whole MLP call: y = down(requant(SiLU(x~ . Wg~^T) *
 * (x~ . Wu~^T))) with x~ = NVFP4(x), i.e. nvfp4_quantize_act (computed
 * global scale) + nvfp4_mlp_gu_act + nvfp4_mlp_down in one call, the MLP
 * shard run over T tokens of [vllm] "Problem" done as one launch set per
 * batch ([vllm] Fix directions 1).  x~ and H~ (codes, scales, global scales)
 * are written to x_q and h_q as the separate calls write them, and y is
 * bit-identical to theirs.
 *   x      : float32 or bf16 (x_dtype) [T][K], row stride ld_x >= K
 *   x_amax : NULL (gs_x from max|x| on the device), or the NVFP4_AMAX_SLOTS
 *            partial maxima of |x| an earlier call wrote (the previous
 *            layer's y_amax): gs_x is formed from them, no amax pass
 *   w_gate, w_up : [I][K] NVFP4;  w_down : [K][I] NVFP4;  K, I multiples of 128
 *   x_q    : [T][K] NVFP4 out;  h_q : [T][I] NVFP4 out
 *   y      : float32 or bf16 (y_dtype) [T][K], row stride ldy >= K
 *   y_amax : NULL, or NVFP4_AMAX_SLOTS float32 receiving partial maxima of
 *            |y| as stored (every slot written), for the next layer's x_amax;
 *            not the same buffer as x_amax (NVFP4_ERR_ARG): chained layers
 *            alternate two buffers
 *   ws     : required (size query as usual); contents unspecified on return
 * Decode batches -- T <= 16 with both projections on the weight streams (T
 * <= 2 with 1024 <= K <= 5120 and I >= 1024, or 3 <= T <= 16 with K and I
 * multiples of 256; T * K <= 131072) -- take four launches: (1) quantise x
 * (one to eight work-groups, each reducing the amax itself), which also clears
 * the per-column-group arrival tickets and the y_amax slots; (2) the gate/up
 * weight stream with the SiLU*up epilogue, float32 H and its partial maxima;
 * (3) requantisation of H; (4) the down weight stream.  In each stream whose
 * K is split, the splits store their partial sums with device-coherent
 * stores and, once those are acknowledged, take a ticket of their column
 * group; the arrival that completes the group adds the partial sums in split
 * order and runs the epilogue -- nothing waits for anything, and no
 * reduction launch follows.  Other shapes run the separate calls' kernels
 * minus their two expansion launches -- the quantisers of x and H also write
 * the f16 operand copies the matrix-core contractions read -- so six launches
 * (quantise 2, gate/up contraction, requantisation, down contraction, split-K
 * reduction), five with x_amax or an x of at most 8192 blocks of 16.
 */
int nvfp4_mlp(const void *x, int x_dtype, int64_t ld_x, const float *x_amax, int64_t T, int64_t K, int64_t I,
              nvfp4_tensor w_gate, nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q,
              void *y, int y_dtype, int64_t ldy, float *y_amax, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_mlp_gu_act_static -- nvfp4_mlp_gu_act with a static global scale
 * for H~.  [dsv4] P0, fix 1: the activation global scales are measured once
 * by a warm-up pass (for instance the scale nvfp4_mlp_gu_act wrote to its
 * h_out.gscale) and kept on the device; [dsv4] P8, item 1: with the scale
 * known in advance the producer quantises its own output.  *h_out.gscale is
 * READ on the device (never written); the GLU output is quantised in the
 * contraction's epilogue (values above 6 * 448 * gscale saturate to block
 * scale 448 and codes +-6), so no float32 H is written and no amax or
 * requantisation pass runs.
 *   x, w_gate, w_up, K, I : as nvfp4_mlp_gu_act
 *   h_out : [T][I] NVFP4; codes and scales written, gscale read
 *   ws    : required (the f16 copy of x~)
 * Two launches per call (expansion, contraction); one on the weight streams
 * (as nvfp4_mlp_gu_act), where a split K at 3 <= T <= 16 instead takes the
 * ticket-clearing launch (two).
 */
int nvfp4_mlp_gu_act_static(nvfp4_tensor x, nvfp4_tensor w_gate, nvfp4_tensor w_up,
                            int64_t T, int64_t K, int64_t I, nvfp4_tensor h_out,
                            void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_mlp_down_quant -- the down projection emitting NVFP4 directly:
 * y_out = NVFP4(Y) with Y = (H~ . Wd~^T) * gscale_h * gscale_wd in float32
 * (the values nvfp4_mlp_down stores as float32) and the global scale
 * *y_out.gscale READ on the device -- the next layer's static input scale
 * ([dsv4] P8, item 1: no wide-precision output for the consumer to
 * re-quantise; P0, fix 1: scale from a warm-up pass).
 *   h : [T][I] NVFP4;  w_down : [K][I] NVFP4;  I multiple of 128,
 *   K multiple of 16;  y_out : [T][K] NVFP4 (codes, scales written)
 *   ws : required, as nvfp4_mlp_down
 * Three launches per call (expansion, contraction, quantising split
 * reduction); two on the weight streams (as nvfp4_mlp_down).
 */
int nvfp4_mlp_down_quant(nvfp4_tensor h, nvfp4_tensor w_down, int64_t T, int64_t I, int64_t K,
                         nvfp4_tensor y_out, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_moe_mlp -- the expert MLP over routed slots in one call ([llama]
 * "Verified", MUL_MAT_ID; [dsv4] P8 item 5): x~ = NVFP4(x) with its global
 * scale computed on the device; for every slot s of expert e (slots
 * [group_offsets[e], group_offsets[e+1])) the gate/up pair of expert e on
 * token row a_rows[s], SiLU(gate) * up requantised into h_q with one global
 * scale over all M slots, and the down projection of expert e into row s of
 * y_slots, scaled by gscale_h * w_down.gscale[e].  The values are those of
 * nvfp4_quantize_act, then nvfp4_grouped_gemm with NVFP4_EPI_SILU_MUL_REQUANT
 * and with NVFP4_EPI_STORE (bit-identical); the quantiser and the
 * requantisation also write the f16 operand copies the contractions stage
 * (the gate/up gathers its slots' rows from the token copy), so no launch
 * expands or gathers an operand: six launches in all (five when x has at
 * most 8192 blocks of 16: one quantiser launch).
 *   x             : [T][K] float32 or bf16 (x_dtype), row stride ld_x
 *   a_rows        : [M] token row of each slot (values < T); group_offsets
 *                   [E+1] as nvfp4_grouped_gemm (group_offsets[E] == M)
 *   w_gate, w_up  : [E][I][K] expert stacks;  w_down : [E][K][I]
 *   K, I          : multiples of 128;  T * K * 2 < 2^31
 *   x_q           : [T][K] NVFP4 (codes, scales, gscale written)
 *   h_q           : [M][I] NVFP4 (codes, scales, gscale written)
 *   y_slots       : [M][K] float32 or bf16 (y_dtype), row stride ld_y
 *   ws            : required (size query with ws == NULL)
 * T == 0 or M == 0: a no-op.  Routing (nvfp4_moe_route) and the weighted
 * combine (nvfp4_moe_combine) are their own calls.
 */
int nvfp4_moe_mlp(const void *x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                  const int32_t *a_rows, const int32_t *group_offsets, int64_t M, nvfp4_tensor w_gate,
                  nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q, void *y_slots,
                  int y_dtype, int64_t ld_y, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_moe_mlp_static -- the expert MLP over routed slots in one call with
 * static global scales ([dsv4] P0, fix 1: scales from a warm-up pass; P8
 * item 1: the GLU output quantised in the producer's epilogue): as
 * nvfp4_moe_mlp, but *x_q.gscale and *h_q.gscale are READ on the device (the
 * scales x~ and H~ are quantised with) instead of computed, and the gate/up
 * pair quantises SiLU(gate) * up in its epilogue (no float32 H, no
 * requantisation launch).  The values are those of nvfp4_quantize_act with
 * NVFP4_GS_GIVEN, then nvfp4_grouped_gemm with NVFP4_EPI_SILU_MUL_QUANT_GIVEN
 * and with NVFP4_EPI_STORE (bit-identical); the quantiser writes the f16 copy
 * of x that the gate/up stages its slots' rows from, and the gate/up's
 * epilogue writes the f16 copy of H~ that the down projection stages: four
 * launches, none of them an expansion.  Arguments and limits as
 * nvfp4_moe_mlp; x_q and h_q: codes and scales written, gscale read.
 */
int nvfp4_moe_mlp_static(const void *x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                         const int32_t *a_rows, const int32_t *group_offsets, int64_t M, nvfp4_tensor w_gate,
                         nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q, void *y_slots,
                         int y_dtype, int64_t ld_y, void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_tile_weight -- the tile-contiguous copy of a weight (or expert
 * stack) for the large-batch contractions ([llama] "What the patch does":
 * aligned whole-tile loads feeding the matrix unit).  A permutation of the
 * weight's codes and scales, no value changes: every contraction call gives
 * bit-identical results with and without it.  Written once per weight (like
 * the weight's quantisation), then passed as w.tiled to the calls; the
 * large-batch contractions (more than 32 tokens, and the expert-grouped
 * GEMMs) stage the weight from it, each chunk of a column tile a run of
 * whole 1 KiB pieces instead of 64 bytes of every row.  The decode weight
 * streams read the row-major codes and scales as before.
 *   w        : [experts][N][K] NVFP4 (codes, scales; gscale not read)
 *   experts  : 1 for a single weight, E for an expert stack
 *   K        : multiple of 128;  N >= 0;  one expert's copy below 2 GiB
 *              (ceil(N/128) * (K/128) * 9216 < 2^31)
 *   tiled    : output, tiled_bytes = experts * ceil(N/128) * (K/128) * 9216
 *              bytes, 256-byte aligned (tiled == NULL: size query).  Block
 *              (e, g, c) -- rows 128g .. 128g+127 of expert e, K elements
 *              128c .. 128c+127 -- starts at byte ((e*G + g)*(K/128) + c) *
 *              9216, G = ceil(N/128): 8192 bytes of codes, the 16-byte unit
 *              u (0..3) of local row r at unit r*4 + (u ^ ((r/4) % 4)), then
 *              local row r's 8 scale bytes at 8192 + 8r.  Rows past N are 0.
 * One launch.  The copy must be rewritten when the weight changes; a call
 * reads it only when its weight operand's tiled pointer is not NULL (with the
 * gate/up pair, both).
 */
int nvfp4_tile_weight(nvfp4_tensor w, int64_t experts, int64_t N, int64_t K, uint8_t *tiled, size_t *tiled_bytes,
                      void *stream);

/*
 * nvfp4_grouped_gemm -- expert-grouped NVFP4 GEMM in one launch per GEMM
 * ([llama] "Verified", MUL_MAT_ID; [dsv4] P8 item 5: no host syncs, no
 * dynamic shapes).  Slot s (0 <= s < M) reads activation row a_rows[s] of a
 * (row s when a_rows is NULL); slots [group_offsets[e], group_offsets[e+1])
 * belong to expert e.  a_rows and group_offsets stay on the device; the host
 * only knows the static slot count M, and group_offsets[E] must equal M.
 *   a             : [rows_a][K] NVFP4 (rows_a is implied by a_rows)
 *   w0            : [E][N][K] NVFP4 expert stack, gscale[E] (gate weights in
 *                   the GLU epilogue)
 *   w1            : [E][N][K] up weights (GLU epilogue only; else ignored)
 *   epilogue      : NVFP4_EPI_STORE -> out [M][N] float32/bf16, row stride
 *                   ld_out, scaled by gscale_a * w0.gscale[e];
 *                   NVFP4_EPI_SILU_MUL_REQUANT -> out_q [M][N] NVFP4 of
 *                   SiLU(gate) * up with one global scale over all M slots
 *                   (written to *out_q.gscale)
 *   K, N          : multiples of 128;  E >= 1
 *                   NVFP4_EPI_SILU_MUL_QUANT_GIVEN -> as the previous, with the
 *                   global scale *out_q.gscale given ([dsv4] P0 fix 1, a warm-up
 *                   scale) and the GLU output quantised in the contraction's
 *                   epilogue: no float32 output, no requantisation launch
 *   ws            : NVFP4_EPI_SILU_MUL_REQUANT: its first M*N*4 bytes hold the
 *                   float32 GLU output [M][N] on return
 */
int nvfp4_grouped_gemm(nvfp4_tensor a, const int32_t *a_rows, const int32_t *group_offsets,
                       int E, int64_t M, nvfp4_tensor w0, nvfp4_tensor w1, int64_t N, int64_t K,
                       int epilogue, void *out, int out_dtype, int64_t ld_out, nvfp4_tensor out_q,
                       void *ws, size_t *ws_bytes, void *stream);

/*
 * nvfp4_moe_route -- top-k routing of T tokens over E experts into the slot
 * layout nvfp4_grouped_gemm takes, on the device (no host read of expert ids:
 * [dsv4] P8 item 5; grouped MUL_MAT_ID slots: [llama] "Verified").  Each
 * token takes the k experts with the largest logits, ties to the lower
 * expert id; its weights are the softmax over those k logits,
 * w_j = exp(l_j - l_max) / sum over the k chosen of exp(l_i - l_max) (float32).
 * Slots are the (token, choice) pairs sorted by (expert, token).
 *   logits        : float32 [T][E], row stride ld >= E elements
 *   E, k          : 1 <= E <= 4096, 1 <= k <= min(E, 16)
 *   group_offsets : int32 [E+1] out: first slot of each expert; [E] = T*k
 *   a_rows        : int32 [T*k] out: token of each slot
 *   slot_of       : int32 [T][k] out: slot of token t's j-th choice (choices
 *                   by decreasing logit)
 *   weights       : float32 [T][k] out: the combine weights, same order
 *   ws            : required (per-token choices and ranks, per-block counts)
 * Three launches, independent of T; the slot order does not depend on
 * scheduling (no atomics).  Logits must be finite.
 */
int nvfp4_moe_route(const float *logits, int64_t T, int E, int k, int64_t ld, int32_t *group_offsets,
                    int32_t *a_rows, int32_t *slot_of, float *weights, void *ws, size_t *ws_bytes,
                    void *stream);

/*
 * nvfp4_moe_combine -- y[t][n] = sum over j of weights[t][j] *
 * y_slots[slot_of[t][j]][n]: the weighted sum of each token's expert outputs
 * (float32 accumulation, choices in order j = 0 .. k-1).
 *   y_slots : float32 or bf16 (slots_dtype) [M][N], row stride ld_slots
 *   slot_of, weights : [T][k] as written by nvfp4_moe_route; every slot index
 *             must be a row of y_slots (undefined behaviour otherwise)
 *   y       : float32 or bf16 (y_dtype) [T][N], row stride ldy
 *   N       : multiple of 8; rows of y_slots and y 16-byte aligned
 * One launch.
 */
int nvfp4_moe_combine(const void *y_slots, int slots_dtype, int64_t ld_slots, const int32_t *slot_of,
                      const float *weights, int64_t T, int k, int64_t N, void *y, int y_dtype, int64_t ldy,
                      void *stream);

/* Static message for a status code (host string, never NULL). */
const char *nvfp4_strerror(int status);

/* Number of kernel launches this library has enqueued in this process
 * (a host counter; lets a caller check that the launch count of a call does
 * not depend on T -- [vllm] "Problem": identical per-token launches). */
uint64_t nvfp4_launch_count(void);

/*
 * Kernel timing (instrumentation; nothing is timed unless a window is open).
 * Kernel classes: every launch of the library belongs to exactly one.
 */
enum nvfp4_kernel_class {
  NVFP4_KC_QUANTIZE = 0,     /* amax partials and quantise kernels (also the requantisation of H) */
  NVFP4_KC_EXPAND = 1,       /* NVFP4 -> f16 activation expansion ahead of a contraction          */
  NVFP4_KC_GEMM_GLU = 2,     /* contraction with the SiLU*up epilogue (gate/up projection)         */
  NVFP4_KC_GEMM_STORE = 3,   /* contraction with the store epilogue (down projection, nvfp4_gemm)  */
  NVFP4_KC_REDUCE = 4,       /* split-K reduction and output scaling                               */
  NVFP4_KC_ROUTE = 5,        /* expert routing kernels (nvfp4_moe_route)                           */
  NVFP4_KC_COMBINE = 6       /* weighted combine of expert outputs (nvfp4_moe_combine)             */
};

#define NVFP4_TIMING_MAX_LAUNCHES 1048576

/*
 * nvfp4_timing_begin -- open a timing window for one kernel class.  Until
 * nvfp4_timing_end, every launch of that class (on any stream, from any
 * thread) is bracketed by two HIP events recorded on the launch's own
 * stream, so the measured span is that kernel alone.  Creates
 * 2 * max_launches HIP events (host-side objects, no device memory);
 * launches beyond max_launches are counted as dropped and not timed.
 * Errors: NVFP4_ERR_ARG for an unknown class, max_launches outside
 * [1, NVFP4_TIMING_MAX_LAUNCHES] or a window already open;
 * NVFP4_ERR_LAUNCH when the events cannot be created.
 */
int nvfp4_timing_begin(int kernel_class, int64_t max_launches);

/*
 * nvfp4_timing_end -- close the window: waits on the host for the last
 * recorded event (the one call of the library that synchronises), then
 * writes to host memory the number of launches timed, the number dropped and
 * the sum of their durations in milliseconds, and destroys the events.
 * Errors: NVFP4_ERR_NULL for a NULL output; NVFP4_ERR_ARG when no window is
 * open; NVFP4_ERR_LAUNCH when an event record or query failed (the window is
 * closed either way).
 */
int nvfp4_timing_end(int64_t *launches, int64_t *dropped, double *total_ms);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
