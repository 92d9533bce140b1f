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

void count_launch();

// ---- quantisation -----------------------------------------------------------
size_t quantize_ws_bytes(int64_t rows, int64_t cols, int gs_mode);
int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                    uint8_t* scales, float* gs, int gs_mode, void* ws, hipStream_t st);
// Requantise a float32 [rows][cols] matrix whose amax is the max of
// `partials` (written by an earlier kernel on the same stream).
int requant_f32_launch(const float* h, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                       float* gs, const float* partials, uint32_t npart, hipStream_t st);

// ---- contractions -----------------------------------------------------------
struct Operand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
};

// C[M][N] = A . B^T * gs_a * gs_b, float32 (c_bf16 = 0) or bf16 output.
int gemm_launch(Operand a, Operand b, int64_t M, int64_t N, int64_t K, void* c, int c_bf16, int64_t ldc,
                hipStream_t st);

// H[M][N] = SiLU(A . G^T * gs_a*gs_g) * (A . U^T * gs_a*gs_u) into h (float32,
// row-major, ld N) with one partial |H| max per work-group in `partials`;
// returns the number of partials through *npart.
size_t glu_partials_needed(int64_t M, int64_t N);
int gemm_glu_launch(Operand a, Operand g, Operand u, int64_t M, int64_t N, int64_t K, float* h,
                    float* partials, uint32_t* npart, hipStream_t st);

// Grouped (expert) variants; slot s reads row a_rows[s] (or s), slots
// [off[e], off[e+1]) use expert e's weights (stride N*K per expert).
size_t grouped_glu_partials_needed(int64_t M, int64_t N, int E);
int grouped_gemm_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand w,
                        int64_t N, int64_t K, void* c, int c_bf16, int64_t ldc, hipStream_t st);
int grouped_glu_launch(Operand a, const int32_t* a_rows, const int32_t* off, int E, int64_t M, Operand g,
                       Operand u, int64_t N, int64_t K, float* h, float* partials, uint32_t* npart,
                       hipStream_t st);

}  // namespace nvfp4
