// Expert routing and combine on the device, around the expert-grouped MLP.
//
// The routing runs without a host read of the expert ids, with a fixed number
// of launches and buffers sized up front (nvfp4-megamoe-kernel performance
// audit, P8 item 5), producing the slot layout the grouped contractions take
// (llama.cpp discussion, "Verified": MUL_MAT_ID).  Readings: each token takes
// the k experts with the largest logits (ties to the lower expert id); its
// combine weights are the softmax over those k logits; slots are the
// (token, choice) pairs sorted by (expert, token).
//
// Three launches: route_topk_wave_kernel (route_topk_kernel for more than 128
// experts) gives each token's top-k, its weights, each choice's rank among its
// 64-token block's choices of the same expert and the per-block expert
// counts; route_scan_kernel turns the counts into per-block and per-expert
// offsets (one work-group); route_scatter_kernel places every choice in its
// slot.  No atomics: the slot order is the same on every run.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kRouteWg = 256;      // threads per work-group; one token per thread
constexpr int kRouteBlock = 64;    // tokens per routing block (one wave)
constexpr int kScanThreads = 1024;
constexpr int kTopkBatch = 16;     // logits loaded together per token

__global__ void __launch_bounds__(kRouteWg) route_topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                              int k, int64_t ld, int32_t* __restrict__ ids,
                                                              float* __restrict__ weights, int32_t* __restrict__ rank,
                                                              int32_t* __restrict__ hist) {
  const int64_t t = (int64_t)blockIdx.x * kRouteWg + threadIdx.x;
  const bool valid = t < T;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t blk = t / kRouteBlock;            // routing block of this token (= its wave)
  float val[kMaxTopK];
  int id[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    val[j] = -__builtin_huge_valf();
    id[j] = 0;
  }
  if (valid) {
    const float* row = logits + t * ld;
    for (int e0 = 0; e0 < E; e0 += kTopkBatch) {
      // the batch's logits are loaded together, then inserted in expert order
      float lv[kTopkBatch];
#pragma unroll
      for (int i = 0; i < kTopkBatch; ++i) lv[i] = e0 + i < E ? row[e0 + i] : 0.f;
#pragma unroll
      for (int i = 0; i < kTopkBatch; ++i) {
        if (e0 + i >= E) break;
        // insert into the list sorted by (logit desc, id asc): the new expert
        // goes before the first entry with a strictly smaller logit (equal
        // logits keep the lower, earlier id first); every entry below shifts
        // down by one, the last one falls off
        float cv = lv[i];
        int ci = e0 + i;
        bool ins = false;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j < k) {
            const bool take = ins || cv > val[j];
            const float tv = val[j];
            const int ti = id[j];
            val[j] = take ? cv : tv;
            id[j] = take ? ci : ti;
            cv = take ? tv : cv;
            ci = take ? ti : ci;
            ins = take;
          }
        }
      }
    }
    float z[kMaxTopK];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      z[j] = j < k ? expf(val[j] - val[0]) : 0.f;
      sum += z[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) {
        ids[t * k + j] = id[j];
        weights[t * k + j] = z[j] / sum;
      }
  }
  // Rank of each choice among the block's earlier tokens that chose the same
  // expert, and the block's count per expert (one ballot per expert).
  int rk[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) rk[j] = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool block_valid = t - lane < T;          // the block exists (its first token does)
  for (int e = 0; e < E; ++e) {
    bool chose = false;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) chose |= (j < k) && valid && id[j] == e;
    const uint64_t m = __ballot(chose);
    if (lane == 0 && block_valid) hist[blk * E + e] = __popcll(m);   // zero counts too
    if (m == 0) continue;                          // wave-uniform
    if (chose) {
      const int r = __popcll(m & below);
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k && id[j] == e) rk[j] = r;
    }
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) rank[t * k + j] = rk[j];
  }
}

// The same results with more parallelism, for E <= kWaveTopkMaxE: one
// work-group (8 waves) per 64-token routing block; each token gets 8 lanes
// of a wave, each lane holding PER of its logits (expert 8i + lane%8; PER = 8
// for up to 64 experts, 16 for up to 128).
// k rounds each pick the largest logit not yet chosen, ties to the lower
// expert id (an arg-max within the 8 lanes), which is the order the insertion
// above produces.  The block's choices go through LDS to the rank and count
// pass, whose experts are shared out over the 8 waves.
constexpr int kWaveTopkMaxE = 128;
constexpr int kWaveTopkWaves = 8;
constexpr int kTokLanes = 8;
constexpr int kPerLane = kWaveTopkMaxE / kTokLanes;   // logits per lane: 16 for up to 128 experts, 8 up to 64

__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  // (v, i) = the better of two candidates: the larger logit, ties to the
  // lower id.  "No candidate" is (-inf, INT_MAX), which every candidate
  // (a -inf logit included) beats and which beats none.  Evaluated without
  // short-circuit branches.
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}

template <int PER>
__global__ void __launch_bounds__(kWaveTopkWaves * 64) route_topk_wave_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int64_t ld, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  static_assert(kWaveTopkWaves * (64 / kTokLanes) == kRouteBlock, "one token per 8 lanes of the block");
  __shared__ int32_t sid[kRouteBlock * kMaxTopK];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = lane & (kTokLanes - 1);
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * kRouteBlock;
  const int tb = wv * (64 / kTokLanes) + (lane >> 3);   // token within the block
  const int64_t tt = t0 + tb;
  const bool tvalid = tt < T;
  float v[PER];
  bool free_[PER];
  const float* row = logits + (tvalid ? tt : 0) * ld;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = sub + kTokLanes * i;
    free_[i] = tvalid && e < E;
    v[i] = free_[i] ? row[e] : 0.f;
  }
  float val[kMaxTopK];
  int id[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    val[j] = -__builtin_huge_valf();
    id[j] = 0;
    if (j < k) {                                    // wave-uniform
      float bv = -__builtin_huge_valf();
      int bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        argmax_merge(bv, bi, free_[i] ? v[i] : -__builtin_huge_valf(), free_[i] ? sub + kTokLanes * i : INT_MAX);
#pragma unroll
      for (int off = kTokLanes / 2; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        argmax_merge(bv, bi, ov, oi);
      }
      val[j] = bv;
      id[j] = bi;
#pragma unroll
      for (int i = 0; i < PER; ++i) free_[i] = free_[i] & (sub + kTokLanes * i != bi);
    }
  }
  if (tvalid && sub == 0) {
    float z[kMaxTopK];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      z[j] = j < k ? expf(val[j] - val[0]) : 0.f;
      sum += z[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) {
        ids[tt * k + j] = id[j];
        weights[tt * k + j] = z[j] / sum;
        sid[tb * kMaxTopK + j] = id[j];
      }
  }
  __syncthreads();
  // ranks and counts: lanes are the block's tokens, experts shared out by wave
  const int64_t t = t0 + lane;
  const bool valid = t < T;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int mine[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) mine[j] = (valid && j < k) ? sid[lane * kMaxTopK + j] : -1;
  for (int e = wv; e < E; e += kWaveTopkWaves) {
    bool chose = false;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) chose |= mine[j] == e;
    const uint64_t m = __ballot(chose);
    if (lane == 0) hist[blk * E + e] = __popcll(m);   // zero counts too
    if (chose) {
      const int r = __popcll(m & below);
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (mine[j] == e) rank[t * k + j] = r;
    }
  }
}

// hist[b][e] (counts) -> hist[b][e] = number of expert e's choices in the
// blocks before b (exclusive scan over the blocks, in place);
// group_offsets[e] = first slot of expert e, group_offsets[E] = T*k.  A slot
// is group_offsets[e] + hist[b][e] + the choice's rank in its block.  One
// thread per expert (kMaxExperts / kScanThreads experts each when E is
// larger); the block counts are read kScanBatch at a time so that the loads of
// one expert's column are in flight together.
constexpr int kScanBatch = 16;

__global__ void __launch_bounds__(kScanThreads) route_scan_kernel(int32_t* __restrict__ hist, int64_t nb, int E,
                                                                  int32_t* __restrict__ group_offsets) {
  constexpr int kPer = kMaxExperts / kScanThreads;
  __shared__ int32_t totals[kMaxExperts];
  __shared__ int32_t part[kScanThreads];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = q * kScanThreads + threadIdx.x;
    int32_t run = 0;
    if (e < E) {
      for (int64_t b0 = 0; b0 < nb; b0 += kScanBatch) {
        int32_t h[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) h[i] = b0 + i < nb ? hist[(b0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i)
          if (b0 + i < nb) {
            hist[(b0 + i) * E + e] = run;
            run += h[i];
          }
      }
    }
    totals[e] = run;
  }
  __syncthreads();
  // exclusive scan of the totals in expert order: thread i owns experts
  // kPer*i .. kPer*i+kPer-1
  int32_t mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) mine += totals[threadIdx.x * kPer + q];
  part[threadIdx.x] = mine;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t base = part[threadIdx.x] - mine;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = threadIdx.x * kPer + q;
    if (e < E) group_offsets[e] = base;
    base += totals[e];
  }
  if (threadIdx.x == kScanThreads - 1) group_offsets[E] = part[kScanThreads - 1];
}

__global__ void __launch_bounds__(256) route_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ rank,
                                                            const int32_t* __restrict__ hist,
                                                            const int32_t* __restrict__ group_offsets, int64_t T,
                                                            int E, int k, int32_t* __restrict__ a_rows,
                                                            int32_t* __restrict__ slot_of) {
  const int64_t n = T * k;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / k;
    const int32_t e = ids[i];
    const int32_t s = group_offsets[e] + hist[(t / kRouteBlock) * E + e] + rank[i];
    if (s >= 0 && s < n) a_rows[s] = (int32_t)t;   // always true; keeps the write in bounds regardless
    slot_of[i] = s;
  }
}

// y[t][n] = sum_j weights[t][j] * y_slots[slot_of[t][j]][n], float32
// accumulation with the choices in order; 8 columns per thread.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) combine_kernel(const TI* __restrict__ ys, int64_t ld_s,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ weights, int64_t T, int k, int64_t N,
                                                      TO* __restrict__ y, int64_t ldy) {
  const int64_t n8 = N / 8, total = T * n8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / n8, c = (i - t * n8) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int64_t s = slot_of[t * k + j];
      const float w = weights[t * k + j];
      float v[8];
      if constexpr (sizeof(TI) == 2) {
        const uint4 q = *reinterpret_cast<const uint4*>(ys + s * ld_s + c);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[2 * h] = __uint_as_float(u[h] << 16);
          v[2 * h + 1] = __uint_as_float(u[h] & 0xFFFF0000u);
        }
      } else {
        const float4 a = *reinterpret_cast<const float4*>(ys + s * ld_s + c);
        const float4 b = *reinterpret_cast<const float4*>(ys + s * ld_s + c + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) acc[h] = fmaf(w, v[h], acc[h]);
    }
    if constexpr (sizeof(TO) == 2) {
      uint4 q;
      q.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
      q.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
      q.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
      q.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
      *reinterpret_cast<uint4*>(y + t * ldy + c) = q;
    } else {
      *reinterpret_cast<float4*>(y + t * ldy + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(y + t * ldy + c + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

static size_t a256(size_t v) { return (v + 255) / 256 * 256; }

size_t route_ws_bytes(int64_t T, int E, int k) {
  const int64_t nb = (T + kRouteBlock - 1) / kRouteBlock;
  return 2 * a256((size_t)T * k * 4) + a256((size_t)nb * E * 4);
}

int route_launch(const float* logits, int64_t T, int E, int k, int64_t ld, int32_t* group_offsets, int32_t* a_rows,
                 int32_t* slot_of, float* weights, void* ws, hipStream_t st) {
  const int64_t nb = (T + kRouteBlock - 1) / kRouteBlock;
  int32_t* ids = reinterpret_cast<int32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + a256((size_t)T * k * 4));
  int32_t* hist = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + 2 * a256((size_t)T * k * 4));
  int slot = launch_begin(KC_ROUTE, st);
  if (E <= kWaveTopkMaxE) {
    if (E <= kWaveTopkMaxE / 2)
      hipLaunchKernelGGL((route_topk_wave_kernel<kPerLane / 2>), dim3((uint32_t)nb), dim3(kWaveTopkWaves * 64), 0, st,
                         logits, T, E, k, ld, ids, weights, rank, hist);
    else
      hipLaunchKernelGGL((route_topk_wave_kernel<kPerLane>), dim3((uint32_t)nb), dim3(kWaveTopkWaves * 64), 0, st,
                         logits, T, E, k, ld, ids, weights, rank, hist);
  } else {
    const uint32_t g1 = (uint32_t)((T + kRouteWg - 1) / kRouteWg);
    hipLaunchKernelGGL(route_topk_kernel, dim3(g1), dim3(kRouteWg), 0, st, logits, T, E, k, ld, ids, weights, rank,
                       hist);
  }
  launch_end(slot, st);
  slot = launch_begin(KC_ROUTE, st);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, hist, nb, E, group_offsets);
  launch_end(slot, st);
  int64_t g3 = (T * k + 255) / 256;
  if (g3 > 4096) g3 = 4096;
  slot = launch_begin(KC_ROUTE, st);
  hipLaunchKernelGGL(route_scatter_kernel, dim3((uint32_t)g3), dim3(256), 0, st, ids, rank, hist, group_offsets, T,
                     E, k, a_rows, slot_of);
  launch_end(slot, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int combine_launch(const void* ys, int ys_bf16, int64_t ld_s, const int32_t* slot_of, const float* weights, int64_t T,
                   int k, int64_t N, void* y, int y_bf16, int64_t ldy, hipStream_t st) {
  int64_t g = (T * (N / 8) + 255) / 256;
  if (g > 8192) g = 8192;
  const dim3 grid((uint32_t)g), blk(256);
  const int slot = launch_begin(KC_COMBINE, st);
  if (ys_bf16 && y_bf16)
    hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t>), grid, blk, 0, st,
                       reinterpret_cast<const uint16_t*>(ys), ld_s, slot_of, weights, T, k, N,
                       reinterpret_cast<uint16_t*>(y), ldy);
  else if (ys_bf16)
    hipLaunchKernelGGL((combine_kernel<uint16_t, float>), grid, blk, 0, st, reinterpret_cast<const uint16_t*>(ys),
                       ld_s, slot_of, weights, T, k, N, reinterpret_cast<float*>(y), ldy);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_kernel<float, uint16_t>), grid, blk, 0, st, reinterpret_cast<const float*>(ys), ld_s,
                       slot_of, weights, T, k, N, reinterpret_cast<uint16_t*>(y), ldy);
  else
    hipLaunchKernelGGL((combine_kernel<float, float>), grid, blk, 0, st, reinterpret_cast<const float*>(ys), ld_s,
                       slot_of, weights, T, k, N, reinterpret_cast<float*>(y), ldy);
  launch_end(slot, st);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // namespace nvfp4
