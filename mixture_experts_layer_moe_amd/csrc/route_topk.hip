// Top-k routing with renormalised gate weights.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts", section 2.1 (MoE Structure): each token activates only
// the experts its router selects, and the gate weights weight the top-k
// reduce.  Gate = softmax over the k selected logits (full softmax
// renormalised over the top-k).
//
// One wavefront per token.  Lane l holds logits e = l, l+64, ... (E <= 1024,
// so at most 16 per lane).  k rounds of a wave-wide arg-max on the key
// (value desc, id asc) select the experts in slot order; the comparisons are
// exact, so the ids are bit-identical to any correct sort with that key.
// A round is a wave-wide max of the lanes' best logits (DPP inside each
// 16-lane row, then the four row results by readlane).  With E <= 64 (one
// logit per lane) a ballot of the lanes holding it follows: the lowest such
// lane is the lowest expert id among equal logits; otherwise a wave-wide
// minimum of the ids of the lanes holding it.
#include "common.h"

#include <type_traits>

namespace moe {
namespace {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Wave-wide reductions, result in every lane: quad swaps and the 8- and
// 16-lane mirrors (DPP) give each lane its 16-lane row's result, and the four
// row results are read with readlane (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lanef(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return fmaxf(fmaxf(lanef(x, 0), lanef(x, 16)), fmaxf(lanef(x, 32), lanef(x, 48)));
}

__device__ __forceinline__ int wave_min(int x) {
  x = min(x, dpp<0xB1>(x));
  x = min(x, dpp<0x4E>(x));
  x = min(x, dpp<0x141>(x));
  x = min(x, dpp<0x140>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// E <= 64: lane l holds logit l.
__global__ __launch_bounds__(256) void route_topk_small_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                               int k, int renormalize,
                                                               int32_t* __restrict__ topk_idx,
                                                               float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float x = lane < E ? logits[t * (int64_t)E + lane] : -__builtin_inff();
  float v = x, top = 0.f, sel_v = 0.f, zsum = 0.f;
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    const float m = wave_max(v);
    // k <= E and finite logits: some lane still holds m.
    const int win = __builtin_ctzll(__ballot(v == m));
    if (lane == win) v = -__builtin_inff();
    if (j == 0) top = m;
    zsum += expf(m - top);
    if (lane == j) {
      sel_v = m;
      sel_i = win;
    }
  }
  float denom = zsum;
  if (!renormalize) {
    // Full softmax denominator over all E logits.
    float s = lane < E ? expf(x - top) : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    denom = s;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = sel_i;
    topk_w[t * k + lane] = expf(sel_v - top) / denom;
  }
}

// General E (<= 64 * PL): lane l holds logits l, l + 64, ...
template <int PL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int k, int renormalize,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  constexpr int kMaxPerLane = PL;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float* row = logits + t * (int64_t)E;

  float v[kMaxPerLane];
  const int per_lane = (E + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = (i < per_lane && e < E) ? row[e] : -__builtin_inff();
  }
  uint32_t taken = 0;  // bit i set: v[i] already selected (or absent)
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (!(i < per_lane && lane + i * kWave < E)) taken |= 1u << i;

  float top = 0.f, sel_v = 0.f;
  int sel_i = 0;
  float zsum = 0.f;
  // Slot results are kept by lane j (j < k <= 32).
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (!(taken & (1u << i)) && better(v[i], lane + i * kWave, bv, bi)) {
        bv = v[i];
        bi = lane + i * kWave;
      }
    }
    // Wave arg-max on (value desc, id asc): the largest value, then the lowest id holding it.
    const float m = wave_max(bv);
    bi = wave_min(bv == m ? bi : 0x7fffffff);
    bv = m;
    // bv, bi are now wave-uniform: the j-th expert of this token.
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) top = bv;
    const float z = expf(bv - top);
    zsum += z;
    if (lane == j) {
      sel_v = bv;
      sel_i = bi;
    }
  }
  float denom = zsum;
  if (!renormalize) {
    // Full softmax denominator over all E logits.
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (i < per_lane && e < E) s += expf(v[i] - top);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    denom = s;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = sel_i;
    topk_w[t * k + lane] = expf(sel_v - top) / denom;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int renormalize,
                             int32_t* topk_idx, float* topk_w, hipStream_t s) {
  constexpr int kTokensPerBlock = 4;
  const int64_t blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
  const dim3 grid((unsigned)blocks), block(kTokensPerBlock * kWave);
  const int pl = (E + kWave - 1) / kWave;
  if (pl <= 1)
    hipLaunchKernelGGL(route_topk_small_kernel, grid, block, 0, s, logits, T, E, k, renormalize, topk_idx, topk_w);
  else if (pl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, renormalize, topk_idx, topk_w);
  else if (pl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, renormalize, topk_idx, topk_w);
  else if (pl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, renormalize, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, renormalize, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
