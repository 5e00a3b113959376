// Top-k routing with renormalised gate weights.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts", section 2.1 (MoE Structure): each token activates only
// the experts its router selects, and the gate weights weight the top-k
// reduce.  Gate = softmax over the k selected logits (full softmax
// renormalised over the top-k).
//
// E <= 64 and k <= 8: four lanes per token, each keeping the best k of its
// sixteen logits, merged inside the quad (route_topk_quad_kernel).
// Otherwise one wavefront per token.  Lane l holds logits e = l, l+64, ...
// (E <= 1024, so at most 16 per lane).  k rounds of a wave-wide arg-max on the key
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

// E <= 64 and k <= KS <= 8: four lanes (a quad) per token, lane s of the quad
// holding logits 16 s .. 16 s + 15.  Each lane keeps the best KS of its
// logits, sorted on (value desc, id asc), by insertion in id order (an equal
// logit never displaces an earlier one).  Two exchanges inside the quad (DPP
// quad permutations) merge the lists: a descending list followed by the
// partner's reversed is bitonic, so the element-wise better of the two holds
// the best KS, and a bitonic merge network sorts them.  Every comparison is
// exact, so the ids equal those of the wave-wide arg-max rounds.
template <int KS>
__global__ __launch_bounds__(256) void route_topk_quad_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                              int k, int renormalize, int vec4,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_w) {
  const int sub = threadIdx.x & 3;
  const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const bool valid = t < T;  // a quad's lanes agree
  float x[16];
  const int e0 = 16 * sub;
  if (valid && vec4 && e0 + 16 <= E) {  // 16-byte loads: E % 4 == 0 and logits 16-byte aligned
    const floatx4* row = reinterpret_cast<const floatx4*>(logits + t * (int64_t)E + e0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4 v4 = row[q];
      x[4 * q] = v4[0]; x[4 * q + 1] = v4[1]; x[4 * q + 2] = v4[2]; x[4 * q + 3] = v4[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (valid && e0 + i < E) ? logits[t * (int64_t)E + e0 + i] : -__builtin_inff();
  }
  float v[KS];
  int id[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    v[j] = -__builtin_inff();
    id[j] = 0x7fffffff;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (e0 + i >= E) break;
    const float xv = x[i];
    // The new logit ranks ahead of entry j iff it is strictly larger (its id is larger).
#pragma unroll
    for (int j = KS - 1; j >= 0; --j) {
      const bool ahead = xv > v[j];
      const bool ahead_prev = j > 0 && xv > v[j > 0 ? j - 1 : 0];
      const float nv = ahead_prev ? v[j > 0 ? j - 1 : 0] : (ahead ? xv : v[j]);
      const int ni = ahead_prev ? id[j > 0 ? j - 1 : 0] : (ahead ? e0 + i : id[j]);
      v[j] = nv;
      id[j] = ni;
    }
  }
  auto merge = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    float pv[KS];
    int pi[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      pv[j] = dpp<C>(v[j]);
      pi[j] = dpp<C>(id[j]);
    }
#pragma unroll
    for (int j = 0; j < KS; ++j)
      if (better(pv[KS - 1 - j], pi[KS - 1 - j], v[j], id[j])) {
        v[j] = pv[KS - 1 - j];
        id[j] = pi[KS - 1 - j];
      }
#pragma unroll
    for (int d = KS / 2; d >= 1; d /= 2)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        if ((j & d) == 0 && better(v[j + d], id[j + d], v[j], id[j])) {
          const float tv = v[j];
          const int ti = id[j];
          v[j] = v[j + d];
          id[j] = id[j + d];
          v[j + d] = tv;
          id[j + d] = ti;
        }
  };
  merge(std::integral_constant<int, 0xB1>{});  // quad_perm [1,0,3,2]
  merge(std::integral_constant<int, 0x4E>{});  // quad_perm [2,3,0,1]
  float denom = 0.f;
  if (renormalize) {
#pragma unroll
    for (int j = 0; j < KS; ++j)
      if (j < k) denom += expf(v[j] - v[0]);
  } else {
    // Full softmax denominator over all E logits: this lane's sixteen, then the quad.
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (e0 + i < E) s += expf(x[i] - v[0]);
    s += dpp<0xB1>(s);
    s += dpp<0x4E>(s);
    denom = s;
  }
  if (valid && sub == 0) {
#pragma unroll
    for (int j = 0; j < KS; ++j)
      if (j < k) {
        topk_idx[t * k + j] = id[j];
        topk_w[t * k + j] = expf(v[j] - v[0]) / denom;
      }
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
  if (E <= 64 && k <= 8) {
    const dim3 qgrid((unsigned)((T + 63) / 64));  // 64 tokens (256 lanes) per block
    const int vec4 = (E % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
#define MOE_QUAD(KS_)                                                                                    \
  hipLaunchKernelGGL(route_topk_quad_kernel<KS_>, qgrid, dim3(256), 0, s, logits, T, E, k, renormalize, vec4, \
                     topk_idx, topk_w)
    if (k <= 1) MOE_QUAD(1);
    else if (k <= 2) MOE_QUAD(2);
    else if (k <= 4) MOE_QUAD(4);
    else MOE_QUAD(8);
#undef MOE_QUAD
  } else if (pl <= 1)
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
