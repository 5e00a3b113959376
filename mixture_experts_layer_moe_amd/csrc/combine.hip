// Gather and top-k weighted reduce back to token order.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts", section 2.1: expert outputs are gathered back to their
// tokens and reduced over the top-k choices.
//
//   out[t, :] = sum_{j = 0..k-1, inv_perm[t, j] >= 0} topk_w[t, j] * y_perm[inv_perm[t, j], :]
//
// HBM-bound: reads each routed row once (fp32), writes each token row once.
// A block owns one token (blockIdx.x, block-uniform, so its k row indices and weights are
// scalar loads) and a span of kCols float4 columns; each thread issues the
// loads of all k slots before the first add, then sums in slot order in
// registers, so the result is deterministic and needs no atomics.  Rows are
// streamed once, so loads and stores bypass the caches' retention
// (nontemporal).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// kVec float4 columns per thread (1, 2 or 4: a block covers up to a 4096-wide row).
template <int K, int kVec>
__global__ __launch_bounds__(kThreads) void combine_kernel(const floatx4* __restrict__ y_perm,
                                                           const int32_t* __restrict__ inv_perm,
                                                           const float* __restrict__ topk_w, int k_rt,
                                                           int H4, int64_t R_cap,
                                                           floatx4* __restrict__ out) {
  constexpr int kCols = kThreads * kVec;  // float4 columns per block
  const int kk = K > 0 ? K : k_rt;
  const int64_t t = blockIdx.x;
  const int c0 = blockIdx.y * kCols + threadIdx.x;
  floatx4 acc[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (K > 0) {
    int rows[K > 0 ? K : 1];
    float w[K > 0 ? K : 1];
    floatx4 y[K > 0 ? K : 1][kVec];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int p = inv_perm[t * K + j];
      rows[j] = (p >= 0 && p < R_cap) ? p : -1;
      w[j] = topk_w[t * K + j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int c = c0 + v * kThreads;
        y[j][v] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (rows[j] >= 0 && c < H4) y[j][v] = __builtin_nontemporal_load(y_perm + (int64_t)rows[j] * H4 + c);
      }
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (rows[j] >= 0)
#pragma unroll
        for (int v = 0; v < kVec; ++v) acc[v] += w[j] * y[j][v];
  } else {
    for (int j = 0; j < kk; ++j) {
      const int p = inv_perm[t * kk + j];
      if (p < 0 || p >= R_cap) continue;
      const float w = topk_w[t * kk + j];
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        const int c = c0 + v * kThreads;
        if (c < H4) acc[v] += w * y_perm[(int64_t)p * H4 + c];
      }
    }
  }
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    const int c = c0 + v * kThreads;
    if (c < H4) __builtin_nontemporal_store(acc[v], out + t * H4 + c);
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T,
                          int k, int H, int64_t R_cap, float* out, hipStream_t s) {
  const int H4 = H / 4;
  const floatx4* y = reinterpret_cast<const floatx4*>(y_perm);
  floatx4* o = reinterpret_cast<floatx4*>(out);
  // Float4 columns per thread: enough that one block covers the row (up to 4),
  // so a token's index and weight loads are paid once.
  const int vec = H4 >= 4 * kThreads ? 4 : H4 >= 2 * kThreads ? 2 : 1;
#define MOE_COMBINE_LAUNCH(KV, V)                                                                              \
  hipLaunchKernelGGL((combine_kernel<KV, V>), dim3((unsigned)T, (unsigned)((H4 + kThreads * V - 1) / (kThreads * V))), \
                     dim3(kThreads), 0, s, y, inv_perm, topk_w, k, H4, R_cap, o)
#define MOE_COMBINE_V(V)                                  \
  switch (k) {                                            \
    case 1: MOE_COMBINE_LAUNCH(1, V); break;              \
    case 2: MOE_COMBINE_LAUNCH(2, V); break;              \
    case 4: MOE_COMBINE_LAUNCH(4, V); break;              \
    case 6: MOE_COMBINE_LAUNCH(6, V); break;              \
    case 8: MOE_COMBINE_LAUNCH(8, V); break;              \
    default: MOE_COMBINE_LAUNCH(0, V); break;             \
  }
  if (vec == 4) {
    MOE_COMBINE_V(4)
  } else if (vec == 2) {
    MOE_COMBINE_V(2)
  } else {
    MOE_COMBINE_V(1)
  }
#undef MOE_COMBINE_V
#undef MOE_COMBINE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
