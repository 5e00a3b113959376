// Gather and top-k weighted reduce back to token order.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts", section 2.1: expert outputs are gathered back to their
// tokens and reduced over the top-k choices.
//
//   out[t, :] = sum_{j = 0..k-1, inv_perm[t, j] >= 0} topk_w[t, j] * y_perm[inv_perm[t, j], :]
//
// HBM-bound: reads each routed row once (fp32), writes each token row once.
// One block per group of tokens; each thread owns 16-byte (float4) column
// chunks and sums the k slots in slot order in registers, so the result is
// deterministic and needs no atomics.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const floatx4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w, int64_t T,
                                                      int k, int H4, int64_t R_cap,
                                                      floatx4* __restrict__ out, int tokens_per_block) {
  // Threads split into tokens_per_block groups; group g handles token t.
  const int group_size = blockDim.x / tokens_per_block;
  const int g = threadIdx.x / group_size, gt = threadIdx.x % group_size;
  const int64_t t = (int64_t)blockIdx.x * tokens_per_block + g;
  if (t >= T) return;
  int rows[32];
  float w[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    rows[j] = -1;
    w[j] = 0.f;
    if (j < k) {
      const int p = inv_perm[t * k + j];
      rows[j] = (p >= 0 && p < R_cap) ? p : -1;
      w[j] = topk_w[t * k + j];
    }
  }
  floatx4* o = out + t * H4;
  for (int c = gt; c < H4; c += group_size) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (rows[j] < 0) continue;
      const floatx4 y = y_perm[(int64_t)rows[j] * H4 + c];
      acc += w[j] * y;
    }
    o[c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T,
                          int k, int H, int64_t R_cap, float* out, hipStream_t s) {
  const int H4 = H / 4;
  // Enough threads per token to cover a row in a few passes; small rows share a block.
  int tpb = 1;  // tokens per block; each token keeps a multiple of 64 threads
  while (tpb < 4 && 256 / (tpb * 2) >= H4) tpb *= 2;
  const int64_t blocks = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const floatx4*>(y_perm), inv_perm, topk_w, T, k, H4, R_cap,
                     reinterpret_cast<floatx4*>(out), tpb);
  return hipGetLastError();
}

}  // namespace moe
