// Shared device helpers and internal launcher declarations for libmoe.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int intx4;

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// ---------------------------------------------------------------------------
// Internal launchers (implemented in the .hip files; called by moe_api.hip
// after argument validation).  All return hipGetLastError() after launching.
// ---------------------------------------------------------------------------
hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int renormalize,
                             int32_t* topk_idx, float* topk_w, hipStream_t s);

struct PermuteArgs {
  const uint16_t* x;
  const int32_t* topk_idx;
  const int32_t* src_rank;  // may be null
  int64_t T;
  int H, k, E, expert_begin, E_loc, num_ranks, tile_m;
  int64_t R_cap, tiles_cap;
  uint16_t* x_perm;
  int32_t *counts, *offsets, *row_src, *inv_perm, *tiles, *num_tiles;
  void* ws;
};
size_t permute_ws_bytes(int64_t T, int k, int E_loc, int num_ranks);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// Fixed per-device scratch of moe_permute_noalloc (a static device array).
constexpr size_t kPermuteStaticWsBytes = (size_t)8 << 20;
// Its device address on the current device (looked up on the first call per device).
hipError_t permute_static_ws(void** ptr);

struct FfnArgs {
  const uint16_t* x_perm;
  const int32_t *counts, *offsets, *tiles, *num_tiles;
  const uint16_t *w0, *w0_up, *w1;
  int E_loc, H, F, act, tile_m;
  int64_t R_cap, tiles_cap;
  uint16_t* act_buf;
  float* y_perm;
  void* ws;  // split-K partials of layer1's last round, or null
  // x_perm == null: layer0 gathers its rows from x [T, H] through row_src (t * topk + slot; < 0 padding)
  const uint16_t* x;
  const int32_t* row_src;
  int topk;
  int64_t T;
  int cus;  // CUs the launch stream may use (set by launch_grouped_ffn)
  hipStream_t stream;
};
size_t grouped_ffn_ws_bytes(int tile_m, int H);
hipError_t launch_grouped_ffn(const FfnArgs& a);
// One persistent launch of layer0, layer1 and the combine with tile-level signals (tile_m 256).
size_t fused_ffn_ws_bytes(int64_t tiles_cap, int H);
hipError_t launch_ffn_fused(const FfnArgs& a, const int32_t* inv_perm, const float* topk_w, float* out);

hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                          int64_t T, int k, int H, int64_t R_cap, float* out, hipStream_t s);

}  // namespace moe
