// extern "C" entry points of libmoe.so: host-side validation, then launch.
// The operations and their argument conventions are documented in include/moe.h.
#include "../../include/moe.h"
#include "common.h"

namespace {

constexpr int32_t kAbiVersion = 5;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool tile_m_ok(int32_t tm) { return tm == 16 || tm == 32 || tm == 64 || tm == 128 || tm == 256; }
moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_abi_version(void) { return kAbiVersion; }

int64_t moe_rows_capacity(int64_t T, int32_t k, int32_t E_loc, int32_t tile_m) {
  if (T < 0 || k < 1 || E_loc < 1 || tile_m < 1) return -1;
  return T * min64(k, E_loc) + (int64_t)E_loc * (tile_m - 1);
}

int64_t moe_tiles_capacity(int64_t T, int32_t k, int32_t E_loc, int32_t tile_m) {
  if (T < 0 || k < 1 || E_loc < 1 || tile_m < 1) return -1;
  return T * min64(k, E_loc) / tile_m + E_loc;
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E_loc, int32_t num_ranks) {
  if (T < 0 || k < 1 || E_loc < 1 || num_ranks < 1) return 0;
  return moe::permute_ws_bytes(T, k, E_loc, num_ranks);
}

moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                          int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || k > 32) return MOE_ERR_UNSUPPORTED;
  if (T > (int64_t)INT32_MAX / 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w)) return MOE_ERR_INVALID_ARG;
  return launched(moe::launch_route_topk(logits, T, E, k, renormalize, topk_idx, topk_w,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared validation and launch of moe_permute (caller's workspace) and
// moe_permute_noalloc (static == true: the library's fixed scratch).
moe_status permute_impl(const void* x, const int32_t* topk_idx, const int32_t* src_rank, int64_t T, int32_t H,
                        int32_t k, int32_t E, int32_t expert_begin, int32_t E_loc, int32_t num_ranks,
                        int32_t tile_m, void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* row_src, int32_t* inv_perm, int32_t* tiles, int32_t* num_tiles, void* ws,
                        size_t ws_bytes, bool static_ws, void* stream) {
  if (T < 0 || H < 1 || k < 1 || E < 1 || k > E || E_loc < 1 || expert_begin < 0 ||
      (int64_t)expert_begin + E_loc > E || num_ranks < 1)
    return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0 || !tile_m_ok(tile_m) || k > 32 || num_ranks > 64 || (int64_t)E_loc * num_ranks > 4096)
    return MOE_ERR_UNSUPPORTED;
  const int64_t R_cap = moe_rows_capacity(T, k, E_loc, tile_m);
  if (T * (int64_t)k > INT32_MAX || R_cap > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  // x and x_perm both null: indices only (the rows are gathered later by moe_grouped_ffn_gather).
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {topk_idx, expert_counts, expert_offsets, row_src, inv_perm, tiles, num_tiles};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (src_rank && !aligned16(src_rank)) return MOE_ERR_INVALID_ARG;
  if (static_ws) {
    static_assert(moe::kPermuteStaticWsBytes == MOE_PERMUTE_NOALLOC_MAX_BYTES, "header and library agree");
    if (moe::permute_ws_bytes(T, k, E_loc, num_ranks) > moe::kPermuteStaticWsBytes) return MOE_ERR_WORKSPACE;
    if (moe::permute_static_ws(&ws) != hipSuccess) return MOE_ERR_LAUNCH;
  } else {
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe::permute_ws_bytes(T, k, E_loc, num_ranks)) return MOE_ERR_WORKSPACE;
  }
  moe::PermuteArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.topk_idx = topk_idx;
  a.src_rank = src_rank;
  a.T = T;
  a.H = H;
  a.k = k;
  a.E = E;
  a.expert_begin = expert_begin;
  a.E_loc = E_loc;
  a.num_ranks = src_rank ? num_ranks : 1;
  a.tile_m = tile_m;
  a.R_cap = R_cap;
  a.tiles_cap = moe_tiles_capacity(T, k, E_loc, tile_m);
  a.x_perm = static_cast<uint16_t*>(x_perm);
  a.counts = expert_counts;
  a.offsets = expert_offsets;
  a.row_src = row_src;
  a.inv_perm = inv_perm;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.ws = ws;
  return launched(moe::launch_permute(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

moe_status moe_permute(const void* x, const int32_t* topk_idx, const int32_t* src_rank, int64_t T, int32_t H,
                       int32_t k, int32_t E, int32_t expert_begin, int32_t E_loc, int32_t num_ranks,
                       int32_t tile_m, void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* row_src, int32_t* inv_perm, int32_t* tiles, int32_t* num_tiles, void* ws,
                       size_t ws_bytes, void* stream) {
  return permute_impl(x, topk_idx, src_rank, T, H, k, E, expert_begin, E_loc, num_ranks, tile_m, x_perm,
                      expert_counts, expert_offsets, row_src, inv_perm, tiles, num_tiles, ws, ws_bytes, false,
                      stream);
}

moe_status moe_permute_noalloc(const void* x, const int32_t* topk_idx, const int32_t* src_rank, int64_t T,
                               int32_t H, int32_t k, int32_t E, int32_t expert_begin, int32_t E_loc,
                               int32_t num_ranks, int32_t tile_m, void* x_perm, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* row_src, int32_t* inv_perm, int32_t* tiles,
                               int32_t* num_tiles, void* stream) {
  return permute_impl(x, topk_idx, src_rank, T, H, k, E, expert_begin, E_loc, num_ranks, tile_m, x_perm,
                      expert_counts, expert_offsets, row_src, inv_perm, tiles, num_tiles, nullptr, 0, true, stream);
}

size_t moe_grouped_ffn_workspace_bytes(int32_t tile_m, int32_t H) {
  if (!tile_m_ok(tile_m) || H < 1) return 0;
  return moe::grouped_ffn_ws_bytes(tile_m, H);
}

namespace {

// Shared validation and launch of moe_grouped_ffn (x_perm given) and
// moe_grouped_ffn_gather (x, row_src, T, k given, x_perm null).
moe_status grouped_ffn_impl(const void* x_perm, const void* x, const int32_t* row_src, int64_t T, int32_t k,
                            const int32_t* expert_counts, const int32_t* expert_offsets, const int32_t* tiles,
                            const int32_t* num_tiles, const void* w0, const void* w0_up, const void* w1,
                            int32_t E_loc, int32_t H, int32_t F, int32_t act, int32_t tile_m, int64_t R_cap,
                            int64_t tiles_cap, void* act_buf, float* y_perm, void* ws, size_t ws_bytes,
                            void* stream) {
  if (E_loc < 1 || H < 1 || F < 1 || R_cap < 0 || tiles_cap < 0) return MOE_ERR_INVALID_ARG;
  if (act != MOE_ACT_GELU && act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if ((act == MOE_ACT_SWIGLU) != (w0_up != nullptr)) return MOE_ERR_INVALID_ARG;
  if (H % 128 != 0 || F % 128 != 0 || !tile_m_ok(tile_m)) return MOE_ERR_UNSUPPORTED;
  if (H > (1 << 20) || F > (1 << 20)) return MOE_ERR_UNSUPPORTED;  // 32-bit operand-panel offsets
  if (R_cap > INT32_MAX || tiles_cap > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const bool gather = x_perm == nullptr;
  if (gather) {
    if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
    if (T * (int64_t)H * 2 > INT32_MAX || T * (int64_t)k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  }
  if (R_cap == 0 || tiles_cap == 0) return MOE_OK;
  const void* ptrs[] = {gather ? x : x_perm, expert_counts, expert_offsets, tiles, num_tiles, w0, w1, act_buf, y_perm};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (gather && (!row_src || !aligned16(row_src))) return MOE_ERR_INVALID_ARG;
  if (w0_up && !aligned16(w0_up)) return MOE_ERR_INVALID_ARG;
  if (ws) {
    if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe::grouped_ffn_ws_bytes(tile_m, H)) return MOE_ERR_WORKSPACE;
  }
  moe::FfnArgs a{};
  a.x_perm = static_cast<const uint16_t*>(x_perm);
  a.x = static_cast<const uint16_t*>(x);
  a.row_src = row_src;
  a.topk = k;
  a.T = T;
  a.counts = expert_counts;
  a.offsets = expert_offsets;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.w0 = static_cast<const uint16_t*>(w0);
  a.w0_up = static_cast<const uint16_t*>(w0_up);
  a.w1 = static_cast<const uint16_t*>(w1);
  a.E_loc = E_loc;
  a.H = H;
  a.F = F;
  a.act = act;
  a.tile_m = tile_m;
  a.R_cap = R_cap;
  a.tiles_cap = tiles_cap;
  a.act_buf = static_cast<uint16_t*>(act_buf);
  a.y_perm = y_perm;
  a.ws = ws;
  a.stream = static_cast<hipStream_t>(stream);
  return launched(moe::launch_grouped_ffn(a));
}

}  // namespace

moe_status moe_grouped_ffn(const void* x_perm, const int32_t* expert_counts, const int32_t* expert_offsets,
                           const int32_t* tiles, const int32_t* num_tiles, const void* w0, const void* w0_up,
                           const void* w1, int32_t E_loc, int32_t H, int32_t F, int32_t act, int32_t tile_m,
                           int64_t R_cap, int64_t tiles_cap, void* act_buf, float* y_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!x_perm) return MOE_ERR_INVALID_ARG;
  return grouped_ffn_impl(x_perm, nullptr, nullptr, 0, 0, expert_counts, expert_offsets, tiles, num_tiles, w0, w0_up,
                          w1, E_loc, H, F, act, tile_m, R_cap, tiles_cap, act_buf, y_perm, ws, ws_bytes, stream);
}

moe_status moe_grouped_ffn_gather(const void* x, const int32_t* row_src, int64_t T, int32_t k,
                                  const int32_t* expert_counts, const int32_t* expert_offsets,
                                  const int32_t* tiles, const int32_t* num_tiles, const void* w0,
                                  const void* w0_up, const void* w1, int32_t E_loc, int32_t H, int32_t F,
                                  int32_t act, int32_t tile_m, int64_t R_cap, int64_t tiles_cap, void* act_buf,
                                  float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  if (!x) return MOE_ERR_INVALID_ARG;
  return grouped_ffn_impl(nullptr, x, row_src, T, k, expert_counts, expert_offsets, tiles, num_tiles, w0, w0_up, w1,
                          E_loc, H, F, act, tile_m, R_cap, tiles_cap, act_buf, y_perm, ws, ws_bytes, stream);
}

size_t moe_ffn_combine_fused_workspace_bytes(int64_t tiles_cap, int32_t H) {
  if (tiles_cap < 0 || H < 256 || H % 256 != 0 || tiles_cap > INT32_MAX / 2) return 0;
  return moe::fused_ffn_ws_bytes(tiles_cap, H);
}

moe_status moe_ffn_combine_fused(const void* x_perm, const int32_t* expert_counts, const int32_t* expert_offsets,
                                 const int32_t* tiles, const int32_t* num_tiles, const void* w0, const void* w0_up,
                                 const void* w1, int32_t E_loc, int32_t H, int32_t F, int32_t act, int32_t tile_m,
                                 int64_t R_cap, int64_t tiles_cap, void* act_buf, float* y_perm,
                                 const int32_t* inv_perm, const float* topk_w, int64_t T, int32_t k, float* out,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (E_loc < 1 || H < 1 || F < 1 || R_cap < 0 || tiles_cap < 0 || T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (act != MOE_ACT_GELU && act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if ((act == MOE_ACT_SWIGLU) != (w0_up != nullptr)) return MOE_ERR_INVALID_ARG;
  if (tile_m != 256 || H % 256 != 0 || F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (H > (1 << 20) || F > (1 << 20) || k > 32) return MOE_ERR_UNSUPPORTED;
  if (R_cap > INT32_MAX || tiles_cap > INT32_MAX / 2 || T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x_perm, expert_counts, expert_offsets, tiles, num_tiles, w0, w1, act_buf, y_perm,
                        inv_perm, topk_w, out, ws};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (w0_up && !aligned16(w0_up)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe::fused_ffn_ws_bytes(tiles_cap, H)) return MOE_ERR_WORKSPACE;
  moe::FfnArgs a{};
  a.x_perm = static_cast<const uint16_t*>(x_perm);
  a.counts = expert_counts;
  a.offsets = expert_offsets;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.w0 = static_cast<const uint16_t*>(w0);
  a.w0_up = static_cast<const uint16_t*>(w0_up);
  a.w1 = static_cast<const uint16_t*>(w1);
  a.E_loc = E_loc;
  a.H = H;
  a.F = F;
  a.act = act;
  a.tile_m = tile_m;
  a.R_cap = R_cap;
  a.tiles_cap = tiles_cap;
  a.act_buf = static_cast<uint16_t*>(act_buf);
  a.y_perm = y_perm;
  a.ws = ws;
  a.topk = k;
  a.T = T;
  a.stream = static_cast<hipStream_t>(stream);
  return launched(moe::launch_ffn_fused(a, inv_perm, topk_w, out));
}

moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T, int32_t k,
                       int32_t H, int64_t R_cap, float* out, void* stream) {
  if (T < 0 || k < 1 || H < 1 || R_cap < 0) return MOE_ERR_INVALID_ARG;
  if (H % 4 != 0 || k > 32 || T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv_perm || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(inv_perm) || !aligned16(topk_w) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  return launched(moe::launch_combine(y_perm, inv_perm, topk_w, T, k, H, R_cap, out,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
