/*
 * moe.h -- C ABI of libmoe.so: one GPU's share of a Mixture-of-Experts layer
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer, as "Comet: Fine-grained Computation-communication Overlapping for
 * Mixture-of-Experts" (paperlayer.ai summary) states it in section 2.1 (MoE
 * Structure), routes every token to its top-k experts, runs each selected
 * expert's feed-forward network on it, and gathers and reduces the expert
 * outputs over the k choices.  The four calls below are the steps of that
 * path, in order:
 *
 *   moe_route_topk   top-k routing and gate weights
 *   moe_permute      reorganisation into expert-contiguous, tile-aligned rows
 *   moe_grouped_ffn  layer0 grouped GEMM + activation, layer1 grouped GEMM
 *                    (moe_grouped_ffn_gather: the same, with layer0's token
 *                    rows gathered from x instead of read from x_perm)
 *   moe_combine      top-k weighted reduce back to token order
 *
 * Two more entry points: moe_ffn_combine_fused runs moe_grouped_ffn and
 * moe_combine as one persistent launch with tile-level signals, and
 * moe_permute_noalloc is moe_permute on a fixed per-device scratch array for
 * callers that cannot allocate.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise, and
 *     must be 16-byte aligned.  The caller owns all memory: the library never
 *     allocates, frees or synchronises.  Work is enqueued on `stream` (a
 *     hipStream_t passed as void*; NULL = the default stream) and the call
 *     returns without waiting.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns its code and enqueues nothing.  Device-side faults
 *     surface at the caller's next synchronisation.  T == 0 returns MOE_OK and
 *     launches nothing.  No C++ exception crosses this interface.
 *   - Data-dependent sizes (rows per expert, number of tiles) stay on the
 *     device; capacities are host formulas (moe_rows_capacity,
 *     moe_tiles_capacity), so the four calls can be enqueued back to back
 *     without any device-to-host copy.
 *   - bf16 arguments are passed as void* and hold IEEE bfloat16 values.
 *   - Calls are stateless and re-entrant; concurrent calls on different
 *     streams must not share output or workspace buffers (nor, for
 *     moe_permute_noalloc, run concurrently on one GPU: they share its
 *     scratch array).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, misalignment, negative or inconsistent size */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement (e.g. moe_grouped_ffn with H % 128 != 0) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_permute_workspace_bytes() */
  MOE_ERR_LAUNCH = 4       /* the HIP runtime reported an error when launching */
} moe_status;

typedef enum {
  MOE_ACT_GELU = 0,  /* a = gelu(x.W1), exact erf form; y = a.W2 */
  MOE_ACT_SWIGLU = 1 /* a = silu(x.Wg) * (x.Wu), silu(z) = z/(1+e^-z); y = a.Wd */
} moe_act;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(int status);

/* Library ABI version (incremented on any signature change). */
int32_t moe_abi_version(void);

/* R_cap: rows of the reorganised buffers (x_perm, act_buf, y_perm) for T
 * tokens, top-k, E_loc local experts and row tile tile_m:
 *   T * min(k, E_loc) + E_loc * (tile_m - 1).
 * Returns -1 on invalid arguments. */
int64_t moe_rows_capacity(int64_t T, int32_t k, int32_t E_loc, int32_t tile_m);

/* Capacity of the tile list: floor(T * min(k, E_loc) / tile_m) + E_loc
 * (each tile is two int32).  Returns -1 on invalid arguments. */
int64_t moe_tiles_capacity(int64_t T, int32_t k, int32_t E_loc, int32_t tile_m);

/* Bytes of device workspace moe_permute needs.  Returns 0 on invalid arguments. */
size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E_loc, int32_t num_ranks);

/* Bytes of optional device workspace for moe_grouped_ffn with this tile_m and
 * H on the current device (0 for tile_m <= 64, which never uses it; 0 on
 * invalid arguments).  The workspace holds fp32 partial tiles: one CU-count's
 * worth of tile_m x 256 blocks. */
size_t moe_grouped_ffn_workspace_bytes(int32_t tile_m, int32_t H);

/*
 * moe_route_topk -- top-k routing (section 2.1: each token activates only the
 * experts its router selects; the gate weights weight the top-k reduce).
 *
 *   logits      [T, E] fp32, row-major; finite values (precondition).
 *   topk_idx    [T, k] int32 out: expert ids of token t in descending logit
 *               order; equal logits are taken lower id first.
 *   topk_w      [T, k] fp32 out: renormalize != 0 -> softmax over the k
 *               selected logits (each row sums to 1); renormalize == 0 ->
 *               full softmax over all E evaluated at the selected experts.
 * Requires 1 <= k <= E, E <= 1024, k <= 32.
 */
moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                          int32_t renormalize, int32_t* topk_idx, float* topk_w,
                          void* stream);

/*
 * moe_permute -- token reorganisation into expert-contiguous, tile-aligned
 * sub-tensors (section 3.1.2: sub-tensors are regrouped into GEMM tiles;
 * layer0 sorts tokens by source rank and prioritises tiles with local
 * tokens; section 2.2.1: reorganisation exposes only the data a tile needs).
 *
 * The (token t, slot j) pairs whose expert e = topk_idx[t, j] lies in the
 * local range [expert_begin, expert_begin + E_loc) are sorted by
 * (e - expert_begin, src_rank[t], t); each local expert's rows are padded up
 * to a multiple of tile_m.  Outputs:
 *   x_perm          [R_cap, H] bf16: row p = x[row_src[p] / k]; padding rows
 *                   are left untouched (their content is unspecified).
 *   expert_counts   [E_loc] int32: real rows per local expert.
 *   expert_offsets  [E_loc + 1] int32: padded first row of each expert.
 *   row_src         [R_cap] int32: t * k + j of a real row, -1 otherwise.
 *   inv_perm        [T, k] int32: row of pair (t, j), -1 if not local.
 *   tiles           [tiles_cap, 2] int32: (local expert, first row) of every
 *                   row tile, ordered by (priority, expert, tile index) where
 *                   a tile's priority is the largest source rank among its rows.
 *   num_tiles       [1] int32: number of valid entries in tiles.
 * Inputs: x [T, H] bf16; topk_idx [T, k] int32 (from moe_route_topk, or any
 * ids in [0, E) with no repeat within a row); src_rank [T] int32 with values
 * in [0, num_ranks), or NULL = every token is local (rank 0).
 * x and x_perm may both be NULL: then only the index outputs are written, for
 * moe_grouped_ffn_gather, which reads the token rows from x itself.
 * ws / ws_bytes: device scratch of at least moe_permute_workspace_bytes().
 * Requires H % 8 == 0, tile_m in {16, 32, 64, 128, 256},
 * E_loc * num_ranks <= 4096, num_ranks <= 64, k <= 32.
 */
moe_status moe_permute(const void* x, const int32_t* topk_idx, const int32_t* src_rank,
                       int64_t T, int32_t H, int32_t k, int32_t E, int32_t expert_begin,
                       int32_t E_loc, int32_t num_ranks, int32_t tile_m,
                       void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* row_src, int32_t* inv_perm, int32_t* tiles,
                       int32_t* num_tiles, void* ws, size_t ws_bytes, void* stream);

/* Scratch bytes moe_permute_noalloc can use: moe_permute_workspace_bytes()
 * must not exceed this (8 MiB, e.g. T * k up to about 2 million pairs). */
#define MOE_PERMUTE_NOALLOC_MAX_BYTES ((size_t)8 << 20)

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments, outputs and errors as
 * moe_permute, without ws / ws_bytes.  Its scratch is a fixed device array
 * inside the library, one copy per GPU, held until the process ends (its
 * address is looked up on the first call on each device); no call allocates
 * or frees memory.  Returns MOE_ERR_WORKSPACE, launching nothing, when
 * moe_permute_workspace_bytes(T, k, E_loc, num_ranks) exceeds
 * MOE_PERMUTE_NOALLOC_MAX_BYTES.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and corrupt each other's
 * results; calls ordered on one stream are safe.  Nothing in the scratch has
 * to start at zero (each launch rewrites all it reads).
 */
moe_status moe_permute_noalloc(const void* x, const int32_t* topk_idx, const int32_t* src_rank,
                               int64_t T, int32_t H, int32_t k, int32_t E, int32_t expert_begin,
                               int32_t E_loc, int32_t num_ranks, int32_t tile_m,
                               void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* row_src, int32_t* inv_perm, int32_t* tiles,
                               int32_t* num_tiles, void* stream);

/*
 * moe_grouped_ffn -- the experts' feed-forward networks as two grouped GEMMs
 * over all local experts (section 3.1.2: one GroupGEMM covers the experts of
 * this rank; section 3.1.1: layer0 is decomposed along M (token rows),
 * layer1 along N (output columns), because the top-k reduce couples rows
 * across experts; tile-level-signalling follow-up, abstract: one persistent
 * kernel covers all local experts).
 *
 *   layer0:  act_buf[p, :] = act( x_perm[p, :] . W0[e] (, x_perm[p, :] . W0u[e]) )
 *   layer1:  y_perm[p, :]  = act_buf[p, :] . W1[e]
 * for every real row p of every local expert e.  Weights are stored
 * output-major (each stored matrix is the transpose of the mathematical one,
 * so the reduction dimension is contiguous):
 *   w0      [E_loc, F, H] bf16: W_gate^T (SwiGLU) or W1^T (GELU)
 *   w0_up   [E_loc, F, H] bf16: W_up^T (SwiGLU); must be NULL for GELU
 *   w1      [E_loc, H, F] bf16: W_down^T (SwiGLU) or W2^T (GELU)
 * This is not the input-major layout a literal reading of "W1 H x F" gives
 * ([E_loc, H, F] for w0 and [E_loc, F, H] for w1): with K contiguous in both
 * GEMM operands, every operand row is one 128-byte LDS row per 64-wide K
 * stage and the MFMA fragments are read without a transpose (the storage of
 * a torch Linear weight).  A caller holding input-major weights transposes
 * them once, at load time.
 *   act_buf [R_cap, F] bf16 out: the activation, rounded to nearest even.
 *   y_perm  [R_cap, H] fp32 out.
 * Only real rows are written; padding rows of act_buf and y_perm are left
 * untouched.  x_perm, expert_counts, expert_offsets, tiles and num_tiles are
 * moe_permute's outputs for the same tile_m; R_cap and tiles_cap are the
 * capacities they were allocated with.  Accumulation is fp32.
 * ws / ws_bytes: optional device scratch (NULL / 0 is allowed) of at least
 * moe_grouped_ffn_workspace_bytes(tile_m, H); with it, the last scheduling
 * round of each layer splits its tiles along K into fp32 partials that a
 * second kernel sums in a fixed order (and then applies layer0's
 * activation), so the result stays deterministic; it can differ from the
 * result without ws by fp32 summation order (layer0: by an ulp of the bf16
 * activation).  A non-NULL ws that is too small returns MOE_ERR_WORKSPACE.
 * Requires H % 128 == 0, F % 128 == 0 (the kernels' column blocks are 128
 * wide, so a multiple of 64 alone is not accepted), H <= 1048576,
 * F <= 1048576, tile_m in {16, 32, 64, 128, 256}.
 */
moe_status moe_grouped_ffn(const void* x_perm, const int32_t* expert_counts,
                           const int32_t* expert_offsets, const int32_t* tiles,
                           const int32_t* num_tiles, const void* w0, const void* w0_up,
                           const void* w1, int32_t E_loc, int32_t H, int32_t F, int32_t act,
                           int32_t tile_m, int64_t R_cap, int64_t tiles_cap,
                           void* act_buf, float* y_perm, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * moe_grouped_ffn_gather -- moe_grouped_ffn with the permutation fused into
 * layer0's operand load (section 4: the MoE GEMMs locate their token rows
 * through an index instead of a materialised permuted copy).  Layer0 reads
 * row p of its operand as x[row_src[p] / k] straight from the token matrix
 * x [T, H] bf16 (padding rows, row_src[p] < 0, read as zeros and are never
 * stored), so moe_permute can run with x = x_perm = NULL.  row_src [R_cap]
 * int32, T and k are those of the moe_permute call that produced row_src;
 * every other argument, the outputs and the errors are as for
 * moe_grouped_ffn.  Also requires T * H * 2 <= 2^31 - 1.
 */
moe_status moe_grouped_ffn_gather(const void* x, const int32_t* row_src, int64_t T, int32_t k,
                                  const int32_t* expert_counts, const int32_t* expert_offsets,
                                  const int32_t* tiles, const int32_t* num_tiles, const void* w0,
                                  const void* w0_up, const void* w1, int32_t E_loc, int32_t H,
                                  int32_t F, int32_t act, int32_t tile_m, int64_t R_cap,
                                  int64_t tiles_cap, void* act_buf, float* y_perm, void* ws,
                                  size_t ws_bytes, void* stream);

/* Bytes of device workspace moe_ffn_combine_fused needs for this tile capacity
 * and H on the current device (0 on invalid arguments or H % 256 != 0). */
size_t moe_ffn_combine_fused_workspace_bytes(int64_t tiles_cap, int32_t H);

/*
 * moe_ffn_combine_fused -- moe_grouped_ffn followed by moe_combine as one
 * persistent launch with tile-level signals (section 3.1.2: layer1's reduce
 * and its hand-off can begin once the first column blocks are done;
 * tile-level-signalling follow-up, abstract: tiles are signalled to their
 * consumers as they become ready instead of at kernel boundaries).  Every
 * workgroup takes work items in one global order -- layer0 tiles, layer1
 * tiles column group by column group, the K slices of the last layer1 items,
 * then combine blocks of 64 tokens per column group -- and a layer1 item
 * starts as soon as the layer0 items of its row tile have signalled, a
 * combine block as soon as its column group's layer1 items have.
 *
 * Arguments, layouts and results are those of moe_grouped_ffn (act_buf,
 * y_perm) and moe_combine (inv_perm, topk_w, T, k, out): act_buf, y_perm and
 * out equal what the two calls give, up to fp32 summation order in layer1's
 * split items (deterministic run to run).  Requires tile_m == 256,
 * H % 256 == 0, F % 128 == 0, k <= 32.
 * ws / ws_bytes: device workspace of at least
 * moe_ffn_combine_fused_workspace_bytes(tiles_cap, H), ZERO-FILLED before its
 * first use; every launch leaves its counters zero again for the next one (so
 * no clearing is needed between calls, including replays of a captured
 * graph).  Its first int32 is an error word: nonzero after a launch means a
 * wait between work items timed out and that launch's outputs are invalid
 * (the launch still ends); the caller reads it after synchronising and
 * writes it back to zero.  One workspace must not be used by two launches
 * that may overlap.
 */
moe_status moe_ffn_combine_fused(const void* x_perm, const int32_t* expert_counts,
                                 const int32_t* expert_offsets, const int32_t* tiles,
                                 const int32_t* num_tiles, const void* w0, const void* w0_up,
                                 const void* w1, int32_t E_loc, int32_t H, int32_t F, int32_t act,
                                 int32_t tile_m, int64_t R_cap, int64_t tiles_cap, void* act_buf,
                                 float* y_perm, const int32_t* inv_perm, const float* topk_w,
                                 int64_t T, int32_t k, float* out, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * moe_combine -- gather and top-k reduce (section 2.1: expert outputs are
 * gathered back to their tokens and reduced over the top-k choices).
 *
 *   out[t, :] = sum over j = 0..k-1 with inv_perm[t, j] >= 0 of
 *               topk_w[t, j] * y_perm[inv_perm[t, j], :]
 * summed in slot order in fp32; a token with no local slot gets a zero row.
 *   y_perm  [R_cap, H] fp32;  inv_perm [T, k] int32 (values < R_cap or -1);
 *   topk_w  [T, k] fp32;      out [T, H] fp32 out.
 * Requires H % 4 == 0.
 */
moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                       int64_t T, int32_t k, int32_t H, int64_t R_cap, float* out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
