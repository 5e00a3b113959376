// Grouped expert GEMMs with a fused activation epilogue, for gfx950.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts":
//   - section 3.1.2: one GroupGEMM computes all experts of this rank over
//     tile-aligned sub-tensors, tiles holding local tokens first; layer1 runs
//     column block by column block so the reduce can start after the first
//     column blocks;
//   - section 3.1.1: layer0 is decomposed along M (token rows are
//     independent), layer1 along N (the top-k reduce couples rows across
//     experts);
//   - section 4: the MoE GEMMs avoid re-reading row indices from global
//     memory on every K iteration: with the permuted copy a tile needs only
//     its first row and its expert; the gathered layer0 (GATHER) reads each
//     lane's token-row offsets once per work item and keeps them in
//     registers for the whole K loop.
// Tile-level-signalling follow-up (abstract): a persistent kernel covers all
// local experts without relaunches.
//
// Design (MI355X / CDNA4):
//   * Persistent grid of one workgroup per CU the launch stream may use (its
//     CU mask); the work items are (row tile, column block) pairs read from
//     the device tile list, so the host never needs the per-expert row counts.
//   * Workgroup ids are remapped so that each XCD (workgroups are dispatched
//     round-robin over the 8 XCDs) runs a contiguous run of work items: the
//     items an XCD runs together form a small rectangle of row tiles x
//     column blocks whose operand panels are shared through that XCD's L2.
//   * Layer0 order: groups of kGroupM consecutive tiles of the tile list;
//     inside a group, column block major then tile.  Layer1 order: column
//     groups of kGroupN blocks (N-decomposition: a column group is finished
//     for all tiles before the next starts); inside a group, tile major.
//   * Operands are staged HBM -> LDS in stages of BK = 64.  Each LDS row holds
//     64 bf16 (128 B) of one operand row; the 16-byte chunk index is
//     XOR-swizzled with (row & 7) ^ ((row >> 3) & 1), so that the fragment
//     reads (consecutive lanes read consecutive rows at one chunk) hit
//     distinct banks both for 8 lanes within 128 B and for 16 lanes within
//     256 B.  Three load pipelines:
//     - tile_m = 256 (two 64 KiB LDS stages fit): two LDS buffers and
//       register staging; iteration kt writes stage kt+1 from VGPRs into the
//       free buffer while loading the token rows of stage kt+2 and the weight
//       rows of stage kt+3 (two register sets by stage parity) into those
//       VGPRs with plain 16-byte buffer loads (the vector-load path moves
//       more bytes per CU than direct-to-LDS loads when the operands stream
//       from L2);
//     - tile_m = 128: a ring of 3 LDS stages filled by direct-to-LDS loads
//       (buffer_load_dwordx4 ... lds, no VGPR round trip);
//     - small tiles: a ring of 4 LDS stages filled by global_load_lds, the
//       weight rows loaded non-temporal.
//   * Big tiles: the loads of a stage are spread evenly over the K steps of
//     the previous one, between MFMAs (a burst of them right after the
//     barrier backs up the CU's address unit and stalls the issuing waves'
//     matrix cores; a smooth request stream also sees lower L2 latency).
//     Stages past the end load through a buffer resource with no records,
//     so every iteration runs the same schedule.
//   * The stage boundary is software-pipelined: the wait for the next stage,
//     the barrier and the next stage's first fragment reads are issued
//     before the last MFMAs of the current stage, which keep the matrix
//     cores busy meanwhile.  The barrier is a bare s_barrier after explicit
//     waits, so the stages in flight stay in flight across it.
//   * Big tiles (tile_m >= 128): 4 waves (one per SIMD), each owning a
//     128 x 128 (or 64 x 128) accumulator tile of v_mfma_f32_32x32x16_bf16,
//     which keeps LDS traffic per flop at half of the LDS bandwidth.  Small
//     tiles (tile_m <= 64, weight-streaming shapes): 8 waves of
//     v_mfma_f32_16x16x32_bf16.
//   * Operand roles are swapped: the weight tile feeds the MFMA A side
//     (rows = output columns n) and the token tile the B side (columns =
//     token rows m).  Each lane then holds 4 consecutive output columns of
//     one row, so the epilogue stores 8 B (bf16) or 16 B (fp32) vectors.
//   * Epilogue: SwiGLU silu(g) * u, or exact-erf GELU, in fp32, rounded to
//     bf16 (nearest even) for layer0; plain fp32 for layer1.  Rows past the
//     expert's real count are never stored.
//   * Last scheduling round: the items left after the whole rounds run (with
//     a workspace) as up to 8 K slices whose fp32 partials
//     reduce_slices_kernel sums in order before the layer's epilogue
//     (layer0's activation included), else as half-width pieces when those
//     fit in one round, else whole.
//   * Token rows past an expert's real count read as zeros (out-of-range
//     buffer offsets): they fetch nothing and their MFMAs multiply zeros.
#include "common.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int BK = 64;          // K per stage (one 128-byte LDS row per operand row)
constexpr int kGroupM = 8;      // layer0: tiles per rasterisation group
constexpr int kGroupN = 4;      // layer1: column blocks per column group
constexpr int kXcds = 8;
constexpr int MOE_ACT_SWIGLU_I = 1;  // moe_act value of SwiGLU

// EPI_PARTIAL: raw fp32 partial sums of a K slice, the up matrix's (DUAL) in the columns after the gate's.
enum Epi { EPI_GELU = 0, EPI_SWIGLU = 1, EPI_F32 = 2, EPI_PARTIAL = 3 };
enum Order { ORDER_M = 0, ORDER_N = 1 };

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;  // one 16-byte load

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each, far below the
// bf16 rounding that follows).
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}
__device__ __forceinline__ float gelu_f(float h) { return 0.5f * h * (1.0f + erff(h * 0.70710678118654752f)); }

// s_waitcnt with vmcnt = n (0..63) and the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Raw buffer resource over [base, base + bytes): out-of-range reads return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x8 lds_frag(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((chunk ^ swz(row)) << 4));
}

// s_waitcnt lgkmcnt(0), other counters left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier of an LDS ring.  The caller has already waited for its own
// LDS reads (lgkmcnt) and for the direct-to-LDS loads that must have landed
// (vmcnt); the empty asm statements keep the compiler from moving memory
// accesses across the barrier.  __syncthreads() would in addition make the
// compiler wait for every direct-to-LDS load still in flight, draining the
// stages the ring keeps in flight across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most n * per direct-to-LDS loads of this wave are in flight (n small, runtime).
template <int per, int max_n>
__device__ __forceinline__ void wait_stages(int n) {
  if (max_n >= 2 && n >= 2) wait_vmcnt<(max_n >= 2 ? 2 * per : 0)>();
  else if (max_n >= 1 && n >= 1) wait_vmcnt<(max_n >= 1 ? per : 0)>();
  else wait_vmcnt<0>();
}

// Memory operation t of one K step that issues nread fragment reads and nload
// direct-to-LDS loads: the reads first (the next step needs them), then the
// loads; the index of the read (>= 0) or -1 - the index of the load.  The LDS
// reads and the loads stay in program order (the compiler cannot tell they
// touch different buffers), so this is the order they issue in.
__host__ __device__ constexpr int step_slot(int t, int nread, int nload) {
  return t < nread ? t : -1 - (t - nread);
}

// Work item -> (tile index, column block).
template <int ORDER>
__device__ __forceinline__ void item_coords(int64_t item, int nt, int nbn, int& tile_i, int& nb) {
  if (ORDER == ORDER_N) {
    const int64_t per_group = (int64_t)nt * kGroupN;
    const int g = (int)(item / per_group);
    const int rem = (int)(item % per_group);
    const int gsize = (nbn - g * kGroupN) < kGroupN ? (nbn - g * kGroupN) : kGroupN;
    tile_i = rem / gsize;
    nb = g * kGroupN + rem % gsize;
  } else {
    const int64_t per_group = (int64_t)kGroupM * nbn;
    const int grp = (int)(item / per_group);
    const int rem = (int)(item % per_group);
    const int gsize = (nt - grp * kGroupM) < kGroupM ? (nt - grp * kGroupM) : kGroupM;
    nb = rem / gsize;
    tile_i = grp * kGroupM + rem % gsize;
  }
}

__device__ __forceinline__ int xcd_remap(int bid, int G) { return (bid % kXcds) * (G / kXcds) + bid / kXcds; }

// Cache-policy bit of a buffer access that makes a store write through this XCD's L2 (sc1), as the
// compiler emits for an agent-scope atomic store; on a load it is what an agent-scope atomic load uses.
constexpr int kSc1 = 16;

// Epilogue for 4 consecutive output columns of one row.
template <int EPI>
__device__ __forceinline__ void store4(void* C, int64_t row, int N, int n, const float* g, const float* u) {
  static_assert(EPI != EPI_PARTIAL, "partial tiles are stored as two fp32 halves");
  if (EPI == EPI_F32) {
    *reinterpret_cast<floatx4*>(static_cast<float*>(C) + row * N + n) = floatx4{g[0], g[1], g[2], g[3]};
  } else {
    uint16_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = (EPI == EPI_SWIGLU) ? silu_f(g[q]) * u[q] : gelu_f(g[q]);
      h[q] = f2bf_bits(a);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + row * N + n) =
        uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
  }
}

// ---------------------------------------------------------------------------
// Big-tile path: 4 waves (2 x 2), v_mfma_f32_32x32x16_bf16, STAGES-deep LDS ring.
// ---------------------------------------------------------------------------

// One work item: rows [row0, row0 + BM) of expert le (valid of them real) times
// output columns [n0, n0 + BN), reduction over [k_begin, k_begin + k_len).
// Output element (m, n0 + c) goes to C[(c_row0 + m) * ldc + c_n0 + c]; only
// the valid rows are stored.
//
// smem is deliberately not restrict-qualified: a restrict LDS pointer gives
// the LDS accesses alias-scope metadata after inlining, and with it the
// compiler starts matching LDS reads against the direct-to-LDS loads still in
// flight and inserts full vmcnt(0) drains inside the K loop.  The ring is
// synchronised by the explicit waits below instead.
//
// GATHER: A is the token matrix x [T, K] itself and padded row p of the tile
// reads token row_src[p] / topk (row_src < 0: padding, read as zeros) -- the
// layer0 operand gathered on the fly instead of from a permuted copy.
//
// COH: the output is read later in the same launch by workgroups on other
// XCDs, so it is written through L2, in whole lines (staged through LDS).
template <int BM, int BN, bool DUAL, int EPI, int STAGES, bool GATHER, bool COH = false>
__device__ __forceinline__ void gemm_item(char* smem, const uint16_t* __restrict__ A,
                                          const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
                                          int N, int K, int le, int row0, int valid, int n0, int k_begin, int k_len,
                                          void* __restrict__ C, int64_t c_row0, int ldc, int c_n0, int wave,
                                          int lane, const int32_t* __restrict__ row_src, int topk, int64_t T) {
  constexpr int NWAVES = 4, WN = 2;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BROWS = NMAT * BN;               // weight rows staged per stage
  constexpr int A_BYTES = BM * 128, B_BYTES = BROWS * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int WT_M = BM / 2, WT_N = BN / WN;   // wave tile (per matrix)
  constexpr int TM = WT_M / 32, TN = WT_N / 32;
  constexpr int LOADS = (BM + BROWS) / 8 / NWAVES;  // direct-to-LDS loads per wave per stage
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(STAGES >= 2 && STAGES <= 3 && (STAGES - 1) * LOADS < 64, "vmcnt range");
  constexpr int A_PIECES = BM / (8 * NWAVES), B_PIECES = BN / (8 * NWAVES);  // loads per wave: A, each weight matrix
  const int wm = wave / WN, wn = wave % WN;
  const int nk = k_len / BK;
  const int64_t b_expert = (int64_t)N * K;

  // Buffer resources based at this item's operand panels (ranges of a few MiB,
  // out-of-range reads return zeros).  The weight panels share the row stride
  // K, so one per-lane byte offset serves every weight load of this wave:
  // row (q * NWAVES + wave) * 8 + lane / 8, logical chunk swizzled for that row.
  const __amdgpu_buffer_rsrc_t ra = GATHER ? make_rsrc(A, T * K * 2) : make_rsrc(A + (int64_t)row0 * K, BM * K * 2);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + le * b_expert + (int64_t)n0 * K, BN * K * 2);
  const __amdgpu_buffer_rsrc_t rb1 = DUAL ? make_rsrc(B1 + le * b_expert + (int64_t)n0 * K, BN * K * 2) : rb0;
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(A, 0);  // no records: every load reads zero, fetches nothing
  const int r_in = lane >> 3;
  const uint32_t voff = (uint32_t)(((wave * 8 + r_in) * K + (((lane & 7) ^ r_in ^ (wave & 1)) * 8)) * 2);
  // Per A load q, this lane's byte offset: its row of the token panel (GATHER:
  // its token's row of x), same swizzled chunk.  Rows past the expert's real
  // count (GATHER: padding rows) get an offset past every resource, so they
  // read zeros and fetch nothing, and their MFMAs multiply zeros.
  const uint32_t chunk_b = (uint32_t)((((lane & 7) ^ r_in ^ (wave & 1)) * 8) * 2);
  uint32_t voff_a[A_PIECES];
#pragma unroll
  for (int q = 0; q < A_PIECES; ++q) {
    const int r = (q * NWAVES + wave) * 8 + r_in;
    if (GATHER) {
      const int src = row_src[row0 + r];
      const int64_t t = src >= 0 ? src / topk : -1;
      voff_a[q] = (t >= 0 && t < T) ? (uint32_t)(t * K * 2) + chunk_b : 0x80000000u;
    } else {
      voff_a[q] = r < valid ? (uint32_t)(r * K * 2) + chunk_b : 0x80000000u;
    }
  }
  floatx16 acc[NMAT][TN][TM];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][j][i][v] = 0.f;
  // Direct-to-LDS load number p (0 <= p < LOADS, a constant after unrolling)
  // of stage buffer `stage` for K offset k0, through the resources (a, b0, b1)
  // and this lane's byte offset vo (MOE_VOFF(p)): the first A_PIECES stage
  // 8 * NWAVES token rows each, the rest the rows of the weight matrices.
  auto load = [&](int p, int stage, int k0, __amdgpu_buffer_rsrc_t a, __amdgpu_buffer_rsrc_t b0,
                  __amdgpu_buffer_rsrc_t b1, uint32_t vo) {
    const bool is_a = p < A_PIECES;
    const int pb = is_a ? 0 : p - A_PIECES, m = pb / B_PIECES, q = is_a ? p : pb % B_PIECES;
    const int lds_off = (is_a ? 0 : A_BYTES + m * BN * 128) + (q * NWAVES + wave) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a : (m ? b1 : b0), (lds_void*)(smem + stage * STAGE + lds_off), 16,
                                             vo, ((is_a ? 0 : q * 8 * NWAVES * K) + k_begin + k0) * 2, 0, 0);
  };
// Byte offset of this lane for load p: its own row for an A load, else the shared weight-row one.
#define MOE_VOFF(p) ((p) < A_PIECES ? voff_a[(p) < A_PIECES ? (p) : 0] : voff)
  struct Frags {
    bf16x8 a[TM];
    bf16x8 b[NMAT][TN];
  };
  // Fragment read r of K step ks: r < TM the token rows, else weight rows.
  auto read_one = [&](Frags& f, int stage, int ks, int r) {
    const char* sA = smem + stage * STAGE;
    const int chunk = ks * 2 + (lane >> 5);
    if (r < TM) {
      f.a[r] = lds_frag(sA, wm * WT_M + r * 32 + (lane & 31), chunk);
    } else {
      const int m = (r - TM) / TN, j = (r - TM) % TN;
      f.b[m][j] = lds_frag(sA + A_BYTES, m * BN + wn * WT_N + j * 32 + (lane & 31), chunk);
    }
  };
  auto read_frags = [&](int stage, int ks) {
    const char* sA = smem + stage * STAGE;
    const char* sB = sA + A_BYTES;
    const int chunk = ks * 2 + (lane >> 5);
    Frags f;
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = lds_frag(sA, wm * WT_M + i * 32 + (lane & 31), chunk);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < TN; ++j) f.b[m][j] = lds_frag(sB, m * BN + wn * WT_N + j * 32 + (lane & 31), chunk);
    return f;
  };
// MFMAs number [first, first + count) of one 16-wide K step (order: matrix, column block, row block).
#define MOE_MFMAS(F, FIRST, COUNT)                                                                        \
  _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                                        \
  _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                          \
  _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                                        \
  const int idx_ = (m * TN + j) * TM + i;                                                               \
  if (idx_ >= (FIRST) && idx_ < (FIRST) + (COUNT))                                                      \
    acc[m][j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((F).b[m][j], (F).a[i], acc[m][j][i], 0, 0, 0); \
  }
  constexpr int NMFMA = NMAT * TN * TM;   // MFMAs per 16-wide K step
  constexpr int NREAD = TM + NMAT * TN;   // fragment reads per 16-wide K step

  // Direct-to-LDS ring: the loads of one stage are spread evenly over the K
  // steps of the previous stage but its last (which straddles the stage
  // barrier): issued in one burst they back up the CU's address unit, which
  // stalls the issuing waves (and with them their matrix cores) for a large
  // part of the stage, and a smoother request stream also lowers their
  // latency from L2.
  constexpr int SPREAD = BK / 16 - 1;
  constexpr int PER_STEP = (LOADS + SPREAD - 1) / SPREAD;

// K steps of one stage but the last: the next step's fragments are read
// while this step's MFMAs issue; with LD, steps below SPREAD also issue
// their share of the direct-to-LDS loads of stage TS into buffer TBUF
// through (RA, RB0, RB1).
#define MOE_INNER_STEPS(BUF, LD, TBUF, TS, RA, RB0, RB1)                              \
  _Pragma("unroll") for (int ks = 0; ks + 1 < BK / 16; ++ks) {                        \
  const int np_ = (LD) && ks < SPREAD                                               \
                      ? (LOADS - ks * PER_STEP < PER_STEP ? LOADS - ks * PER_STEP : PER_STEP) \
                      : 0;                                                          \
  Frags nxt;                                                                        \
  _Pragma("unroll") for (int t = 0; t < NREAD + np_; ++t) {                         \
    const int sl = step_slot(t, NREAD, np_);                                        \
    if (sl >= 0) read_one(nxt, (BUF), ks + 1, sl);                                  \
    else load(ks * PER_STEP - 1 - sl, (TBUF), (TS) * BK, (RA), (RB0), (RB1), MOE_VOFF(ks * PER_STEP - 1 - sl)); \
  }                                                                                 \
  MOE_MFMAS(cur, 0, NMFMA)                                                          \
  /* Keep this step's MFMAs ahead of the loads that follow them (MFMAs have no */   \
  /* side effects, so without a use here they could drift into later steps). */     \
  if (np_ > 0)                                                                      \
  _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                  \
  _Pragma("unroll") for (int j = 0; j < TN; ++j)                                    \
  _Pragma("unroll") for (int i = 0; i < TM; ++i) asm volatile("" : "+a"(acc[m][j][i])); \
  _Pragma("unroll") for (int t = 0; t < NMFMA || t < NREAD + np_; ++t) {            \
    if (t < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               \
    if (t < NREAD + np_) {                                                          \
      if (step_slot(t, NREAD, np_) >= 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); \
      else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                       \
    }                                                                               \
  }                                                                                 \
  __builtin_amdgcn_sched_barrier(0);                                                \
  cur = nxt;                                                                        \
  }
  Frags cur;
  if constexpr (STAGES == 2) {
  // Two LDS buffers and register-staged loads: iteration kt computes stage
  // kt from buffer kt % 2 while it writes stage kt+1, which arrived in
  // registers earlier, into the other buffer.  Token rows are then reloaded
  // with stage kt+2 (one register set: a whole K stage to land); weight rows,
  // which mostly come from HBM rather than the last-level cache, alternate
  // between two register sets by stage parity and are reloaded with stage
  // kt+3 (two K stages to land).  The LDS writes are spread over the MFMAs,
  // and the plain vector loads move more bytes per CU than direct-to-LDS
  // ones when the tile streams from L2.  Load p of a stage goes to the same
  // LDS place as the direct-to-LDS load p would, so the fragment reads are
  // shared with the ring below.
  constexpr int WP = LOADS - A_PIECES;
  u32x4 stga[A_PIECES > 0 ? A_PIECES : 1];
  u32x4 stgw[2][WP];
  // The writes and loads of a stage are spread evenly over all four K steps
  // of the previous one: PSV per step, NPL of them in the step that straddles
  // the stage barrier (issued with its first half of MFMAs, before the wait).
  constexpr int PSV = (LOADS + BK / 16 - 1) / (BK / 16);
  constexpr int NPL = LOADS - (BK / 16 - 1) * PSV > 0 ? LOADS - (BK / 16 - 1) * PSV : 0;
  auto vload = [&](int p, int set, int k0, __amdgpu_buffer_rsrc_t a, __amdgpu_buffer_rsrc_t b0,
                   __amdgpu_buffer_rsrc_t b1, uint32_t vo) {
    const bool is_a = p < A_PIECES;
    const int pb = is_a ? 0 : p - A_PIECES, m = pb / B_PIECES, q = is_a ? p : pb % B_PIECES;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(is_a ? a : (m ? b1 : b0), vo,
                                                          ((is_a ? 0 : q * 8 * NWAVES * K) + k_begin + k0) * 2, 0);
    if (is_a) stga[p] = v; else stgw[set][pb] = v;
  };
  auto vwrite = [&](int p, int set, int buf) {
    const bool is_a = p < A_PIECES;
    const int pb = is_a ? 0 : p - A_PIECES, m = pb / B_PIECES, q = is_a ? p : pb % B_PIECES;
    const int lds_off = (is_a ? 0 : A_BYTES + m * BN * 128) + (q * NWAVES + wave) * 1024;
    *reinterpret_cast<u32x4*>(smem + buf * STAGE + lds_off + lane * 16) = is_a ? stga[p] : stgw[set][pb];
  };
  // Prologue: stage 0 into buffer 0, stage 1 into the registers (weights: set 1), stage 2's weights into set 0.
#pragma unroll
  for (int p = 0; p < LOADS; ++p) vload(p, 0, 0, ra, rb0, rb1, MOE_VOFF(p));
#pragma unroll
  for (int p = 0; p < LOADS; ++p) vwrite(p, 0, 0);
#pragma unroll
  for (int p = 0; p < LOADS; ++p)
    vload(p, 1, BK, 1 < nk ? ra : rnone, 1 < nk ? rb0 : rnone, 1 < nk ? rb1 : rnone, MOE_VOFF(p));
#pragma unroll
  for (int p = A_PIECES; p < LOADS; ++p) vload(p, 0, 2 * BK, ra, 2 < nk ? rb0 : rnone, 2 < nk ? rb1 : rnone, voff);
  wait_lgkm0();
  ring_barrier();
  cur = read_frags(0, 0);
  // Piece p of stage kt+1 goes from registers to LDS buffer WB (weights from set WB, the parity of kt+1), then
  // its registers reload: tokens stage kt+2 through (RA, RB0, RB1), weights stage kt+3 through (RB0W, RB1W).
  auto piece = [&](int p, int wb, int kt, __amdgpu_buffer_rsrc_t RA, __amdgpu_buffer_rsrc_t RB0,
                   __amdgpu_buffer_rsrc_t RB1, __amdgpu_buffer_rsrc_t RB0W, __amdgpu_buffer_rsrc_t RB1W) {
    vwrite(p, wb, wb);
    if (p < A_PIECES) vload(p, wb, (kt + 2) * BK, RA, RB0, RB1, MOE_VOFF(p));
    else vload(p, wb, (kt + 3) * BK, RA, RB0W, RB1W, MOE_VOFF(p));
  };
#define MOE_INNER_STEPS_VL(BUF, WBUF, KT, RA, RB0, RB1, RB0W, RB1W)                    \
  _Pragma("unroll") for (int ks = 0; ks + 1 < BK / 16; ++ks) {                        \
  const int np_ = LOADS - ks * PSV < PSV ? LOADS - ks * PSV : PSV;                  \
  Frags nxt;                                                                        \
  _Pragma("unroll") for (int t = 0; t < NREAD; ++t) read_one(nxt, (BUF), ks + 1, t); \
  _Pragma("unroll") for (int t = 0; t < np_; ++t)                                   \
    piece(ks * PSV + t, (WBUF), (KT), (RA), (RB0), (RB1), (RB0W), (RB1W));          \
  MOE_MFMAS(cur, 0, NMFMA)                                                          \
  if (np_ > 0)                                                                      \
  _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                  \
  _Pragma("unroll") for (int j = 0; j < TN; ++j)                                    \
  _Pragma("unroll") for (int i = 0; i < TM; ++i) asm volatile("" : "+a"(acc[m][j][i])); \
  _Pragma("unroll") for (int t = 0; t < NMFMA + NREAD + 2 * LOADS; ++t) {          \
    if (t < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               \
    if (t < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               \
    else if (t < NREAD + 2 * np_) {                                                 \
      if ((t - NREAD) % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  \
      else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                       \
    }                                                                               \
  }                                                                                 \
  __builtin_amdgcn_sched_barrier(0);                                                \
  cur = nxt;                                                                        \
  }
  // Iteration kt, whose parity is the constant `par`: computes stage kt from buffer par.
  auto iter = [&](auto par, int kt) {
    constexpr int buf = decltype(par)::value, wbuf = buf ^ 1;
    const bool real = kt + 2 < nk, real3 = kt + 3 < nk;
    const __amdgpu_buffer_rsrc_t RA = real ? ra : rnone, RB0 = real ? rb0 : rnone, RB1 = real ? rb1 : rnone;
    const __amdgpu_buffer_rsrc_t RB0W = real3 ? rb0 : rnone, RB1W = real3 ? rb1 : rnone;
    MOE_INNER_STEPS_VL(buf, wbuf, kt, RA, RB0, RB1, RB0W, RB1W)
    constexpr int P0 = (BK / 16 - 1) * PSV;
#pragma unroll
    for (int t = 0; t < NPL; ++t) piece(P0 + t, wbuf, kt, RA, RB0, RB1, RB0W, RB1W);
    MOE_MFMAS(cur, 0, NMFMA / 2)
    if (NPL > 0)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TM; ++i) asm volatile("" : "+a"(acc[m][j][i]));
#pragma unroll
    for (int t = 0; t < NMFMA / 2 || t < 2 * NPL; ++t) {
      if (t < NMFMA / 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t < 2 * NPL) {
        if (t % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();     // this wave's reads of stage kt and writes of stage kt+1 are complete
    ring_barrier();   // stage kt+1 visible to all; buffer kt % 2 is free from the next iteration on
    __builtin_amdgcn_sched_barrier(0);
    const Frags nxt = read_frags(wbuf, 0);
    MOE_MFMAS(cur, NMFMA / 2, NMFMA - NMFMA / 2)
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  };
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    iter(std::integral_constant<int, 0>{}, kt);
    iter(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt + 1 < nk) iter(std::integral_constant<int, 0>{}, kt);
#undef MOE_INNER_STEPS_VL
  } else {
  // STAGES-deep ring of direct-to-LDS loads: the prologue loads stages 0 .. STAGES-2; iteration kt
  // (computing stage kt) loads stage kt + STAGES - 1 into buffer
  // (kt - 1) mod STAGES, which every wave has finished reading at the barrier
  // that ended iteration kt - 1 (and which the prologue left empty for
  // kt = 0).  A stage past the end is "loaded" through resources with no
  // records: every lane reads zero, nothing is fetched, and the zeros land in
  // that free buffer, so the schedule is the same in every iteration.
#pragma unroll
  for (int st = 0; st + 1 < STAGES; ++st)
    if (st < nk)
#pragma unroll
      for (int p = 0; p < LOADS; ++p) load(p, st, st * BK, ra, rb0, rb1, MOE_VOFF(p));
  {  // stage 0 has landed once only the prologue's later stages are in flight
    const int later = (nk < STAGES - 1 ? nk : STAGES - 1) - 1;
    wait_stages<LOADS, STAGES - 2>(later);
  }
  ring_barrier();
  cur = read_frags(0, 0);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int buf = kt % STAGES;
    const int ts = kt + STAGES - 1;
    const bool real = ts < nk;
    MOE_INNER_STEPS(buf, true, (kt + STAGES - 1) % STAGES, ts, real ? ra : rnone, real ? rb0 : rnone,
                    real ? rb1 : rnone)
    // Last K step of the stage: half of its MFMAs keep the matrix cores busy
    // across the stage boundary.
    MOE_MFMAS(cur, 0, NMFMA / 2)
    __builtin_amdgcn_sched_barrier(0);
    // Stage kt+1 has landed once only the STAGES - 2 load groups issued after
    // it (one per iteration) are in flight.
    wait_vmcnt<(STAGES - 2) * LOADS>();
    wait_lgkm0();     // this wave's reads of stage kt are complete
    ring_barrier();   // stage kt+1 visible to all; buffer kt is free from the next iteration on
    __builtin_amdgcn_sched_barrier(0);
    const Frags nxt = read_frags((kt + 1) % STAGES, 0);
    MOE_MFMAS(cur, NMFMA / 2, NMFMA - NMFMA / 2)
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
  }
  {  // the last stage
    const int buf = (nk - 1) % STAGES;
    MOE_INNER_STEPS(buf, false, 0, 0, ra, rb0, rb1)
    MOE_MFMAS(cur, 0, NMFMA)
  }
#undef MOE_INNER_STEPS
#undef MOE_VOFF
#undef MOE_MFMAS

  // Epilogue: lane holds, for token row m = lane % 32 of each 32-row block,
  // output columns q*8 + (lane/32)*4 + 0..3 (q = 0..3) of each 32-column block.
  if constexpr (COH) {
    // Results for consumers on other XCDs are written through L2.  A write-through store that covers
    // only part of a 128-byte line is completed by a read-modify-write at the memory side, so the tile
    // is first laid out row-major in LDS (the ring is free once every wave is past its last K step)
    // and then stored 16 bytes per lane along whole rows: a wavefront covers 1 KiB of one fp32 row
    // (or four 256-byte bf16 rows) per store, whole lines only.
    static_assert(!(COH && DUAL && EPI == EPI_PARTIAL), "no split-K pieces of the dual layer here");
    constexpr int ES = (EPI == EPI_F32 || EPI == EPI_PARTIAL) ? 4 : 2;  // output element bytes
    constexpr int PITCH = BN * ES + 16;                                 // LDS row pitch (bank offset)
    constexpr int RING = STAGES * STAGE;
    constexpr int RP = 256 * PITCH <= RING ? 256 : 128 * PITCH <= RING ? 128 : 64 * PITCH <= RING ? 64 : 32;
    static_assert(RP * PITCH <= RING && RP % 32 == 0 && (BM % RP) == 0, "staging pass fits the ring");
    constexpr int CPR = BN * ES / 16;  // 16-byte chunks per output row
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(static_cast<char*>(C) + (c_row0 * ldc + c_n0) * ES, (int64_t)(BM - 1) * ldc * ES + BN * ES);
    __syncthreads();  // every wave is done reading the ring
#pragma unroll
    for (int p0 = 0; p0 < BM; p0 += RP) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int mb = wm * WT_M + i * 32;  // first row of this 32-row block
        if (mb < p0 || mb >= p0 + RP) continue;  // wave-uniform
        const int ml = mb - p0 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = wn * WT_N + j * 32 + q * 8 + (lane >> 5) * 4;
            char* d = smem + ml * PITCH + n * ES;
            if constexpr (ES == 4) {
              *reinterpret_cast<floatx4*>(d) =
                  floatx4{acc[0][j][i][q * 4], acc[0][j][i][q * 4 + 1], acc[0][j][i][q * 4 + 2], acc[0][j][i][q * 4 + 3]};
            } else {
              uint16_t h[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float g = acc[0][j][i][q * 4 + r], u = acc[NMAT - 1][j][i][q * 4 + r];
                h[r] = f2bf_bits(EPI == EPI_SWIGLU ? silu_f(g) * u : gelu_f(g));
              }
              *reinterpret_cast<uint2*>(d) =
                  uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
            }
          }
      }
      __syncthreads();
      for (int c = threadIdx.x; c < RP * CPR; c += NWAVES * 64) {
        const int r = c / CPR, cc = c % CPR;
        if (p0 + r >= valid) break;  // rows are visited in order; the rest of this pass is padding
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * PITCH + cc * 16);
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, (p0 + r) * ldc * ES + cc * 16, 0, kSc1);
      }
      __syncthreads();  // the next pass rewrites the staging rows
    }
  } else {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WT_M + i * 32 + (lane & 31);
    if (m >= valid) continue;
    const int64_t row = c_row0 + m;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = c_n0 + wn * WT_N + j * 32 + q * 8 + (lane >> 5) * 4;
        float g[4], u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g[r] = acc[0][j][i][q * 4 + r];
          u[r] = acc[NMAT - 1][j][i][q * 4 + r];
        }
        if constexpr (EPI == EPI_PARTIAL) {
          store4<EPI_F32>(C, row, ldc, n, g, g);
          if (NMAT == 2) store4<EPI_F32>(C, row, ldc, n + BN, u, u);
        } else {
          store4<EPI>(C, row, ldc, n, g, u);
        }
      }
  }
  }
  wait_vmcnt<0>();  // epilogue stores retired before the next item's load accounting
  __syncthreads();  // the next item's first stages overwrite LDS
}

template <int BM, int BN, bool DUAL>
constexpr int big_lds_bytes(int stages) {
  return stages * (BM + (DUAL ? 2 : 1) * BN) * 128;
}

// Number of K slices of each last-round item (1 = no split) when the rem
// items left after the whole rounds are split along K: as many slices as fit
// in one round of G workgroups, at most kMaxSlices and at most the nk stages
// of K.  Slice s covers stages [s * nk / S, (s + 1) * nk / S).
constexpr int kMaxSlices = 8;
__host__ __device__ inline int tail_ksplit(int64_t rem, int G, int nk) {
  if (rem <= 0) return 1;
  int64_t S = G / rem;
  S = S > kMaxSlices ? kMaxSlices : S;
  S = S > nk ? nk : S;
  return S < 1 ? 1 : (int)S;
}

// Persistent kernel over (row tile, column block) items.  With G workgroups
// and W items, the first floor(W / G) * G items run whole (every workgroup
// gets the same number).  The remaining items run in one more round:
//  * with SPLITK and S = tail_ksplit > 1, each is split into S slices of K
//    whose fp32 partial tiles go to ws (piece p at ws + p * BM * NMAT * BN,
//    row-major, the up matrix's columns after the gate's);
//    reduce_slices_kernel sums them in slice order afterwards (and applies
//    layer0's activation), so the result is deterministic;
//  * otherwise, if the two half-width pieces of each fit in one round (at
//    most G / 2 items left), they run as such pieces; else (more than G / 2
//    items left and no split) the items run whole in one last round.
// The last round then costs a fraction of a full item instead of leaving
// most CUs idle behind a few full ones, or at most one full item.
template <int BM, int BN, bool DUAL, int EPI, int ORDER, int STAGES, bool SPLITK, bool GATHER>
__global__ __launch_bounds__(256, 1) void gemm_mfma32_kernel(
    const uint16_t* __restrict__ A,    // [R_cap, K] bf16 (x_perm or act)
    const uint16_t* __restrict__ B0,   // [E_loc, N, K] bf16
    const uint16_t* __restrict__ B1,   // [E_loc, N, K] bf16 (DUAL) or null
    int N, int K, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int64_t tiles_cap,
    int64_t R_cap, int E_loc, void* __restrict__ C, float* __restrict__ ws, const int32_t* __restrict__ row_src,
    int topk, int64_t T) {
  __shared__ __attribute__((aligned(1024))) char smem[big_lds_bytes<BM, BN, DUAL>(STAGES)];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  const int vid = xcd_remap(blockIdx.x, G);
  int nt = *num_tiles;
  if (nt > tiles_cap) nt = (int)tiles_cap;
  const int nbn = N / BN;
  const int64_t total = (int64_t)nt * nbn;
  const int64_t full = total / G * G;  // items run whole
  const int S = SPLITK ? tail_ksplit(total - full, G, K / BK) : 1;

  // Item -> (expert, first row, real rows, first column); false if the tile entry is inconsistent.
  auto coords = [&](int64_t item, int& le, int& row0, int& valid, int& n0) {
    int tile_i, nb;
    item_coords<ORDER>(item, nt, nbn, tile_i, nb);
    le = tiles[2 * tile_i];
    row0 = tiles[2 * tile_i + 1];
    if (le < 0 || le >= E_loc || row0 < 0 || (int64_t)row0 + BM > R_cap) return false;
    valid = counts[le] - (row0 - offsets[le]);
    valid = valid < BM ? valid : BM;
    n0 = nb * BN;
    return true;
  };

  for (int64_t item = vid; item < full; item += G) {
    int le, row0, valid, n0;
    if (!coords(item, le, row0, valid, n0)) continue;  // block-uniform
    gemm_item<BM, BN, DUAL, EPI, STAGES, GATHER>(smem, A, B0, B1, N, K, le, row0, valid, n0, 0, K, C, row0, N, n0,
                                                 wave, lane, row_src, topk, T);
  }
  if (S > 1) {
    constexpr int PIECE = BM * (DUAL ? 2 : 1) * BN;  // floats per partial tile
    const int nk = K / BK;
    for (int64_t piece = vid; piece < S * (total - full); piece += G) {
      int le, row0, valid, n0;
      if (!coords(full + piece / S, le, row0, valid, n0)) continue;
      const int s = (int)(piece % S), kb = s * nk / S, ke = (s + 1) * nk / S;
      gemm_item<BM, BN, DUAL, EPI_PARTIAL, STAGES, GATHER>(smem, A, B0, B1, N, K, le, row0, valid, n0, kb * BK,
                                                           (ke - kb) * BK, ws + piece * (int64_t)PIECE, 0,
                                                           (DUAL ? 2 : 1) * BN, 0, wave, lane, row_src, topk, T);
    }
    return;
  }
  if (2 * (total - full) > G) {  // the pieces would take two rounds: one round of whole items is shorter
    for (int64_t item = full + vid; item < total; item += G) {
      int le, row0, valid, n0;
      if (!coords(item, le, row0, valid, n0)) continue;
      gemm_item<BM, BN, DUAL, EPI, STAGES, GATHER>(smem, A, B0, B1, N, K, le, row0, valid, n0, 0, K, C, row0, N, n0,
                                                   wave, lane, row_src, topk, T);
    }
    return;
  }
  for (int64_t piece = vid; piece < 2 * (total - full); piece += G) {
    int le, row0, valid, n0;
    if (!coords(full + piece / 2, le, row0, valid, n0)) continue;
    const int nh = n0 + (int)(piece % 2) * (BN / 2);
    gemm_item<BM, BN / 2, DUAL, EPI, STAGES, GATHER>(smem, A, B0, B1, N, K, le, row0, valid, nh, 0, K, C, row0, N,
                                                     nh, wave, lane, row_src, topk, T);
  }
}

// Sums the K slices that gemm_mfma32_kernel<..., SPLITK> left in ws for its
// last-round items (same G, tile list and shapes), slice by slice in order,
// and stores the valid rows through the layer's epilogue EPI (fp32 for
// layer1; the activation, rounded to bf16, for layer0, whose DUAL partial
// tiles hold the up matrix's columns after the gate's).  Block b covers rows
// [(b % (BM / RB)) * RB, + RB) of unit b / (BM / RB); launched with
// G * BM / RB blocks of 256 threads.
template <int BM, int BN, bool DUAL, int EPI, int ORDER>
__global__ __launch_bounds__(256) void reduce_slices_kernel(const float* __restrict__ ws, int N, int K, int G,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ tiles,
                                                            const int32_t* __restrict__ num_tiles, int64_t tiles_cap,
                                                            int64_t R_cap, int E_loc, void* __restrict__ C) {
  constexpr int RB = 16;
  int nt = *num_tiles;
  if (nt > tiles_cap) nt = (int)tiles_cap;
  const int nbn = N / BN;
  const int64_t total = (int64_t)nt * nbn, full = total / G * G;
  const int S = tail_ksplit(total - full, G, K / BK);
  const int64_t u = blockIdx.x / (BM / RB);
  const int rc = blockIdx.x % (BM / RB);
  if (S <= 1 || u >= total - full) return;  // block-uniform
  int tile_i, nb;
  item_coords<ORDER>(full + u, nt, nbn, tile_i, nb);
  const int le = tiles[2 * tile_i], row0 = tiles[2 * tile_i + 1];
  if (le < 0 || le >= E_loc || row0 < 0 || (int64_t)row0 + BM > R_cap) return;
  int valid = counts[le] - (row0 - offsets[le]);
  valid = valid < BM ? valid : BM;
  constexpr int NMAT = DUAL ? 2 : 1, W4 = NMAT * BN / 4;  // float4 groups per partial row
  const floatx4* part = reinterpret_cast<const floatx4*>(ws + u * S * (int64_t)(BM * NMAT * BN));
  for (int e = threadIdx.x; e < RB * (BN / 4); e += 256) {
    const int m = rc * RB + e / (BN / 4), c4 = e % (BN / 4);
    if (m >= valid) continue;
    const int idx = m * W4 + c4;
    floatx4 g4 = part[idx], u4 = part[idx + (NMAT - 1) * (BN / 4)];
    for (int q = 1; q < S; ++q) {
      g4 += part[q * (BM * W4) + idx];
      if (DUAL) u4 += part[q * (BM * W4) + idx + BN / 4];
    }
    const float g[4] = {g4[0], g4[1], g4[2], g4[3]}, uu[4] = {u4[0], u4[1], u4[2], u4[3]};
    store4<EPI>(C, (int64_t)row0 + m, N, nb * BN + c4 * 4, g, uu);
  }
}

// ---------------------------------------------------------------------------
// One persistent launch for layer0 -> activation -> layer1 -> top-k combine, with tile-level signals.
//
// Comet section 3.1.2: layer1's N-decomposed reduction can start after its first column blocks;
// tile-level-signalling follow-up (abstract): tiles are signalled as they become ready instead of
// waiting for whole kernels.  Here the work items form one global order: all layer0 items (256-row
// tile x 128 columns of F, the unfused order), then layer1 items (tile x 256 columns of H, column groups
// of kGroupN blocks first), then the K slices of the last layer1 items (as many as the unfused layer1
// would leave for its last round), then combine items (64 tokens x one column group, group by group).
// Each XCD's workgroups take that order's items from a queue of their own (a device counter per XCD;
// see the kernel), each queue in increasing order.  Signals:
//   ready[tile]   layer0 items of the tile done; a layer1 item waits for F / 128 of them;
//   group[g]      layer1 items (a split item counting once, when its last slice has reduced) of column
//                 group g done; a combine item waits for num_tiles x (blocks of g) of them;
//   slices[u]     K slices of split item u done; the one that brings it to S sums all S in slice order.
// Every wait ends: an item only waits for items earlier in the global order, and the earliest item held
// by a waiting workgroup waits for one that is done, running, or not yet taken from its queue -- and then
// every workgroup on that queue's XCD holds an earlier item, so none of them waits and the queue moves on
// (all workgroups are resident: one per CU).  Each wait is still bounded (on time-out the error word is
// set and the item proceeds, giving wrong values rather than a hang).
// Visibility across XCDs without an L2 write-back: every result another workgroup reads (activations,
// layer1 rows, partial slices) is written through L2 in whole lines (gemm_item's COH epilogue); the
// producer waits for its stores, synchronises its workgroup and then increments the counter; the
// consumer polls with device-scope loads and then reads the data, which its own L2 and L1 have not held
// since the launch began (each row range is produced once and read only after its signal).  The last
// workgroup to finish returns every counter it used to zero for the next launch.
// ---------------------------------------------------------------------------
constexpr int kCombineTokens = 64;
constexpr int kCombineWin = 32;     // y rows in flight per thread in a combine item
constexpr int kMaxTopk = 32;      // the entry point's limit on k
constexpr int64_t kSpinLimit = 1 << 20;

struct FusedCounters {
  int err;            // nonzero: a wait timed out (the launch's results are not valid); cleared by the caller
  int done;           // workgroups finished
  int pad[2];
  int next[kXcds];    // next work item of each XCD's queue
};

// Thread 0: poll *p (device-scope loads) until it reaches target; false (and the error word set) on time-out.
__device__ __forceinline__ bool wait_count(int* p, int target, int* err) {
  for (int64_t it = 0;; ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    if (it >= kSpinLimit) {
      __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// After the workgroup's write-through stores: every wave waits for its own, then thread 0 signals.
__device__ __forceinline__ int publish(int* p) {
  wait_vmcnt<0>();
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

template <bool DUAL, int EPI0>
__global__ __launch_bounds__(256, 1) void ffn_fused_kernel(
    const uint16_t* __restrict__ x_perm, const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w0_up,
    const uint16_t* __restrict__ w1, int H, int F, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    int64_t tiles_cap, int64_t R_cap, int E_loc, uint16_t* __restrict__ act, float* __restrict__ y,
    const int32_t* __restrict__ inv_perm, const float* __restrict__ topk_w, int64_t T, int topk,
    float* __restrict__ out, FusedCounters* __restrict__ ctr, int* __restrict__ ready, int* __restrict__ group,
    int* __restrict__ slices, float* __restrict__ part) {
  constexpr int BM = 256, BN0 = 128, BN1 = 256;
  __shared__ __attribute__((aligned(1024))) char smem[big_lds_bytes<BM, BN1, false>(2)];
  static_assert(big_lds_bytes<BM, BN0, DUAL>(2) <= big_lds_bytes<BM, BN1, false>(2), "layer0 stages fit");
  __shared__ int s_item, s_flag;
  __shared__ int s_row[kCombineTokens * kMaxTopk];
  __shared__ float s_w[kCombineTokens * kMaxTopk];
  __shared__ uint8_t s_tok[kCombineTokens * kMaxTopk];
  __shared__ int s_cnt[kCombineTokens], s_beg[kCombineTokens], s_nslot;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  int nt = *num_tiles;
  if (nt > tiles_cap) nt = (int)tiles_cap;
  const int nb0 = F / BN0, nb1 = H / BN1;
  const int ngroups = (nb1 + kGroupN - 1) / kGroupN;
  const int64_t W0 = (int64_t)nt * nb0, W1 = (int64_t)nt * nb1;
  const int64_t R1 = W1 % G;                                  // items the unfused layer1 leaves for its last round
  const int S = R1 > 0 ? tail_ksplit(R1, G, F / BK) : 1;
  const int64_t W1w = S > 1 ? W1 - R1 : W1;                   // layer1 items run whole
  const int64_t P1 = S > 1 ? R1 * S : 0;                      // their K slices
  const int64_t TC = (T + kCombineTokens - 1) / kCombineTokens;
  const int64_t total = W0 + W1w + P1 + TC * ngroups;

  auto tile_of = [&](int tile_i, int& le, int& row0, int& valid) {
    le = tiles[2 * tile_i];
    row0 = tiles[2 * tile_i + 1];
    if (le < 0 || le >= E_loc || row0 < 0 || (int64_t)row0 + BM > R_cap) return false;
    valid = counts[le] - (row0 - offsets[le]);
    valid = valid < BM ? valid : BM;
    return true;
  };
  // Layer1 item u's tile, column block and column group; waits for the tile's activations.
  auto layer1_coords = [&](int64_t u, int& tile_i, int& nb) {
    item_coords<ORDER_N>(u, nt, nb1, tile_i, nb);
    if (threadIdx.x == 0) wait_count(&ready[tile_i], nb0, &ctr->err);
    __syncthreads();
  };

  // Each XCD (workgroups b with b % 8 == x, dispatched round-robin over the XCDs) has its own queue: its
  // k-th item is item (k / C) * G + x * C + k % C (C = G / 8), so in every round of G items it runs a
  // contiguous run of C of them, the rectangle of row tiles x column blocks that shares operand panels
  // in its L2 (the unfused kernels' item placement), and each queue runs in increasing item order.
  const int xq = blockIdx.x % kXcds, C = G / kXcds;
  for (;;) {
    if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(&ctr->next[xq], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t kq = s_item;
    const int64_t item = kq / C * G + (int64_t)xq * C + kq % C;
    __syncthreads();
    if (item >= total) break;
    if (item < W0) {  // layer0: activations of a tile's 128 columns
      int tile_i, nb, le, row0, valid;
      item_coords<ORDER_M>(item, nt, nb0, tile_i, nb);
      if (tile_of(tile_i, le, row0, valid))
        gemm_item<BM, BN0, DUAL, EPI0, 2, false, true>(smem, x_perm, w0, w0_up, F, H, le, row0, valid, nb * BN0, 0, H,
                                                      act, row0, F, nb * BN0, wave, lane, nullptr, 0, 0);
      publish(&ready[tile_i]);
    } else if (item < W0 + W1w) {  // layer1, whole item
      int tile_i, nb, le, row0, valid;
      layer1_coords(item - W0, tile_i, nb);
      if (tile_of(tile_i, le, row0, valid))
        gemm_item<BM, BN1, false, EPI_F32, 2, false, true>(smem, act, w1, nullptr, H, F, le, row0, valid, nb * BN1, 0,
                                                          F, y, row0, H, nb * BN1, wave, lane, nullptr, 0, 0);
      publish(&group[nb / kGroupN]);
    } else if (item < W0 + W1w + P1) {  // layer1, one K slice of a split item
      const int64_t pc = item - W0 - W1w, u = pc / S;
      const int s = (int)(pc % S), nk = F / BK, kb = s * nk / S, ke = (s + 1) * nk / S;
      int tile_i, nb, le, row0, valid;
      layer1_coords(W1w + u, tile_i, nb);
      const bool ok = tile_of(tile_i, le, row0, valid);
      if (ok)
        gemm_item<BM, BN1, false, EPI_PARTIAL, 2, false, true>(smem, act, w1, nullptr, H, F, le, row0, valid,
                                                              nb * BN1, kb * BK, (ke - kb) * BK,
                                                              part + pc * (int64_t)(BM * BN1), 0, BN1, 0, wave, lane,
                                                              nullptr, 0, 0);
      const int old = publish(&slices[u]);
      if (threadIdx.x == 0) s_flag = old;
      __syncthreads();
      if (s_flag == S - 1) {  // the last slice of item u: sum the S slices in order, store the rows, signal
        if (ok) {
          // 16-byte accesses along whole rows, written through (whole lines, as in the tile epilogue).
          const __amdgpu_buffer_rsrc_t rp = make_rsrc(part + u * S * (int64_t)(BM * BN1), (int64_t)S * BM * BN1 * 4);
          const __amdgpu_buffer_rsrc_t ry =
              make_rsrc(y + (int64_t)row0 * H + nb * BN1, (int64_t)(BM - 1) * H * 4 + BN1 * 4);
          for (int e = threadIdx.x; e < valid * (BN1 / 4); e += 256) {
            const int m = e / (BN1 / 4), c4 = e % (BN1 / 4);
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int q = 0; q < S; ++q)
              acc += __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rp, (q * (BM * BN1) + m * BN1 + c4 * 4) * 4, 0, kSc1));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ry, (m * H + c4 * 4) * 4, 0, kSc1);
          }
        }
        publish(&group[nb / kGroupN]);
      }
    } else {  // combine: kCombineTokens tokens x one column group
      const int64_t c = item - W0 - W1w - P1;
      const int g = (int)(c / TC);
      const int64_t t0 = (c % TC) * kCombineTokens;
      const int nt_c = (int)(T - t0 < kCombineTokens ? T - t0 : kCombineTokens);
      const int gsize = (nb1 - g * kGroupN) < kGroupN ? (nb1 - g * kGroupN) : kGroupN;
      // While the group's layer1 items finish: the item's local slots, compacted in token and slot order
      // (row, weight, token), so that the reads below keep kCombineWin rows in flight whatever the share
      // of non-local slots.
      // Thread t < kCombineTokens holds token t0 + t's slots in registers (all its loads in flight at once).
      const int tt = threadIdx.x;
      const bool own = tt < nt_c;
      int pr[kMaxTopk];
      float pw[kMaxTopk];
      int n = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopk; ++j) {
        pr[j] = -1;
        pw[j] = 0.f;
        if (own && j < topk) {
          const int v = inv_perm[(t0 + tt) * topk + j];
          pr[j] = (v >= 0 && v < R_cap) ? v : -1;
          pw[j] = topk_w[(t0 + tt) * topk + j];
        }
        n += pr[j] >= 0;
      }
      if (tt < kCombineTokens) s_cnt[tt] = n;
      __syncthreads();
      if (threadIdx.x == 0) {
        int run = 0;
        for (int t = 0; t < kCombineTokens; ++t) {
          s_beg[t] = run;
          run += s_cnt[t];
        }
        s_nslot = run;
      }
      __syncthreads();
      if (own) {
        int o = s_beg[tt];
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j)
          if (pr[j] >= 0) {
            s_row[o] = pr[j];
            s_w[o] = pw[j];
            s_tok[o] = (uint8_t)tt;
            ++o;
          }
      }
      if (threadIdx.x == 0) wait_count(&group[g], nt * gsize, &ctr->err);
      __syncthreads();
      const int col = g * kGroupN * BN1 + threadIdx.x * 4;  // this thread's float4 column of the group
      if (threadIdx.x * 4 < gsize * BN1) {
        for (int t = 0; t < nt_c; ++t)  // tokens with no local slot
          if (s_cnt[t] == 0) *reinterpret_cast<floatx4*>(out + (t0 + t) * H + col) = floatx4{0.f, 0.f, 0.f, 0.f};
        const int ns = s_nslot;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < ns; s0 += kCombineWin) {
          floatx4 v[kCombineWin];
#pragma unroll
          for (int q = 0; q < kCombineWin; ++q)
            v[q] = s0 + q < ns ? *reinterpret_cast<const floatx4*>(y + (int64_t)s_row[s0 + q] * H + col)
                               : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < kCombineWin; ++q) {
            const int sq = s0 + q;
            if (sq < ns) {
              acc += s_w[sq] * v[q];  // each token's slots in slot order
              const int tq = s_tok[sq];
              if (sq + 1 == ns || s_tok[sq + 1] != tq) {
                *reinterpret_cast<floatx4*>(out + (t0 + tq) * H + col) = acc;
                acc = floatx4{0.f, 0.f, 0.f, 0.f};
              }
            }
          }
        }
      }
      __syncthreads();  // the slot lists are rewritten by the next combine item
    }
  }
  // The last workgroup to finish resets the counters of this launch for the next one.
  if (threadIdx.x == 0) {
    const int d = __hip_atomic_fetch_add(&ctr->done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = d;
  }
  __syncthreads();
  if (s_flag == G - 1) {
    for (int64_t i = threadIdx.x; i < nt; i += 256) ready[i] = 0;
    for (int i = threadIdx.x; i < ngroups; i += 256) group[i] = 0;
    for (int64_t i = threadIdx.x; i < R1; i += 256) slices[i] = 0;
    if (threadIdx.x < kXcds) ctr->next[threadIdx.x] = 0;
    if (threadIdx.x == 0) ctr->done = 0;
  }
}

// ---------------------------------------------------------------------------
// Small-tile kernel (tile_m <= 64): WM x WN waves of v_mfma_f32_16x16x32_bf16,
// a 4-stage LDS ring of direct-to-LDS loads (three stages in flight while one
// is computed).  These shapes stream weights from HBM.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool DUAL, int EPI, int ORDER, bool GATHER>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_mfma16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    int N, int K, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int64_t tiles_cap,
    int64_t R_cap, int E_loc, void* __restrict__ C, const int32_t* __restrict__ row_src, int topk, int64_t T) {
  constexpr int NWAVES = WM * WN;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BROWS = NMAT * BN;
  constexpr int A_BYTES = BM * 128, B_BYTES = BROWS * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int WT_M = BM / WM, WT_N = BN / WN;
  constexpr int TM = WT_M / 16, TN = WT_N / 16;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(BM % 8 == 0 && BROWS % 8 == 0, "rows per stage");
  static_assert(BM / 8 <= NWAVES, "token rows: at most one 8-row group per wave");
  static_assert((BN / 8) % NWAVES == 0, "weight rows: the same number of 8-row groups on every wave");
  // Ring of SR stages: SR - 1 stages of weights stream in while one is computed.
  constexpr int SR = 4;
  constexpr int LW_B = NMAT * (BN / 8 / NWAVES);  // direct-to-LDS loads per wave per stage (weights)

  __shared__ __attribute__((aligned(1024))) char smem[SR * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int G = gridDim.x;
  const int vid = xcd_remap(blockIdx.x, G);

  int nt = *num_tiles;
  if (nt > tiles_cap) nt = (int)tiles_cap;
  const int nbn = N / BN;
  const int64_t total = (int64_t)nt * nbn;
  const int nk = K / BK;
  const int64_t b_expert = (int64_t)N * K;

  // rows per stage may not be a multiple of 8 * NWAVES: guard per 8-row group.
  // Weight rows are read once per launch at these shapes: they are loaded
  // non-temporal (streaming), which lets a read-only stream run near the HBM
  // peak instead of settling around 6 TB/s.
  auto stage_any = [&](const uint16_t* g, int rows, char* lds, bool stream) {
    const int r_in = lane >> 3;
    for (int grp = wave; grp < rows / 8; grp += NWAVES) {
      const int chunk = (lane & 7) ^ swz(grp * 8 + r_in);
      if (stream)
        __builtin_amdgcn_global_load_lds(g + (int64_t)(grp * 8 + r_in) * K + chunk * 8, (lds_void*)(lds + grp * 1024),
                                         16, 0, 2);
      else
        __builtin_amdgcn_global_load_lds(g + (int64_t)(grp * 8 + r_in) * K + chunk * 8, (lds_void*)(lds + grp * 1024),
                                         16, 0, 0);
    }
  };

  for (int64_t item = vid; item < total; item += G) {
    int tile_i, nb;
    item_coords<ORDER>(item, nt, nbn, tile_i, nb);
    const int le = tiles[2 * tile_i];
    const int row0 = tiles[2 * tile_i + 1];
    if (le < 0 || le >= E_loc || row0 < 0 || (int64_t)row0 + BM > R_cap) continue;  // block-uniform
    int valid = counts[le] - (row0 - offsets[le]);
    valid = valid < BM ? valid : BM;
    const int n0 = nb * BN;

    const uint16_t* a_g = A + (int64_t)row0 * K;
    // GATHER: this lane's token row of x for its wave's 8-row group of A
    // (padding rows read token 0: valid memory, never stored).
    const uint16_t* a_row = A;
    if (GATHER && wave < BM / 8) {
      const int src = row_src[row0 + wave * 8 + (lane >> 3)];
      const int64_t t = src >= 0 ? src / topk : 0;
      a_row = A + (t < T ? t : 0) * (int64_t)K;
    }
    const uint16_t* b0_g = B0 + le * b_expert + (int64_t)n0 * K;
    const uint16_t* b1_g = DUAL ? B1 + le * b_expert + (int64_t)n0 * K : nullptr;

    floatx4 acc[NMAT][TN][TM];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[m][i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int stage, int k0) {
      char* s = smem + stage * STAGE;
      if (GATHER) {
        if (wave < BM / 8)
          __builtin_amdgcn_global_load_lds(a_row + k0 + ((lane & 7) ^ swz(wave * 8 + (lane >> 3))) * 8,
                                           (lds_void*)(s + wave * 1024), 16, 0, 0);
      } else {
        stage_any(a_g + k0, BM, s, false);
      }
      stage_any(b0_g + k0, BN, s + A_BYTES, true);
      if (DUAL) stage_any(b1_g + k0, BN, s + A_BYTES + BN * 128, true);
    };

    // Loads per wave per stage: the weight rows, plus one token-row group on
    // the first BM / 8 waves.  Stage kt has landed once only the stages issued
    // after it (at most SR - 2) are in flight.
    const bool has_a = wave < BM / 8;
#pragma unroll
    for (int st = 0; st + 1 < SR; ++st)
      if (st < nk) issue(st, st * BK);
    for (int kt = 0; kt < nk; ++kt) {
      const int later = (nk - 1 - kt) < SR - 2 ? (nk - 1 - kt) : SR - 2;
      if (has_a) {
        if (later >= 2) wait_vmcnt<2 * (LW_B + 1)>();
        else if (later == 1) wait_vmcnt<LW_B + 1>();
        else wait_vmcnt<0>();
      } else {
        if (later >= 2) wait_vmcnt<2 * LW_B>();
        else if (later == 1) wait_vmcnt<LW_B>();
        else wait_vmcnt<0>();
      }
      wait_lgkm0();    // this wave's reads of stage kt - 1 are complete
      ring_barrier();  // stage kt visible to all; buffer (kt - 1) % SR is free
      if (kt + SR - 1 < nk) issue((kt + SR - 1) % SR, (kt + SR - 1) * BK);
      const char* sA = smem + (kt % SR) * STAGE;
      const char* sB = sA + A_BYTES;
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int chunk = ks * 4 + (lane >> 4);
        bf16x8 bf[NMAT][TN], af[TM];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int i = 0; i < TN; ++i)
            bf[m][i] = lds_frag(sB, m * BN + wn * WT_N + i * 16 + (lane & 15), chunk);
#pragma unroll
        for (int j = 0; j < TM; ++j) af[j] = lds_frag(sA, wm * WT_M + j * 16 + (lane & 15), chunk);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
              acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[m][i], af[j], acc[m][i][j], 0, 0, 0);
      }
    }

    // Epilogue: lane holds columns n..n+3 of row m for every (i, j).
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = wm * WT_M + j * 16 + (lane & 15);
      if (m >= valid) continue;
      const int64_t row = (int64_t)row0 + m;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = n0 + wn * WT_N + i * 16 + 4 * (lane >> 4);
        float g[4], u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g[r] = acc[0][i][j][r];
          u[r] = acc[NMAT - 1][i][j][r];
        }
        store4<EPI>(C, row, N, n, g, u);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the next item's first stage overwrites LDS
  }
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// CUs that kernels launched on stream s may use: the popcount of its CU mask
// (a stream created with hipExtStreamCreateWithCUMask), else every CU.
int stream_cus(hipStream_t s) {
  const int n = num_cus();
  uint32_t mask[32] = {0};  // up to 1024 CUs
  if (n > 1024 || hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) return n;
  int c = 0;
  for (uint32_t m : mask) c += __builtin_popcount(m);
  return (c > 0 && c < n) ? c : n;
}

// Persistent grid: one workgroup per usable CU, rounded down to a multiple of
// the XCD count (so every workgroup is resident at once), fewer if there are
// fewer items.
int64_t persistent_grid(int64_t max_items, int cus) {
  int64_t grid = cus >= kXcds ? cus / kXcds * kXcds : kXcds;
  if (max_items < grid) grid = (max_items + kXcds - 1) / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  return grid;
}

template <typename Kern, typename... Extra>
hipError_t launch_persistent(Kern kern, int threads, int64_t max_items, const uint16_t* A, const uint16_t* B0,
                             const uint16_t* B1, int N, int K, const FfnArgs& a, void* C, Extra... extra) {
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid(max_items, a.cus)), dim3(threads), 0, a.stream, A, B0, B1, N, K,
                     a.counts, a.offsets, a.tiles, a.num_tiles, a.tiles_cap, a.R_cap, a.E_loc, C, extra...);
  return hipGetLastError();
}

// Layer1 over BM x BN items; with a workspace the last round is split along K.
template <int BM, int BN, int ST>
hipError_t launch_layer1(const FfnArgs& a) {
  const int64_t max_items = a.tiles_cap * (a.H / BN);
  if (a.ws == nullptr)
    return launch_persistent(gemm_mfma32_kernel<BM, BN, false, EPI_F32, ORDER_N, ST, false, false>, 256, max_items,
                             a.act_buf, a.w1, nullptr, a.H, a.F, a, a.y_perm, (float*)nullptr, (const int32_t*)nullptr, 0, (int64_t)0);
  hipError_t e = launch_persistent(gemm_mfma32_kernel<BM, BN, false, EPI_F32, ORDER_N, ST, true, false>, 256, max_items,
                                   a.act_buf, a.w1, nullptr, a.H, a.F, a, a.y_perm, static_cast<float*>(a.ws), (const int32_t*)nullptr, 0, (int64_t)0);
  if (e != hipSuccess) return e;
  const int G = (int)persistent_grid(max_items, a.cus);
  hipLaunchKernelGGL((reduce_slices_kernel<BM, BN, false, EPI_F32, ORDER_N>), dim3((unsigned)(G * (BM / 16))), dim3(256),
                     0, a.stream, static_cast<const float*>(a.ws), a.H, a.F, G, a.counts, a.offsets, a.tiles,
                     a.num_tiles, a.tiles_cap, a.R_cap, a.E_loc, a.y_perm);
  return hipGetLastError();
}

// tile_m >= 128: layer0 = BM x (BN0 gate + BN0 up) (GELU: BM x BN0), layer1 = BM x BN1
// (BM x 128 when H is not a multiple of BN1).
// Layer0 over BM x BN0 items (DUAL: gate and up), reading the token rows from
// x_perm or (GATHER) from x; with a workspace the last round is split along K.
template <int BM, int BN0, int ST0, bool DUAL, int EPI, bool GATHER>
hipError_t launch_layer0(const FfnArgs& a) {
  const int64_t items = a.tiles_cap * (a.F / BN0);
  const uint16_t* A = GATHER ? a.x : a.x_perm;
  const uint16_t* B1 = DUAL ? a.w0_up : nullptr;
  if (a.ws == nullptr)
    return launch_persistent(gemm_mfma32_kernel<BM, BN0, DUAL, EPI, ORDER_M, ST0, false, GATHER>, 256, items, A, a.w0,
                             B1, a.F, a.H, a, a.act_buf, (float*)nullptr, a.row_src, a.topk, a.T);
  hipError_t e = launch_persistent(gemm_mfma32_kernel<BM, BN0, DUAL, EPI, ORDER_M, ST0, true, GATHER>, 256, items, A,
                                   a.w0, B1, a.F, a.H, a, a.act_buf, static_cast<float*>(a.ws), a.row_src, a.topk, a.T);
  if (e != hipSuccess) return e;
  const int G = (int)persistent_grid(items, a.cus);
  hipLaunchKernelGGL((reduce_slices_kernel<BM, BN0, DUAL, EPI, ORDER_M>), dim3((unsigned)(G * (BM / 16))), dim3(256),
                     0, a.stream, static_cast<const float*>(a.ws), a.F, a.H, G, a.counts, a.offsets, a.tiles,
                     a.num_tiles, a.tiles_cap, a.R_cap, a.E_loc, a.act_buf);
  return hipGetLastError();
}

template <int BM, int BN0, int ST0, bool GATHER>
hipError_t launch_big_layer0(const FfnArgs& a) {
  if (a.act == MOE_ACT_SWIGLU_I) return launch_layer0<BM, BN0, ST0, true, EPI_SWIGLU, GATHER>(a);
  return launch_layer0<BM, BN0, ST0, false, EPI_GELU, GATHER>(a);
}

template <int BM, int BN0, int ST0, int BN1, int ST1>
hipError_t launch_big(const FfnArgs& a) {
  hipError_t e = a.x_perm ? launch_big_layer0<BM, BN0, ST0, false>(a) : launch_big_layer0<BM, BN0, ST0, true>(a);
  if (e != hipSuccess) return e;
  if (a.H % BN1 == 0) return launch_layer1<BM, BN1, ST1>(a);
  return launch_layer1<BM, 128, ST0>(a);
}

// tile_m <= 64: weight-streaming shapes.
template <int BM, int BN0, int WM, int WN, bool GATHER>
hipError_t launch_small_layer0(const FfnArgs& a) {
  const int64_t items = a.tiles_cap * (a.F / BN0);
  const uint16_t* A = GATHER ? a.x : a.x_perm;
  if (a.act == MOE_ACT_SWIGLU_I)
    return launch_persistent(gemm_mfma16_kernel<BM, BN0, WM, WN, true, EPI_SWIGLU, ORDER_M, GATHER>, WM * WN * 64, items,
                             A, a.w0, a.w0_up, a.F, a.H, a, a.act_buf, a.row_src, a.topk, a.T);
  return launch_persistent(gemm_mfma16_kernel<BM, BN0, WM, WN, false, EPI_GELU, ORDER_M, GATHER>, WM * WN * 64, items, A,
                           a.w0, nullptr, a.F, a.H, a, a.act_buf, a.row_src, a.topk, a.T);
}

template <int BM, int WM, int WN, int BN0, int BN1, int WM1, int WN1>
hipError_t launch_small(const FfnArgs& a) {
  hipError_t e = a.x_perm ? launch_small_layer0<BM, BN0, WM, WN, false>(a) : launch_small_layer0<BM, BN0, WM, WN, true>(a);
  if (e != hipSuccess) return e;
  return launch_persistent(gemm_mfma16_kernel<BM, BN1, WM1, WN1, false, EPI_F32, ORDER_N, false>, WM1 * WN1 * 64,
                           a.tiles_cap * (a.H / BN1), a.act_buf, a.w1, nullptr, a.H, a.F, a, a.y_perm, (const int32_t*)nullptr, 0, (int64_t)0);
}

// Workspace of the fused launch: counters (zero before the first launch; every launch leaves them zero),
// then the K-slice partial tiles of the split layer1 items.
struct FusedWs {
  FusedCounters* ctr;
  int *ready, *group, *slices;
  float* part;
};
__host__ __device__ inline int64_t fused_ints(int64_t tiles_cap, int H, int G) {
  return (int64_t)(sizeof(FusedCounters) / 4) + tiles_cap + (H / 256 + kGroupN - 1) / kGroupN + G;
}
inline FusedWs fused_ws(void* ws, int64_t tiles_cap, int H, int G) {
  FusedWs w;
  char* p = static_cast<char*>(ws);
  w.ctr = reinterpret_cast<FusedCounters*>(p);
  w.ready = reinterpret_cast<int*>(p) + sizeof(FusedCounters) / 4;
  w.group = w.ready + tiles_cap;
  w.slices = w.group + (H / 256 + kGroupN - 1) / kGroupN;
  w.part = reinterpret_cast<float*>(p + (fused_ints(tiles_cap, H, G) * 4 + 255) / 256 * 256);
  return w;
}

}  // namespace

size_t fused_ffn_ws_bytes(int64_t tiles_cap, int H) {
  const int G = (int)persistent_grid(INT32_MAX, num_cus());
  return (size_t)((fused_ints(tiles_cap, H, G) * 4 + 255) / 256 * 256) + (size_t)G * 256 * 256 * sizeof(float);
}

hipError_t launch_ffn_fused(const FfnArgs& args, const int32_t* inv_perm, const float* topk_w, float* out) {
  FfnArgs a = args;
  a.cus = stream_cus(a.stream);
  const int G = (int)persistent_grid(INT32_MAX, a.cus);
  const FusedWs w = fused_ws(a.ws, a.tiles_cap, a.H, (int)persistent_grid(INT32_MAX, num_cus()));
  if (a.act == MOE_ACT_SWIGLU_I)
    hipLaunchKernelGGL((ffn_fused_kernel<true, EPI_SWIGLU>), dim3(G), dim3(256), 0, a.stream, a.x_perm, a.w0, a.w0_up,
                       a.w1, a.H, a.F, a.counts, a.offsets, a.tiles, a.num_tiles, a.tiles_cap, a.R_cap, a.E_loc,
                       a.act_buf, a.y_perm, inv_perm, topk_w, a.T, a.topk, out, w.ctr, w.ready, w.group, w.slices,
                       w.part);
  else
    hipLaunchKernelGGL((ffn_fused_kernel<false, EPI_GELU>), dim3(G), dim3(256), 0, a.stream, a.x_perm, a.w0, nullptr,
                       a.w1, a.H, a.F, a.counts, a.offsets, a.tiles, a.num_tiles, a.tiles_cap, a.R_cap, a.E_loc,
                       a.act_buf, a.y_perm, inv_perm, topk_w, a.T, a.topk, out, w.ctr, w.ready, w.group, w.slices,
                       w.part);
  return hipGetLastError();
}

size_t grouped_ffn_ws_bytes(int tile_m, int H) {
  // Split-K partial tiles of either layer's last round: at most one round of
  // pieces of tile_m x 256 fp32 (layer1's BM x 256, layer0's BM x (128 gate + 128 up)).
  (void)H;
  if (tile_m < 128) return 0;
  return (size_t)persistent_grid(INT32_MAX, num_cus()) * tile_m * 256 * sizeof(float);
}

hipError_t launch_grouped_ffn(const FfnArgs& args) {
  FfnArgs a = args;
  a.cus = stream_cus(a.stream);  // the same grid for every launch of this call
  switch (a.tile_m) {
    case 256: return launch_big<256, 128, 2, 256, 2>(a);
    case 128: return launch_big<128, 128, 3, 256, 3>(a);
    case 64: return launch_small<64, 1, 8, 128, 128, 1, 8>(a);
    case 32: return launch_small<32, 1, 8, 128, 128, 1, 8>(a);
    case 16: return launch_small<16, 1, 8, 128, 128, 1, 8>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
