// Grouped expert GEMMs with a fused activation epilogue, for gfx950.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts":
//   - section 3.1.2: one GroupGEMM computes all experts of this rank over
//     tile-aligned sub-tensors, tiles holding local tokens first;
//   - section 3.1.1: layer0 is decomposed along M (token rows are
//     independent), layer1 along N (the top-k reduce couples rows across
//     experts, so output columns are produced block by block);
//   - section 4: the MoE GEMMs avoid re-reading row indices from global
//     memory on every K iteration (here the rows are already contiguous, so
//     a tile needs only its first row and its expert).
// Tile-level-signalling follow-up (abstract): a persistent kernel covers all
// local experts without relaunches.
//
// Design (MI355X / CDNA4):
//   * Persistent grid, one workgroup per CU (or more for small tiles); the
//     work-item list is (tile, column block) pairs, read from the device tile
//     list, so the host never needs the per-expert row counts.
//   * Workgroup ids are remapped so that each XCD (workgroups are dispatched
//     round-robin over the 8 XCDs) processes a contiguous run of work items;
//     items that run together share operand panels through that XCD's L2.
//   * Layer0 order: groups of kGroupM consecutive tiles of the tile list;
//     inside a group, column block major then tile.  Layer1 order: column
//     block major over the whole tile list (N-decomposition).
//   * Operands are staged HBM -> LDS with global_load_lds_dwordx4 (16 bytes
//     per lane straight into LDS, no VGPR round trip), double buffered, BK=64.
//     Each LDS row holds 64 bf16 (128 B) of one operand row; the 16-byte
//     chunk index is XOR-swizzled with (row & 7) so the MFMA fragment reads
//     (16 rows x 16 bytes per 16 lanes) are bank-conflict free.
//   * MFMA v_mfma_f32_16x16x32_bf16 with operand roles swapped: the weight
//     tile feeds the A side (rows = output columns n) and the token tile the
//     B side (columns = token rows m).  Each lane then holds 4 consecutive
//     output columns of one row, so the epilogue stores 8 B (bf16) or 16 B
//     (fp32) vectors.
//   * Epilogue: SwiGLU silu(g) * u, or exact-erf GELU, in fp32, rounded to
//     bf16 (nearest even) for layer0; plain fp32 for layer1.  Rows past the
//     expert's real count are never stored.
#include "common.h"

namespace moe {
namespace {

constexpr int BK = 64;          // K per stage (one 128-byte LDS row per operand row)
constexpr int kGroupM = 8;      // layer0: tiles per rasterisation group
constexpr int kXcds = 8;

enum Epi { EPI_GELU = 0, EPI_SWIGLU = 1, EPI_F32 = 2 };

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_f(float h) { return 0.5f * h * (1.0f + erff(h * 0.70710678118654752f)); }

// Load ROWS operand rows x 64 bf16 (row stride ld elements) into a swizzled
// LDS tile with direct-to-LDS loads: one wave instruction moves 8 rows.
template <int ROWS, int NWAVES>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ g, int64_t ld, char* lds,
                                           int wave, int lane) {
  const int r_in = lane >> 3;                  // row within the 8-row group
  const int chunk = (lane & 7) ^ r_in;         // logical 16-byte chunk this lane fetches
  const uint16_t* src = g + (int64_t)r_in * ld + chunk * 8;
#pragma unroll
  for (int grp = wave; grp < ROWS / 8; grp += NWAVES) {
    __builtin_amdgcn_global_load_lds(src + (int64_t)grp * 8 * ld, (lds_void*)(lds + grp * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((chunk ^ (row & 7)) << 4));
}

template <int BM, int BN, int WM, int WN, bool DUAL, int EPI, bool NMAJOR>
__global__ __launch_bounds__(WM * WN * 64, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A,    // [R_cap, K] bf16 (x_perm or act)
    const uint16_t* __restrict__ B0,   // [E_loc, N, K] bf16
    const uint16_t* __restrict__ B1,   // [E_loc, N, K] bf16 (DUAL) or null
    int N, int K, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int64_t tiles_cap,
    int64_t R_cap, int E_loc, void* __restrict__ C) {
  constexpr int NWAVES = WM * WN;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BROWS = NMAT * BN;               // weight rows staged per stage
  constexpr int A_BYTES = BM * 128, B_BYTES = BROWS * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int WT_M = BM / WM, WT_N = BN / WN;  // wave tile (per matrix)
  constexpr int TM = WT_M / 16, TN = WT_N / 16;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(BM % 8 == 0 && BROWS % 8 == 0, "rows per stage");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int G = gridDim.x;
  const int vid = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;

  int nt = *num_tiles;
  if (nt > tiles_cap) nt = (int)tiles_cap;
  const int nbn = N / BN;
  const int64_t total = (int64_t)nt * nbn;
  const int nk = K / BK;
  const int64_t b_expert = (int64_t)N * K;

  for (int64_t item = vid; item < total; item += G) {
    int tile_i, nb;
    if (NMAJOR) {
      nb = (int)(item / nt);
      tile_i = (int)(item % nt);
    } else {
      const int64_t per_group = (int64_t)kGroupM * nbn;
      const int grp = (int)(item / per_group);
      const int64_t rem = item % per_group;
      const int gsize = (nt - grp * kGroupM) < kGroupM ? (nt - grp * kGroupM) : kGroupM;
      nb = (int)(rem / gsize);
      tile_i = grp * kGroupM + (int)(rem % gsize);
    }
    const int le = tiles[2 * tile_i];
    const int row0 = tiles[2 * tile_i + 1];
    if (le < 0 || le >= E_loc || row0 < 0 || (int64_t)row0 + BM > R_cap) continue;  // block-uniform
    int valid = counts[le] - (row0 - offsets[le]);
    valid = valid < BM ? valid : BM;
    const int n0 = nb * BN;

    const uint16_t* a_g = A + (int64_t)row0 * K;
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
      stage_rows<BM, NWAVES>(a_g + k0, K, s, wave, lane);
      stage_rows<BN, NWAVES>(b0_g + k0, K, s + A_BYTES, wave, lane);
      if (DUAL) stage_rows<BN, NWAVES>(b1_g + k0, K, s + A_BYTES + BN * 128, wave, lane);
    };

    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads for stage kt have landed
      __syncthreads();                // ... and everyone's; the other stage is free
      if (kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) * BK);
      const char* sA = smem + (kt & 1) * STAGE;
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
        if (EPI == EPI_F32) {
          *reinterpret_cast<floatx4*>(static_cast<float*>(C) + row * N + n) = acc[0][i][j];
        } else {
          uint16_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[0][i][j][q];
            float a;
            if (EPI == EPI_SWIGLU) a = silu_f(g) * acc[NMAT - 1][i][j][q];
            else a = gelu_f(g);
            h[q] = f2bf_bits(a);
          }
          const uint2 packed = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + row * N + n) = packed;
        }
      }
    }
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

template <int BM, int BN, int WM, int WN, bool DUAL, int EPI, bool NMAJOR>
hipError_t launch_one(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int N, int K, const FfnArgs& a,
                      void* C, hipStream_t s) {
  const int64_t max_items = a.tiles_cap * (N / BN);
  int64_t grid = num_cus();
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (max_items < grid) grid = (max_items + kXcds - 1) / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, DUAL, EPI, NMAJOR>), dim3((unsigned)grid),
                     dim3(WM * WN * 64), 0, s, A, B0, B1, N, K, a.counts, a.offsets, a.tiles, a.num_tiles,
                     a.tiles_cap, a.R_cap, a.E_loc, C);
  return hipGetLastError();
}

// Per-tile_m kernel shapes: layer0 uses BN columns of each of gate and up.
template <int BM, int WM, int WN, int BN0, int BN1, int WM1, int WN1>
hipError_t launch_tm(const FfnArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.act == 1) {
    e = launch_one<BM, BN0, WM, WN, true, EPI_SWIGLU, false>(a.x_perm, a.w0, a.w0_up, a.F, a.H, a, a.act_buf, s);
  } else {
    e = launch_one<BM, BN0, WM, WN, false, EPI_GELU, false>(a.x_perm, a.w0, nullptr, a.F, a.H, a, a.act_buf, s);
  }
  if (e != hipSuccess) return e;
  return launch_one<BM, BN1, WM1, WN1, false, EPI_F32, true>(a.act_buf, a.w1, nullptr, a.H, a.F, a, a.y_perm, s);
}

}  // namespace

hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t s) {
  switch (a.tile_m) {
    case 256: return launch_tm<256, 2, 4, 128, 128, 4, 2>(a, s);
    case 128: return launch_tm<128, 2, 4, 128, 128, 2, 4>(a, s);
    case 64: return launch_tm<64, 1, 8, 128, 128, 1, 8>(a, s);
    case 32: return launch_tm<32, 1, 8, 128, 128, 1, 8>(a, s);
    case 16: return launch_tm<16, 1, 8, 128, 128, 1, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
