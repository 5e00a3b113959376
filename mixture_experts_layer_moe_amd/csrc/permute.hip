// Token reorganisation into expert-contiguous, tile-aligned sub-tensors.
//
// "Comet: Fine-grained Computation-communication Overlapping for
// Mixture-of-Experts", section 3.1.2: the decomposed shared tensor is
// regrouped into GEMM-tile-aligned sub-tensors; layer0 sorts tokens by source
// rank and prioritises tiles holding local tokens.  Section 2.2.1: data
// reorganisation exposes only the data each tile needs.
//
// The (token, slot) pairs of local experts are stably counting-sorted on the
// bucket key b = local_expert * num_ranks + src_rank, visiting tokens in order,
// which yields the order (expert, rank, token).  No atomics decide any order
// (the result is bit-identical run to run):
//   A  count:  one block per chunk of 256 tokens.  Each pair sets its lane's
//              bit in a 64-bit LDS mask of its (bucket, wavefront); a token has
//              at most one pair per bucket, so the rank of a pair inside its
//              bucket and chunk is the number of set bits below it (earlier
//              wavefronts, then lower lanes), and the chunk's count per bucket,
//              hist[b][c], is the masks' total population.
//   P  place:  block 0 turns the bucket totals into per-expert counts,
//              tile-padded offsets, padding markers in row_src and the tile
//              list ordered by (priority, expert, m-tile), each tile's place
//              computed from the per-(priority, expert) tile counts (a tile's
//              priority is the largest source rank among its rows, so an
//              expert's tiles are in priority order).  Every other block owns a run of tokens
//              inside one chunk c: it rebuilds in LDS the bucket starts and,
//              per bucket, the rows of chunks before c (hist is small, so the
//              copies cost less than a launch), then, one wavefront per token,
//              row of each local pair = expert offset + (bucket start - expert
//              start) + rows of earlier chunks + rank in chunk, written to
//              row_src / inv_perm, and the token's row copied once from HBM to
//              each of its rows with the whole row in flight (16-byte loads,
//              non-temporal: each token row is read once, and streaming it
//              cut the placing kernel from 25 to 18 us with cold caches at the
//              Mixtral shape, warm unchanged).
//              The blocks also mark the unused rows past the last expert.
// When hist is too large to copy into every block, a single-block scan (B)
// writes the (bucket, chunk) prefix and the per-expert outputs between A and
// a place launch that reads that prefix from global memory.
#include "common.h"

#include <mutex>

// Scratch of moe_permute_noalloc (per-(bucket, chunk) counts and per-pair
// ranks, as in the caller's workspace of moe_permute): a fixed device array,
// one copy per GPU, held until the process ends.  Host code must never pass
// its name to a kernel -- on the host it is only a stand-in symbol -- but the
// device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[moe::kPermuteStaticWsBytes];

namespace moe {
namespace {

constexpr int kChunk = 256;             // tokens per chunk (one block of kernel A)
constexpr int kBlock = 1024;            // threads of the place and scan kernels (16 wavefronts)
constexpr int kWaves = kBlock / kWave;
constexpr int64_t kFusedReads = 1 << 23;  // place blocks x hist entries up to which hist is copied per block

struct WsLayout {
  int64_t nb, nc;
  int32_t* hist;   // [nb * nc] counts per (bucket, chunk); the scan kernel replaces them by their prefix
  int32_t* lrank;  // [T * k], rank of the pair inside its bucket and chunk, -1 if not local
};

__host__ __device__ inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline WsLayout ws_layout(void* ws, int64_t T, int E_loc, int num_ranks) {
  WsLayout L;
  L.nb = (int64_t)E_loc * num_ranks;
  L.nc = (T + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(ws);
  L.hist = reinterpret_cast<int32_t*>(p);
  p += align_up(L.nb * L.nc * 4, 256);
  L.lrank = reinterpret_cast<int32_t*>(p);
  return L;
}

__device__ __forceinline__ int clamp_rank(const int32_t* src_rank, int64_t t, int R) {
  if (src_rank == nullptr) return 0;
  const int r = src_rank[t];
  return r < 0 ? 0 : (r >= R ? R - 1 : r);
}

// ---------------------------------------------------------------------------
// A: ranks inside (bucket, chunk) and per-chunk bucket counts
// ---------------------------------------------------------------------------
// Dynamic LDS: mask[nb][4] 64-bit words (bit l of word w: lane l of wavefront
// w holds a pair of that bucket).  KS >= k: slot loops are unrolled to KS (a
// power of two) with k as a guard, so the per-lane state stays in registers.
template <int KS>
__global__ __launch_bounds__(kChunk) void permute_count_kernel(const int32_t* __restrict__ topk_idx,
                                                               const int32_t* __restrict__ src_rank, int64_t T,
                                                               int k, int expert_begin, int E_loc, int R,
                                                               int32_t* __restrict__ hist,
                                                               int32_t* __restrict__ lrank, int64_t nb, int64_t nc) {
  extern __shared__ unsigned long long s_mask[];  // [nb][4]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t t = c * kChunk + tid;
  const bool valid = t < T;
  for (int64_t i = tid; i < 4 * nb; i += kChunk) s_mask[i] = 0;
  const int r = valid ? clamp_rank(src_rank, t, R) : 0;
  int own[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    int b = -1;
    if (j < k && valid) {
      const int le = topk_idx[t * k + j] - expert_begin;
      if (le >= 0 && le < E_loc) b = le * R + r;
    }
    own[j] = b;
  }
  __syncthreads();
  const unsigned long long bit = 1ull << lane;
#pragma unroll
  for (int j = 0; j < KS; ++j)
    if (own[j] >= 0) atomicOr(&s_mask[(int64_t)own[j] * 4 + w], bit);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    if (j < k && valid) {
      int rk = -1;
      if (own[j] >= 0) {
        const unsigned long long* m = s_mask + (int64_t)own[j] * 4;
        rk = __popcll(m[w] & (bit - 1));
        for (int wp = 0; wp < w; ++wp) rk += __popcll(m[wp]);
      }
      lrank[t * k + j] = rk;
    }
  }
  for (int64_t b = tid; b < nb; b += kChunk) {
    const unsigned long long* m = s_mask + b * 4;
    hist[b * nc + c] = __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
  }
}

// ---------------------------------------------------------------------------
// Scans and per-expert layout
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active):
// Hillis-Steele steps of 1, 2, 4, 8 inside each row of 16 lanes with DPP row
// shifts (lanes shifted in from outside the row read 0), then each row adds
// the totals of the rows below it, read with readlane.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Orders one wavefront's LDS accesses across lanes (no instruction: LDS
// operations of a wavefront complete in issue order; this only stops the
// compiler from moving accesses across it).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wavefront: in-place exclusive prefix of s[0, n) in LDS, a contiguous run
// per lane; s[n] receives the total.  The caller's barrier publishes it.
__device__ void wave_excl_scan_lds(int* s, int n) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int lo = lane * per, hi = lo + per < n ? lo + per : n;
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += s[i];
  const int inc = wave_incl_scan(sum);
  int run = inc - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = s[i];
    s[i] = run;
    run += v;
  }
  if (lane == 63) s[n] = inc;
}

// Tiles of local expert le whose priority is at most p (priority of a tile =
// largest rank r in [1, R) such that the expert's rows of rank < r do not reach
// past the tile's last row, else 0).  Rows are sorted by rank, so these are
// the first tiles: the ones ending before the expert's first row of rank > p.
__device__ __forceinline__ int tiles_upto(const int* s_bs, int le, int R, int tile_m, int p) {
  const int start = s_bs[le * R], cnt = s_bs[(le + 1) * R] - start;
  const int mt = (cnt + tile_m - 1) / tile_m;
  if (p < 0) return 0;
  if (p >= R - 1) return mt;
  const int C = s_bs[le * R + p + 1] - start;  // rows of rank <= p
  return C >= cnt ? mt : C / tile_m;
}

// One wavefront, s_bs[0, nb] holding the exclusive bucket starts (expert le
// owns buckets [le * R, (le + 1) * R)): padded first row s_off[0, E_loc] and,
// when s_tb is given, first tile s_tb[0, E_loc] of every local expert.
__device__ void wave_expert_layout(const int* s_bs, int E_loc, int R, int tile_m, int* s_off, int* s_tb) {
  const int lane = threadIdx.x & 63;
  const int per = (E_loc + 63) / 64;
  const int lo = lane * per, hi = lo + per < E_loc ? lo + per : E_loc;
  int pad_sum = 0, tile_sum = 0;
  for (int le = lo; le < hi; ++le) {
    const int mt = (s_bs[(le + 1) * R] - s_bs[le * R] + tile_m - 1) / tile_m;
    pad_sum += mt * tile_m;
    tile_sum += mt;
  }
  const int pad_inc = wave_incl_scan(pad_sum), tile_inc = wave_incl_scan(tile_sum);
  int pad_run = pad_inc - pad_sum, tile_run = tile_inc - tile_sum;
  for (int le = lo; le < hi; ++le) {
    const int mt = (s_bs[(le + 1) * R] - s_bs[le * R] + tile_m - 1) / tile_m;
    s_off[le] = pad_run;
    pad_run += mt * tile_m;
    if (s_tb) s_tb[le] = tile_run;
    tile_run += mt;
  }
  if (lane == 63) {
    s_off[E_loc] = pad_inc;
    if (s_tb) s_tb[E_loc] = tile_inc;
  }
}

// Per-expert outputs of a block of kBlock threads, given the exclusive bucket
// starts s_bs[0, nb] (published): counts, offsets, -1 in row_src for the
// padding rows inside each expert's last tile, and the tile list ordered by
// (priority, expert, m-tile).  A tile's place in that order is the number of
// tiles of lower priority, plus the tiles of the same priority in earlier
// experts, plus its index among its expert's tiles of that priority: with
// s_pt[p * E_loc + le] = tiles of expert le with priority p, the exclusive
// prefix of s_pt gives the first two terms.  LDS: s_off, s_tb [E_loc + 1],
// s_pt [nb + 1].
__device__ void expert_outputs(const int* s_bs, int64_t nb, int E_loc, int R, int tile_m, int64_t tiles_cap,
                               int* s_off, int* s_tb, int* s_pt, int32_t* __restrict__ counts,
                               int32_t* __restrict__ offsets, int32_t* __restrict__ row_src,
                               int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  if (tid < kWave) wave_expert_layout(s_bs, E_loc, R, tile_m, s_off, s_tb);
  for (int64_t i = tid; i < nb; i += kBlock) {
    const int p = (int)(i / E_loc), le = (int)(i - (int64_t)p * E_loc);
    s_pt[i] = tiles_upto(s_bs, le, R, tile_m, p) - tiles_upto(s_bs, le, R, tile_m, p - 1);
  }
  __syncthreads();
  if (tid < kWave) wave_excl_scan_lds(s_pt, (int)nb);
  for (int le = tid; le <= E_loc; le += kBlock) {
    offsets[le] = s_off[le];
    if (le < E_loc) counts[le] = s_bs[(le + 1) * R] - s_bs[le * R];
  }
  for (int64_t i = tid; i < (int64_t)E_loc * tile_m; i += kBlock) {
    const int le = (int)(i / tile_m), q = (int)(i - (int64_t)le * tile_m);
    const int64_t row = (int64_t)s_off[le] + (s_bs[(le + 1) * R] - s_bs[le * R]) + q;
    if (row < s_off[le + 1]) row_src[row] = -1;
  }
  __syncthreads();
  const int nt = s_tb[E_loc] < tiles_cap ? s_tb[E_loc] : (int)tiles_cap;
  if (tid == 0) *num_tiles = nt;
  for (int i = tid; i < nt; i += kBlock) {
    int a = 0, b = E_loc;  // expert of tile i: largest le with s_tb[le] <= i
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (s_tb[mid] <= i) a = mid; else b = mid;
    }
    const int le = a, m = i - s_tb[le];
    int p = 0;  // smallest priority whose tiles include m
    while (tiles_upto(s_bs, le, R, tile_m, p) <= m) ++p;
    const int pos = s_pt[p * E_loc + le] + m - tiles_upto(s_bs, le, R, tile_m, p - 1);
    if (pos < nt) {
      tiles[2 * (int64_t)pos] = le;
      tiles[2 * (int64_t)pos + 1] = s_off[le] + m * tile_m;
    }
  }
}

// ---------------------------------------------------------------------------
// B (large hist only): (bucket, chunk) prefix in place, then the per-expert outputs
// ---------------------------------------------------------------------------
// Dynamic LDS: s_bs[nb + 1], s_pt[nb + 1], s_off[E_loc + 1], s_tb[E_loc + 1].
__global__ __launch_bounds__(kBlock) void permute_scan_kernel(
    int32_t* __restrict__ hist, int64_t nb, int64_t nc, int E_loc, int R, int tile_m, int64_t tiles_cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_src,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  extern __shared__ int s_dyn[];
  __shared__ int sh[kWaves + 1];
  int* s_bs = s_dyn;
  int* s_pt = s_bs + nb + 1;
  int* s_off = s_pt + nb + 1;
  int* s_tb = s_off + E_loc + 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t N = nb * nc;
  // 16 consecutive entries per thread per pass (four 16-byte loads when aligned and in range)
  constexpr int V = 16;
  int carry = 0;
  for (int64_t base = 0; base < N; base += (int64_t)kBlock * V) {
    const int64_t lo = base + (int64_t)tid * V;
    int v[V];
    if (lo + V <= N) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const intx4 x = *reinterpret_cast<const intx4*>(hist + lo + 4 * q);
        v[4 * q] = x[0]; v[4 * q + 1] = x[1]; v[4 * q + 2] = x[2]; v[4 * q + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int q = 0; q < V; ++q) v[q] = lo + q < N ? hist[lo + q] : 0;
    }
    int s = 0;
#pragma unroll
    for (int q = 0; q < V; ++q) s += v[q];
    // block-wide exclusive scan of s: per wavefront, then over the wavefront totals
    const int inc = wave_incl_scan(s);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
      const int ws = lane < kWaves ? sh[lane] : 0;
      const int wi = wave_incl_scan(ws);
      if (lane < kWaves) sh[lane] = wi - ws;
      if (lane == kWaves - 1) sh[kWaves] = wi;
    }
    __syncthreads();
    int run = carry + sh[w] + inc - s;
    carry += sh[kWaves];
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const int h = v[q];
      v[q] = run;
      run += h;
    }
    if (lo + V <= N) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q)
        *reinterpret_cast<intx4*>(hist + lo + 4 * q) = intx4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
#pragma unroll
      for (int q = 0; q < V; ++q)
        if (lo + q < N) hist[lo + q] = v[q];
    }
    __syncthreads();  // sh is rewritten by the next pass
  }
  for (int64_t b = tid; b <= nb; b += kBlock) s_bs[b] = b < nb ? hist[b * nc] : carry;
  __syncthreads();
  expert_outputs(s_bs, nb, E_loc, R, tile_m, tiles_cap, s_off, s_tb, s_pt, counts, offsets, row_src, tiles,
                 num_tiles);
}

// ---------------------------------------------------------------------------
// P: per-expert outputs (FUSED block 0), index scatter + row copy
// ---------------------------------------------------------------------------
// FUSED: hist holds per-(bucket, chunk) counts; block 0 writes the per-expert
// outputs, block 1 + i places tokens [i * kWaves * tpw, (i + 1) * kWaves * tpw),
// which lie inside one chunk.  Dynamic LDS: s_bs[nb + 1], s_cp[nb + 1] (block
// 0: s_pt), s_off[E_loc + 1], s_tb[E_loc + 1].
// Not FUSED: hist holds the (bucket, chunk) exclusive prefix and offsets the
// padded expert starts (both from the scan kernel); block i places tokens
// [i * kWaves * tpw, ...).  No dynamic LDS.
template <bool FUSED>
__global__ __launch_bounds__(kBlock) void permute_place_kernel(
    const intx4* __restrict__ x, const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ src_rank,
    int64_t T, int H, int k, int expert_begin, int E_loc, int R, int tile_m, int64_t R_cap, int64_t tiles_cap,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ lrank, int64_t nb, int64_t nc, int tpw,
    intx4* __restrict__ x_perm, int32_t* __restrict__ row_src, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int s_dyn[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t blk = blockIdx.x;
  int nblk = gridDim.x;
  int* s_bs = s_dyn;
  int* s_cp = s_bs + nb + 1;
  int* s_off = s_cp + nb + 1;
  int* s_tb = s_off + E_loc + 1;
  // Token state of this wavefront: lane j < k holds slot j's local expert (-1
  // if not local) and rank in chunk; v holds the first 8 KiB of the row.
  const int nch = H / 8;  // 16-byte chunks per row
  constexpr int U = 8;    // up to 8 x 16 B per lane in flight per pass
  int64_t t = 0;
  int le = -1, lr = -1, r = 0;
  bool any = false;
  intx4 v[U];
  auto fetch = [&]() {
    le = -1;
    if (lane < k) {
      const int e = topk_idx[t * k + lane] - expert_begin;
      lr = lrank[t * k + lane];
      if (e >= 0 && e < E_loc) le = e;
    }
    r = clamp_rank(src_rank, t, R);
    any = __ballot(le >= 0) != 0;
    if (any && x_perm != nullptr) {
      const intx4* src = x + t * nch;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane + u * kWave < nch) v[u] = __builtin_nontemporal_load(src + lane + u * kWave);
    }
  };
  int64_t tail0;
  if constexpr (FUSED) {
    const bool meta = blk == 0;
    blk -= 1;
    nblk -= 1;
    // The first token's indices and row are loaded before the prologue, whose latency they overlap.
    t = blk * tpw * kWaves + wv;
    if (!meta && t < T) fetch();
    // Tokens of this block lie in chunk c; the rows of bucket b in chunks before c go to s_cp[b].
    const int64_t c = meta ? 0 : blk * kWaves * tpw / kChunk;
    for (int64_t i = tid; i <= nb; i += kBlock) {
      s_bs[i] = 0;
      s_cp[i] = 0;
    }
    __syncthreads();
    const int64_t N = nb * nc;
    if ((nc & 3) == 0) {  // four chunks of one bucket per 16-byte load
      const intx4* h4 = reinterpret_cast<const intx4*>(hist);
      for (int64_t q = tid; q < N / 4; q += kBlock) {
        const intx4 h = h4[q];
        const int64_t b = 4 * q / nc, cc = 4 * q - b * nc;
        const int tot = h[0] + h[1] + h[2] + h[3];
        const int cp = (cc < c ? h[0] : 0) + (cc + 1 < c ? h[1] : 0) + (cc + 2 < c ? h[2] : 0) +
                       (cc + 3 < c ? h[3] : 0);
        if (tot) atomicAdd(&s_bs[b], tot);
        if (cp) atomicAdd(&s_cp[b], cp);
      }
    } else {
      for (int64_t i = tid; i < N; i += kBlock) {
        const int h = hist[i];
        const int64_t b = i / nc, cc = i - b * nc;
        if (h) {
          atomicAdd(&s_bs[b], h);
          if (cc < c) atomicAdd(&s_cp[b], h);
        }
      }
    }
    __syncthreads();
    if (meta) {
      if (tid < kWave) wave_excl_scan_lds(s_bs, (int)nb);
      __syncthreads();
      expert_outputs(s_bs, nb, E_loc, R, tile_m, tiles_cap, s_off, s_tb, s_cp, counts, offsets, row_src, tiles,
                     num_tiles);
      return;
    }
    if (tid < kWave) {
      wave_excl_scan_lds(s_bs, (int)nb);
      wave_lds_order();
      wave_expert_layout(s_bs, E_loc, R, tile_m, s_off, nullptr);
    }
    __syncthreads();
    tail0 = s_off[E_loc];
  } else {
    t = blk * tpw * kWaves + wv;
    if (t < T) fetch();
    tail0 = offsets[E_loc];
  }
  {  // rows [tail0, R_cap) are unused: -1 in row_src, a slice per block
    const int64_t n = R_cap - tail0;
    const int64_t per = (n + nblk - 1) / nblk;
    const int64_t lo = tail0 + blk * per, hi = lo + per < R_cap ? lo + per : R_cap;
    for (int64_t row = lo + tid; row < hi; row += kBlock) row_src[row] = -1;
  }
  for (int i = 0; i < tpw; ++i, t += kWaves) {
    if (t >= T) break;  // whole wave leaves together
    if (i > 0) fetch();
    int p = -1;
    if (le >= 0) {
      const int64_t b = (int64_t)le * R + r;
      if constexpr (FUSED)
        p = s_off[le] + (s_bs[b] - s_bs[(int64_t)le * R]) + s_cp[b] + lr;
      else
        p = offsets[le] + (hist[b * nc + t / kChunk] - hist[(int64_t)le * R * nc]) + lr;
      if (p < 0 || p >= R_cap) p = -1;  // inconsistent input; never write out of bounds
      if (p >= 0) row_src[p] = (int32_t)(t * k + lane);
    }
    if (lane < k) inv_perm[t * k + lane] = p;
    if (!any || x_perm == nullptr) continue;  // no local slot, or indices only
    // Lane j < k holds the destination row of slot j (-1 = not local).
    const intx4* src = x + t * nch;
    for (int c0 = lane; c0 < nch; c0 += kWave * U) {
      if (c0 != lane) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (c0 + u * kWave < nch) v[u] = __builtin_nontemporal_load(src + c0 + u * kWave);
      }
      for (int j = 0; j < k; ++j) {
        const int d = __builtin_amdgcn_readlane(p, j);
        if (d < 0) continue;
        intx4* out = x_perm + (int64_t)d * nch;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (c0 + u * kWave < nch) out[c0 + u * kWave] = v[u];
      }
    }
  }
}

// Tokens per wavefront of the fused place kernel, or 0 when hist is too large
// to copy into every block (then the scan kernel runs first).
int fused_tpw(int64_t T, int64_t nb, int64_t nc) {
  for (int tpw = 1; tpw * kWaves <= kChunk; tpw *= 2) {
    const int64_t blocks = (T + (int64_t)kWaves * tpw - 1) / ((int64_t)kWaves * tpw);
    if (blocks * nb * nc <= kFusedReads) return tpw;
  }
  return 0;
}

}  // namespace

hipError_t permute_static_ws(void** ptr) {
  // Device address of `scratch` on each device, looked up once with that device current.
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t permute_ws_bytes(int64_t T, int k, int E_loc, int num_ranks) {
  const int64_t nb = (int64_t)E_loc * num_ranks, nc = (T + kChunk - 1) / kChunk;
  return (size_t)(align_up(nb * nc * 4, 256) + align_up(T * k * 4, 256));
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  WsLayout L = ws_layout(a.ws, a.T, a.E_loc, a.num_ranks);
  const size_t count_lds = 4 * (size_t)L.nb * sizeof(unsigned long long);  // <= 128 KiB
  const int ks = a.k <= 1 ? 1 : a.k <= 2 ? 2 : a.k <= 4 ? 4 : a.k <= 8 ? 8 : a.k <= 16 ? 16 : 32;
  const void* count_fn = ks == 1    ? reinterpret_cast<const void*>(permute_count_kernel<1>)
                         : ks == 2  ? reinterpret_cast<const void*>(permute_count_kernel<2>)
                         : ks == 4  ? reinterpret_cast<const void*>(permute_count_kernel<4>)
                         : ks == 8  ? reinterpret_cast<const void*>(permute_count_kernel<8>)
                         : ks == 16 ? reinterpret_cast<const void*>(permute_count_kernel<16>)
                                    : reinterpret_cast<const void*>(permute_count_kernel<32>);
  if (count_lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(count_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)count_lds);
    if (e != hipSuccess) return e;
  }
#define MOE_COUNT(KS_)                                                                                          \
  hipLaunchKernelGGL(permute_count_kernel<KS_>, dim3((unsigned)L.nc), dim3(kChunk), count_lds, s, a.topk_idx, \
                     a.src_rank, a.T, a.k, a.expert_begin, a.E_loc, a.num_ranks, L.hist, L.lrank, L.nb, L.nc)
  switch (ks) {
    case 1: MOE_COUNT(1); break;
    case 2: MOE_COUNT(2); break;
    case 4: MOE_COUNT(4); break;
    case 8: MOE_COUNT(8); break;
    case 16: MOE_COUNT(16); break;
    default: MOE_COUNT(32); break;
  }
#undef MOE_COUNT
  const int tpw = fused_tpw(a.T, L.nb, L.nc);
  const intx4* x = reinterpret_cast<const intx4*>(a.x);
  intx4* x_perm = reinterpret_cast<intx4*>(a.x_perm);
  // Dynamic LDS of the scan and place kernels: two [nb + 1] and two [E_loc + 1] int arrays (<= 64 KiB + 16 B).
  const size_t lds = (size_t)(2 * (L.nb + 1) + 2 * (a.E_loc + 1)) * sizeof(int);
  const void* lds_fn = tpw > 0 ? reinterpret_cast<const void*>(permute_place_kernel<true>)
                               : reinterpret_cast<const void*>(permute_scan_kernel);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(lds_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (tpw > 0) {
    const int64_t blocks = 1 + (a.T + (int64_t)kWaves * tpw - 1) / ((int64_t)kWaves * tpw);
    hipLaunchKernelGGL(permute_place_kernel<true>, dim3((unsigned)blocks), dim3(kBlock), lds, s, x, a.topk_idx,
                       a.src_rank, a.T, a.H, a.k, a.expert_begin, a.E_loc, a.num_ranks, a.tile_m, a.R_cap,
                       a.tiles_cap, L.hist, L.lrank, L.nb, L.nc, tpw, x_perm, a.row_src, a.inv_perm, a.counts,
                       a.offsets, a.tiles, a.num_tiles);
  } else {
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kBlock), lds, s, L.hist, L.nb, L.nc, a.E_loc,
                       a.num_ranks, a.tile_m, a.tiles_cap, a.counts, a.offsets, a.row_src, a.tiles, a.num_tiles);
    const int64_t blocks = (a.T + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(permute_place_kernel<false>, dim3((unsigned)blocks), dim3(kBlock), 0, s, x, a.topk_idx,
                       a.src_rank, a.T, a.H, a.k, a.expert_begin, a.E_loc, a.num_ranks, a.tile_m, a.R_cap,
                       a.tiles_cap, L.hist, L.lrank, L.nb, L.nc, 1, x_perm, a.row_src, a.inv_perm, a.counts,
                       a.offsets, a.tiles, a.num_tiles);
  }
  return hipGetLastError();
}

}  // namespace moe
