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
// which yields the order (expert, rank, token).  Three launches, no atomics
// deciding any order (the result is bit-identical run to run):
//   A  count:   one block per chunk of 256 tokens.  Each wavefront ranks its
//               pairs inside their bucket with a ballot multisplit over the
//               bits of the bucket id (the rank of a pair is the number of
//               lower lanes holding the same bucket in any slot; a token has
//               at most one pair per bucket); per-wavefront counts in LDS turn
//               those into ranks inside the chunk and the chunk's count per
//               bucket, hist[b][c].
//   B  scan:    one block: exclusive scan of hist in (bucket, chunk) order
//               with 16-byte loads, per-expert counts, tile-padded offsets,
//               padding markers in row_src, and the tile list ordered by
//               (priority, expert, m-tile) with a stable partition on priority.
//   D  scatter: each block marks a slice of the unused rows past the last
//               expert; one wavefront per token: row of each local pair =
//               offsets[expert] + (prefix of its bucket and chunk - prefix of
//               the expert) + rank in chunk, written to row_src / inv_perm, and
//               the token's row copied once from HBM to each of its rows with
//               the whole row in flight (16-byte loads).
#include "common.h"

namespace moe {
namespace {

constexpr int kChunk = 256;         // tokens per chunk (one block of kernel A)
constexpr int kScanThreads = 1024;  // block size of kernel B
constexpr int kMaxExperts = 4096;   // E_loc * num_ranks <= 4096 (validated on the host)

struct WsLayout {
  int64_t nb, nc;
  int32_t* hist;   // [nb * nc], then exclusive prefix
  int32_t* lrank;  // [T * k], rank of the pair inside its bucket and chunk, -1 if not local
};

__host__ __device__ inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline WsLayout ws_layout(void* ws, int64_t T, int k, int E_loc, int num_ranks) {
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
// Dynamic LDS: bucket[k][256] ints, then count[4 wavefronts][nb] ints.
// KS >= k: slot loops are unrolled to KS (a power of two) with k as a guard,
// so the per-lane state stays in registers and the code stays small.
template <int KS>
__global__ __launch_bounds__(kChunk) void permute_count_kernel(const int32_t* __restrict__ topk_idx,
                                                               const int32_t* __restrict__ src_rank, int64_t T,
                                                               int k, int expert_begin, int E_loc, int R, int nbits,
                                                               int32_t* __restrict__ hist,
                                                               int32_t* __restrict__ lrank, int64_t nb, int64_t nc) {
  extern __shared__ int32_t sh[];
  int32_t* s_bucket = sh;                 // [k][kChunk]
  int32_t* s_count = sh + k * kChunk;     // [4][nb]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t t = c * kChunk + tid;
  const bool valid = t < T;
  const int r = valid ? clamp_rank(src_rank, t, R) : 0;

  for (int j = 0; j < k; ++j) {
    int b = -1;
    if (valid) {
      const int le = topk_idx[t * k + j] - expert_begin;
      if (le >= 0 && le < E_loc) b = le * R + r;
    }
    s_bucket[j * kChunk + tid] = b;
  }
  for (int64_t i = tid; i < 4 * nb; i += kChunk) s_count[i] = 0;
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Rank of each of this lane's pairs among the wavefront's pairs with the same
  // bucket, and that bucket's count in the wavefront.  The other lanes' slot jp
  // is compared with all of this lane's slots at once: a lane matches when its
  // bucket agrees on every bit, one ballot per bit narrowing the KS candidate
  // masks.  Rank (< 64) and count (<= 64) are packed into one int as
  // rank | count << 16.
  int own[KS], packed[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    own[j] = j < k ? s_bucket[j * kChunk + tid] : -1;
    packed[j] = 0;
  }
  for (int jp = 0; jp < k; ++jp) {
    const int bo = s_bucket[jp * kChunk + tid];
    const uint64_t vm = __ballot(bo >= 0);
    uint64_t m[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) m[j] = vm;
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t bal = __ballot(bo >= 0 && ((bo >> bit) & 1));
#pragma unroll
      for (int j = 0; j < KS; ++j) m[j] &= ((own[j] >> bit) & 1) ? bal : ~bal;
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) packed[j] += (int)__popcll(m[j] & below) | ((int)__popcll(m[j]) << 16);
  }
  // Each bucket present in this wavefront has exactly one pair with rank 0: it publishes the count.
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    if (j < k) {
      const int b = own[j];
      if (b >= 0 && (packed[j] & 0xFFFF) == 0) s_count[(int64_t)w * nb + b] = packed[j] >> 16;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    if (j < k && valid) {
      const int b = own[j];
      int rk = -1;
      if (b >= 0) {
        rk = packed[j] & 0xFFFF;
        for (int wp = 0; wp < w; ++wp) rk += s_count[(int64_t)wp * nb + b];
      }
      lrank[t * k + j] = rk;
    }
  }
  for (int64_t b = tid; b < nb; b += kChunk)
    hist[b * nc + c] = s_count[b] + s_count[nb + b] + s_count[2 * nb + b] + s_count[3 * nb + b];
}

// ---------------------------------------------------------------------------
// Block-wide scan helpers for kernel B (1024 threads = 16 wavefronts)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan of one int per thread over the block; returns the prefix and
// writes the block total to *total.  Contains __syncthreads().
__device__ int block_excl_scan(int v, int* sh /*[16 + 1]*/, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    int s = lane < 16 ? sh[lane] : 0;
    const int si = wave_incl_scan(s);
    if (lane < 16) sh[lane] = si - s;
    if (lane == 15) sh[16] = si;
  }
  __syncthreads();
  const int res = sh[w] + inc - v;
  *total = sh[16];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// B: scan, offsets, padding markers, tile list
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    int32_t* __restrict__ hist, int64_t nb, int64_t nc, int E_loc, int R, int tile_m, int64_t R_cap,
    int64_t tiles_cap, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int sh[17];
  __shared__ int s_us[kMaxExperts + 1];   // unpadded start of each expert
  __shared__ int s_off[kMaxExperts + 1];  // padded start
  __shared__ int s_tb[kMaxExperts + 1];   // first tile index of each expert
  const int tid = threadIdx.x;
  const int64_t N = nb * nc;

  // 1. exclusive scan of hist in (bucket, chunk) order, 16 consecutive entries
  //    per thread per pass (four 16-byte loads in flight when aligned and in range)
  constexpr int V = 16;
  int carry = 0;
  for (int64_t base = 0; base < N; base += (int64_t)kScanThreads * V) {
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
    int tot;
    int run = carry + block_excl_scan(s, sh, &tot);
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
    carry += tot;
  }
  const int total = carry;
  __syncthreads();

  // 2. per-expert unpadded starts, counts, padded offsets, tile starts
  for (int le = tid; le <= E_loc; le += kScanThreads)
    s_us[le] = le < E_loc ? hist[(int64_t)le * R * nc] : total;
  __syncthreads();
  {
    // E_loc <= 4096 -> at most 4 experts per thread, contiguous.
    const int per = (E_loc + kScanThreads - 1) / kScanThreads;
    const int e_lo = tid * per, e_hi = e_lo + per < E_loc ? e_lo + per : E_loc;
    int pad_sum = 0, tile_sum = 0;
    for (int le = e_lo; le < e_hi; ++le) {
      const int cnt = s_us[le + 1] - s_us[le];
      const int mt = (cnt + tile_m - 1) / tile_m;
      pad_sum += mt * tile_m;
      tile_sum += mt;
    }
    int pad_total, tile_total;
    int pad_run = block_excl_scan(pad_sum, sh, &pad_total);
    int tile_run = block_excl_scan(tile_sum, sh, &tile_total);
    for (int le = e_lo; le < e_hi; ++le) {
      const int cnt = s_us[le + 1] - s_us[le];
      const int mt = (cnt + tile_m - 1) / tile_m;
      s_off[le] = pad_run;
      s_tb[le] = tile_run;
      counts[le] = cnt;
      offsets[le] = pad_run;
      pad_run += mt * tile_m;
      tile_run += mt;
    }
    if (tid == 0) {
      s_off[E_loc] = pad_total;
      s_tb[E_loc] = tile_total;
      offsets[E_loc] = pad_total;
    }
  }
  __syncthreads();

  // 3. padding rows carry -1 in row_src (the unused tail past the last expert
  //    is marked by kernel D, spread over its blocks)
  for (int64_t i = tid; i < (int64_t)E_loc * tile_m; i += kScanThreads) {
    const int le = (int)(i / tile_m), q = (int)(i % tile_m);
    const int64_t row = (int64_t)s_off[le] + (s_us[le + 1] - s_us[le]) + q;
    if (row < s_off[le + 1]) row_src[row] = -1;
  }

  // 4. tile list, stably partitioned on priority (= rank of the tile's last row)
  const int nt = s_tb[E_loc] < tiles_cap ? s_tb[E_loc] : (int)tiles_cap;
  if (tid == 0) *num_tiles = nt;
  // Tile i -> (expert le, m-tile m) by binary search in LDS; its priority
  // from the expert's rank prefix in hist.  The priorities of the first
  // kPrioChunks * kScanThreads tiles are computed once and kept in registers
  // for the R partition passes; later tiles (if any) recompute theirs.
  constexpr int kPrioChunks = 4;
  auto tile_em = [&](int i, int& le, int& m) {
    int a = 0, b = E_loc;  // largest le with s_tb[le] <= i
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (s_tb[mid] <= i) a = mid; else b = mid;
    }
    le = a;
    m = i - s_tb[le];
  };
  auto tile_prio = [&](int le, int m) {
    const int cnt = s_us[le + 1] - s_us[le];
    const int last = ((m + 1) * tile_m < cnt ? (m + 1) * tile_m : cnt) - 1;
    int prio = 0;
    for (int r = 1; r < R; ++r) {
      const int cum = hist[((int64_t)le * R + r) * nc] - s_us[le];  // rows of expert le with rank < r
      if (cum <= last) prio = r;
    }
    return prio;
  };
  int cprio[kPrioChunks];
#pragma unroll
  for (int c = 0; c < kPrioChunks; ++c) {
    const int i = c * kScanThreads + tid;
    cprio[c] = 0;
    if (R > 1 && i < nt) {
      int le, m;
      tile_em(i, le, m);
      cprio[c] = tile_prio(le, m);
    }
  }
  int placed = 0;
  for (int p = 0; p < R; ++p) {
    for (int base_i = 0; base_i < nt; base_i += kScanThreads) {
      const int i = base_i + tid;
      const int c = base_i / kScanThreads;
      int le = 0, prio = -1, m = 0;
      if (i < nt) {
        tile_em(i, le, m);
        if (c < kPrioChunks) {
#pragma unroll
          for (int cc = 0; cc < kPrioChunks; ++cc)
            if (cc == c) prio = cprio[cc];
        } else {
          prio = tile_prio(le, m);
        }
      }
      const int flag = (prio == p) ? 1 : 0;
      int cnt_p;
      const int pos = block_excl_scan(flag, sh, &cnt_p);
      if (flag) {
        tiles[2 * (int64_t)(placed + pos)] = le;
        tiles[2 * (int64_t)(placed + pos) + 1] = s_off[le] + m * tile_m;
      }
      placed += cnt_p;
    }
  }
}

// ---------------------------------------------------------------------------
// D: index scatter + row copy, one wavefront per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const intx4* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ src_rank, int64_t T, int H, int k, int expert_begin, int E_loc, int R,
    int64_t R_cap, const int32_t* __restrict__ prefix, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ lrank, int64_t nc, intx4* __restrict__ x_perm, int32_t* __restrict__ row_src,
    int32_t* __restrict__ inv_perm) {
  const int lane = threadIdx.x & 63;
  {  // rows [offsets[E_loc], R_cap) are unused: -1 in row_src, a slice per block
    const int64_t tail0 = offsets[E_loc], n = R_cap - tail0;
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = tail0 + (int64_t)blockIdx.x * per, hi = lo + per < R_cap ? lo + per : R_cap;
    for (int64_t row = lo + threadIdx.x; row < hi; row += blockDim.x) row_src[row] = -1;
  }
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  int p = -1;
  if (lane < k) {
    const int le = topk_idx[t * k + lane] - expert_begin;
    if (le >= 0 && le < E_loc) {
      const int r = clamp_rank(src_rank, t, R);
      const int64_t b = (int64_t)le * R + r;
      p = offsets[le] + (prefix[b * nc + t / kChunk] - prefix[(int64_t)le * R * nc]) + lrank[t * k + lane];
      if (p < 0 || p >= R_cap) p = -1;  // inconsistent input; never write out of bounds
      if (p >= 0) row_src[p] = (int32_t)(t * k + lane);
    }
    inv_perm[t * k + lane] = p;
  }
  // Destination rows of this token's k slots (-1 = not local), wave-uniform.
  int dst[32];
  bool any = false;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    dst[j] = j < k ? __shfl(p, j) : -1;
    any |= dst[j] >= 0;
  }
  if (!any || x_perm == nullptr) return;  // no local slot, or indices only
  const int nch = H / 8;  // 16-byte chunks per row
  const intx4* src = x + t * nch;
  constexpr int U = 8;    // up to 8 x 16 B per lane in flight: an 8 KiB row per pass
  for (int c0 = lane; c0 < nch; c0 += kWave * U) {
    intx4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * kWave < nch) v[u] = src[c0 + u * kWave];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (dst[j] < 0) continue;
      intx4* out = x_perm + (int64_t)dst[j] * nch;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * kWave < nch) out[c0 + u * kWave] = v[u];
    }
  }
}

}  // namespace

size_t permute_ws_bytes(int64_t T, int k, int E_loc, int num_ranks) {
  const int64_t nb = (int64_t)E_loc * num_ranks, nc = (T + kChunk - 1) / kChunk;
  return (size_t)(align_up(nb * nc * 4, 256) + align_up(T * k * 4, 256));
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  WsLayout L = ws_layout(a.ws, a.T, a.k, a.E_loc, a.num_ranks);
  int nbits = 0;
  while ((1ll << nbits) < L.nb) ++nbits;
  const size_t count_lds = ((size_t)a.k * kChunk + 4 * (size_t)L.nb) * sizeof(int32_t);  // <= 96 KiB
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
#define MOE_COUNT(KS_)                                                                                           \
  hipLaunchKernelGGL(permute_count_kernel<KS_>, dim3((unsigned)L.nc), dim3(kChunk), count_lds, s, a.topk_idx,  \
                     a.src_rank, a.T, a.k, a.expert_begin, a.E_loc, a.num_ranks, nbits, L.hist, L.lrank, L.nb, L.nc)
  switch (ks) {
    case 1: MOE_COUNT(1); break;
    case 2: MOE_COUNT(2); break;
    case 4: MOE_COUNT(4); break;
    case 8: MOE_COUNT(8); break;
    case 16: MOE_COUNT(16); break;
    default: MOE_COUNT(32); break;
  }
#undef MOE_COUNT
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, L.hist, L.nb, L.nc, a.E_loc,
                     a.num_ranks, a.tile_m, a.R_cap, a.tiles_cap, a.counts, a.offsets, a.row_src, a.tiles,
                     a.num_tiles);
  const int wpb = 4;  // wavefronts per block
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)((a.T + wpb - 1) / wpb)), dim3(wpb * kWave), 0, s,
                     reinterpret_cast<const intx4*>(a.x), a.topk_idx, a.src_rank, a.T, a.H, a.k, a.expert_begin,
                     a.E_loc, a.num_ranks, a.R_cap, L.hist, a.offsets, L.lrank, L.nc,
                     reinterpret_cast<intx4*>(a.x_perm), a.row_src, a.inv_perm);
  return hipGetLastError();
}

}  // namespace moe
