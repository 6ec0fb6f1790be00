// Token -> expert dispatch as a stable counting sort of the T*top_k (token, slot)
// pairs by expert id: the single-GPU form of sending every token to the holder of
// its experts ("Use HF Transformers" cookbook, Parallelism).
//
// Stability without comparisons: inside a wavefront, lane l sets bit l of a per-expert
// 64-bit mask in LDS; a pair's rank among earlier pairs of the same expert in that
// wavefront is the popcount of the mask below its lane. Wavefronts, rounds and chunks
// are then stacked in pair order by prefix sums, so equal keys keep ascending pair id.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

constexpr int kWaves = 4;                       // 256-thread blocks in the chunked path
constexpr int kRounds = kChunkPairs / (kWaves * kWave);

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

// Exclusive scan of buf[0..n) in place (n <= blockDim.x); returns the total.
__device__ int block_excl_scan(int* buf, int* tmp, int n) {
    const int t = threadIdx.x;
    int v = t < n ? buf[t] : 0;
    tmp[t] = v;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
        int add = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        tmp[t] += add;
        __syncthreads();
    }
    const int incl = tmp[t];
    const int total = tmp[blockDim.x - 1];
    __syncthreads();
    if (t < n) buf[t] = incl - v;
    __syncthreads();
    return total;
}

// Work tiles for the grouped GEMMs, expert-major: for every tile_m rows of each expert's
// segment a record {expert, first row, index of the expert's first tile, tiles of the
// expert}; n_tiles[0] = the number of tiles, n_tiles[1 .. kTileWords-1] (the GEMMs' work-queue
// counters) = 0. cnt[] holds per-expert counts on entry (clobbered).
__device__ void write_tiles(int* cnt, int* tmp, int E, int tile_m, int32_t* tiles, int32_t* n_tiles) {
    const int t = threadIdx.x;
    int mt = 0;
    if (t < E) {
        mt = (cnt[t] + tile_m - 1) / tile_m;
        cnt[t] = mt;
    }
    __syncthreads();
    const int total = block_excl_scan(cnt, tmp, E);
    if (t < E)
        for (int i = 0; i < mt; ++i) {
            int32_t* rec = tiles + 4 * (cnt[t] + i);
            rec[0] = t;
            rec[1] = i * tile_m;
            rec[2] = cnt[t];
            rec[3] = mt;
        }
    if (t == 0) *n_tiles = total;
    else if (t < kTileWords) n_tiles[t] = 0;
}

// ---------------------------------------------------------------------------------------
// Small batches (P <= 1024 pairs, E <= 256): count, scan and scatter in one 1024-thread block.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pairs,
                                                              int32_t* __restrict__ pair_rank,
                                                              int32_t* __restrict__ tiles, int32_t* n_tiles,
                                                              int tile_m) {
    __shared__ uint64_t bm[16][256];
    __shared__ int cnt[1024];
    __shared__ int tmp[1024];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < 16 * 256; i += 1024) (&bm[0][0])[i] = 0ull;
    __syncthreads();
    const int e = t < P ? idx[t] : -1;
    const bool valid = e >= 0 && e < E;
    if (valid) atomicOr((unsigned long long*)&bm[wave][e], 1ull << lane);
    __syncthreads();
    int rank = 0;
    if (valid) {
        rank = __popcll(bm[wave][e] & lanemask_lt(lane));
        for (int w = 0; w < wave; ++w) rank += __popcll(bm[w][e]);
    }
    if (t < E) {
        int c = 0;
        for (int w = 0; w < 16; ++w) c += __popcll(bm[w][t]);
        cnt[t] = c;
    }
    __syncthreads();
    const int total = block_excl_scan(cnt, tmp, E);
    if (t < E) offsets[t] = cnt[t];
    if (t == 0) offsets[E] = total;
    if (t < P) {
        if (valid) {
            const int pos = cnt[e] + rank;
            sorted_pairs[pos] = t;
            if (pair_rank) pair_rank[t] = pos;
        } else if (pair_rank) {
            pair_rank[t] = -1;
        }
        if (t >= total) sorted_pairs[t] = -1;
    }
    if (tiles) {
        __syncthreads();
        if (t < E) cnt[t] = offsets[t + 1] - offsets[t];
        __syncthreads();
        write_tiles(cnt, tmp, E, tile_m, tiles, n_tiles);
    }
}

// ---------------------------------------------------------------------------------------
// Chunked path. 1) per chunk of kChunkPairs pairs: per-expert counts and each pair's
// stable rank inside its chunk.
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int32_t* __restrict__ rank_in_chunk) {
    extern __shared__ uint64_t smem[];
    uint64_t* bm = smem;                                   // [kWaves][E]
    int* running = reinterpret_cast<int*>(bm + kWaves * E);  // [E]
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < E; i += 256) running[i] = 0;
    const int64_t base = (int64_t)blockIdx.x * kChunkPairs;
    for (int r = 0; r < kRounds; ++r) {
        for (int i = t; i < kWaves * E; i += 256) bm[i] = 0ull;
        __syncthreads();
        const int64_t p = base + r * 256 + t;
        const int e = p < P ? idx[p] : -1;
        const bool valid = e >= 0 && e < E;
        if (valid) atomicOr((unsigned long long*)&bm[wave * E + e], 1ull << lane);
        __syncthreads();
        if (valid) {
            int rank = running[e] + __popcll(bm[wave * E + e] & lanemask_lt(lane));
            for (int w = 0; w < wave; ++w) rank += __popcll(bm[w * E + e]);
            rank_in_chunk[p] = rank;
        }
        __syncthreads();
        for (int i = t; i < E; i += 256) {
            int c = 0;
            for (int w = 0; w < kWaves; ++w) c += __popcll(bm[w * E + i]);
            running[i] += c;
        }
        __syncthreads();
    }
    for (int i = t; i < E; i += 256) chunk_counts[(int64_t)blockIdx.x * E + i] = running[i];
}

// 2) one 1024-thread block: per expert, exclusive prefix of the chunk counts over chunks
// (written back in place), expert offsets, and the GEMM tile list.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ chunk_counts, int n_chunks, int E,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tiles, int32_t* n_tiles,
                                                             int tile_m) {
    __shared__ int part[1024];
    __shared__ int cnt[1024];
    __shared__ int tmp[1024];
    const int t = threadIdx.x;
    const int splits = 1024 / E;
    const int e = t % E, q = t / E;
    const bool act = q < splits;
    const int cb = act ? (int)((int64_t)q * n_chunks / splits) : 0;
    const int ce = act ? (int)((int64_t)(q + 1) * n_chunks / splits) : 0;
    int sum = 0;
    for (int c = cb; c < ce; ++c) sum += chunk_counts[(int64_t)c * E + e];
    part[t] = sum;
    __syncthreads();
    if (act) {
        int run = 0;
        for (int q2 = 0; q2 < q; ++q2) run += part[q2 * E + e];
        for (int c = cb; c < ce; ++c) {
            const int v = chunk_counts[(int64_t)c * E + e];
            chunk_counts[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    __syncthreads();
    if (t < E) {
        int c = 0;
        for (int q2 = 0; q2 < splits; ++q2) c += part[q2 * E + t];
        cnt[t] = c;
    }
    __syncthreads();
    const int total = block_excl_scan(cnt, tmp, E);
    if (t < E) offsets[t] = cnt[t];
    if (t == 0) offsets[E] = total;
    if (tiles) {
        __syncthreads();
        if (t < E) cnt[t] = offsets[t + 1] - offsets[t];
        __syncthreads();
        write_tiles(cnt, tmp, E, tile_m, tiles, n_tiles);
    }
}

// 3) scatter every pair to offsets[e] + (pairs of e in earlier chunks) + rank in chunk.
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ chunk_prefix,
                                                               const int32_t* __restrict__ rank_in_chunk,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ pair_rank) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int e = idx[p];
    if (e >= 0 && e < E) {
        const int pos = offsets[e] + chunk_prefix[(p / kChunkPairs) * E + e] + rank_in_chunk[p];
        sorted_pairs[pos] = (int32_t)p;
        if (pair_rank) pair_rank[p] = pos;
    } else if (pair_rank) {
        pair_rank[p] = -1;
    }
    if (p >= offsets[E]) sorted_pairs[p] = -1;
}

// Expert-parallel share: global expert ids in [e_begin, e_begin + e_count) become local ids
// 0..e_count-1, every other id -1 (the dispatch then leaves that pair out).
__global__ __launch_bounds__(256) void share_idx_kernel(const int32_t* __restrict__ idx, int64_t P, int e_begin,
                                                        int e_count, int32_t* __restrict__ idx_local) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int e = idx[p] - e_begin;
    idx_local[p] = (e >= 0 && e < e_count) ? e : -1;
}

}  // namespace

void launch_share_idx(const int32_t* idx, int64_t P, int e_begin, int e_count, int32_t* idx_local, hipStream_t st) {
    hipLaunchKernelGGL(share_idx_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, st, idx, P, e_begin, e_count,
                       idx_local);
}

void launch_dispatch(const Shape& s, const int32_t* idx, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_rank,
                     int32_t* chunk_counts, int32_t* rank_in_chunk, int32_t* tiles, int32_t* n_tiles, int tile_m,
                     hipStream_t st) {
    const int64_t P = s.T * s.K;
    if (P <= 1024 && s.E <= 256) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, st, idx, (int)P, s.E, offsets,
                           sorted_pairs, pair_rank, tiles, n_tiles, tile_m);
        return;
    }
    const int n_chunks = (int)((P + kChunkPairs - 1) / kChunkPairs);
    const size_t lds = (size_t)kWaves * s.E * sizeof(uint64_t) + (size_t)s.E * sizeof(int);
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(n_chunks), dim3(256), lds, st, idx, P, s.E, chunk_counts,
                       rank_in_chunk);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, chunk_counts, n_chunks, s.E, offsets, tiles,
                       n_tiles, tile_m);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, st, idx, P, s.E,
                       offsets, chunk_counts, rank_in_chunk, sorted_pairs, pair_rank);
}

}  // namespace beam
