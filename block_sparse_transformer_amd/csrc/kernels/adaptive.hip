// adaptive.hip -- content-adaptive block layout, chosen on the device from Q and K.
//
// Adaptive Sparse Transformer page ("Adapt or Perish: 新手入门指南 – Adaptive Sparse
// Transformer 核心原理与实战"), importance evaluation: score the candidate
// positions and keep the highest r% per query.  Here the candidates are the
// 64-token key blocks of the block-sparse storage (SQA page, "Transformer计算效率优化：
// SQA稀疏注意力机制详解", sections 3.1 and 5), scored from block representatives:
//   qs[g, i, d] = sum over u = 0..63 of q[g, 64 i + u, d], added in that order in fp64
//   S[g, i, j]  = sum over d = 0..D-1 of qs[g, i, d] * ks[g, j, d], each product rounded,
//                 added in order of d, in fp64 with no fused multiply-add
// and query block i keeps the `keep` key blocks of highest S, ties to the
// lower index, ascending.  The operations and their order are fixed, so any
// implementation that follows them gets the same bits and the same blocks.
//
// The layout then runs through the ordinary forward: its rows all hold `keep`
// tiles, so the work schedule is data-independent and is built on the host
// with tile entries that hold a position in the row; fill_tiles_kernel
// replaces each position by the chosen key block.
#include <hip/hip_runtime.h>

#include "../internal.h"

namespace bsattn {
namespace {

// One thread per (group, block, d): the block's 64 rows added in order (the
// loads unrolled 16 at a time, ahead of the additions).  Written [g][i][d]
// (transposed = false) or [g][d][i] (transposed = true, so that the threads of
// a wave, one per key block, read consecutive addresses when scoring).
template <int D>
__global__ __launch_bounds__(256) void block_sums_kernel(const uint16_t* x, double* out, int64_t n, int nb,
                                                         bool transposed) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int d = (int)(idx % D);
    const int64_t gi = idx / D;                       // g * nb + i
    const uint16_t* p = x + gi * 64 * D + d;          // row 64 i of group g
    double s = 0.0;
#pragma unroll 16
    for (int u = 0; u < 64; ++u) s += (double)__uint_as_float((uint32_t)p[(size_t)u * D] << 16);
    const int64_t g = gi / nb, i = gi % nb;
    out[transposed ? (g * D + d) * nb + i : idx] = s;
}

constexpr int kSelThreads = 128, kSelWaves = kSelThreads / 64;

// One workgroup per (group, query block).  Thread j scores key block j: its
// key sums (64 at a time, loaded before anything waits, so that they travel
// together with the query block's sums) times the query block's, the rounded
// products added in order of d.  Then each block's rank = #blocks with a
// higher score or an equal score and a lower index; ranks below `keep` are
// kept and written ascending (position = kept blocks before it: a ballot per
// wave plus the counts of the waves before).
template <int D>
__global__ __launch_bounds__(kSelThreads) void select_blocks_kernel(const double* qs, const double* ksT,
                                                                    int32_t* cols, int nb, int keep) {
    __shared__ double sc[kMaxAdaptiveBlocks];
    __shared__ double qrow[D];
    __shared__ int wave_cnt[kMaxAdaptiveBlocks / 64];
    const int gi = blockIdx.x;
    const int g = gi / nb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const double* kbase = ksT + (size_t)g * D * nb;
    double kv[64];
    if (tid < nb) {
#pragma unroll
        for (int e = 0; e < 64; ++e) kv[e] = kbase[(size_t)e * nb + tid];
    }
    for (int d = tid; d < D; d += kSelThreads) qrow[d] = qs[(size_t)gi * D + d];
    __syncthreads();
    for (int j = tid; j < nb; j += kSelThreads) {
#pragma clang fp contract(off)
        double sr = 0.0;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += 64) {
            if (d0 > 0 || j != tid) {
#pragma unroll
                for (int e = 0; e < 64; ++e) kv[e] = kbase[(size_t)(d0 + e) * nb + j];
            }
#pragma unroll
            for (int e = 0; e < 64; ++e) {
                const double p = qrow[d0 + e] * kv[e];
                sr = sr + p;
            }
        }
        sc[j] = sr;
    }
    __syncthreads();
    const int iters = (nb + kSelThreads - 1) / kSelThreads;
    uint64_t masks[kMaxAdaptiveBlocks / kSelThreads];
#pragma unroll
    for (int it = 0; it < kMaxAdaptiveBlocks / kSelThreads; ++it) {
        if (it >= iters) break;
        const int j = it * kSelThreads + tid;
        bool kp = false;
        if (j < nb) {
            const double s = sc[j];
            int rank = 0;
            int jj = 0;
            for (; jj + 16 <= nb; jj += 16) {
                double o[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) o[e] = sc[jj + e];
#pragma unroll
                for (int e = 0; e < 16; ++e) rank += (o[e] > s) || (o[e] == s && jj + e < j);
            }
            for (; jj < nb; ++jj) rank += (sc[jj] > s) || (sc[jj] == s && jj < j);
            kp = rank < keep;
        }
        masks[it] = __ballot(kp);
        if (lane == 0) wave_cnt[it * kSelWaves + wave] = __builtin_popcountll(masks[it]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kMaxAdaptiveBlocks / kSelThreads; ++it) {
        if (it >= iters) break;
        const int j = it * kSelThreads + tid;
        if (j >= nb || !((masks[it] >> lane) & 1ull)) continue;
        int pos = __builtin_popcountll(masks[it] & ((1ull << lane) - 1ull));
        for (int w = 0; w < it * kSelWaves + wave; ++w) pos += wave_cnt[w];
        if (pos < keep) cols[(size_t)gi * keep + pos] = j;
    }
}

// One workgroup per schedule list: tile entry position p of unit (query block
// i, group g) -> key block cols[g][i][p].
__global__ __launch_bounds__(64) void fill_tiles_kernel(const int32_t* skel, int32_t* live, const int4* units,
                                                        const int32_t* unit_ptr, const int32_t* tile_ptr,
                                                        const int32_t* cols, int nb, int keep) {
    const int bin = blockIdx.x;
    const int up0 = unit_ptr[bin];
    const int tp0 = tile_ptr[bin], nt = tile_ptr[bin + 1] - tp0;
    for (int i = threadIdx.x; i < nt; i += 64) {
        const int e = skel[tp0 + i];
        const int4 u = units[up0 + ((e >> kTileUnitShift) & (kMaxBinUnits - 1))];
        const int p = e & kTileJ;
        const int j = cols[((size_t)u.z * nb + u.x) * keep + p];
        live[tp0 + i] = (e & ~kTileJ) | j;
    }
}

}  // namespace

hipError_t launch_adaptive_select(const void* q, const void* k, double* qs, double* ks, int32_t* cols, int G,
                                  int L, int D, int keep, hipStream_t s) {
    const int nb = L / 64;
    const int64_t n = (int64_t)G * nb * D;
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (D == 64) {
        hipLaunchKernelGGL(block_sums_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)q, qs, n, nb, false);
        hipLaunchKernelGGL(block_sums_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)k, ks, n, nb, true);
    } else {
        hipLaunchKernelGGL(block_sums_kernel<128>, grid, dim3(256), 0, s, (const uint16_t*)q, qs, n, nb, false);
        hipLaunchKernelGGL(block_sums_kernel<128>, grid, dim3(256), 0, s, (const uint16_t*)k, ks, n, nb, true);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 sgrid((unsigned)(G * nb));
    if (D == 64)
        hipLaunchKernelGGL(select_blocks_kernel<64>, sgrid, dim3(kSelThreads), 0, s, qs, ks, cols, nb, keep);
    else
        hipLaunchKernelGGL(select_blocks_kernel<128>, sgrid, dim3(kSelThreads), 0, s, qs, ks, cols, nb, keep);
    return hipGetLastError();
}

hipError_t launch_fill_tiles(const int32_t* skel, int32_t* live, const int4* units, const int32_t* unit_ptr,
                             const int32_t* tile_ptr, int n_lists, const int32_t* cols, int nb, int keep,
                             hipStream_t s) {
    if (n_lists == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_tiles_kernel, dim3((unsigned)n_lists), dim3(64), 0, s, skel, live, units, unit_ptr,
                       tile_ptr, cols, nb, keep);
    return hipGetLastError();
}

}  // namespace bsattn
