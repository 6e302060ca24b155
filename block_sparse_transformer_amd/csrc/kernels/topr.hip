// topr.hip -- per-query top-keep key selection.
//
// Adaptive Sparse Transformer page ("Adapt or Perish: 新手入门指南 – Adaptive
// Sparse Transformer 核心原理与实战"), the importance-evaluation step: every
// query keeps the keys with the highest scores (⌊L·r⌋ of them) and attends to
// those alone.  The kept set is an integer decision, so it is taken on a
// score with a fixed evaluation: q·k in fp32, products added in order of d
// from +0 (each bf16 x bf16 product is exact in fp32, so fused and unfused
// give the same bits), keys ranked by (score descending, index ascending).
//
// topr_select_kernel<TPQ, D>: one workgroup of 256 threads holds QW = 256/TPQ
// queries of one (batch, head); TPQ threads share a query.  For every key
// tile of 64 keys (staged in LDS as fp32, d-major, keys permuted so that a
// thread's KPT = 64/TPQ keys are adjacent) each thread runs the exact chains
// of its keys and keeps the scores in registers (L/TPQ <= 128 per thread).
// Each score becomes a 32-bit key whose unsigned order is the score order
// (-0 = +0, NaN lowest).  A radix select, four passes of 8 bits with a
// 256-bin LDS histogram per query, finds the exact keep-th largest key T and
// how many keys equal to T are kept; those are the lowest-index ones, counted
// in index order with ballots.  The result is one 64-bit word per (query, key
// tile): bit b set iff key 64j + b is kept.
//
// topr_select_ks_kernel<KPL> (D = 64, L <= 2048) turns this around: the keys
// stay in registers and the queries arrive as scalar operands, so the FMA
// loop reads no LDS (the LDS-tiled kernel above is bound by its key reads).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../internal.h"

namespace bsattn {
namespace {

constexpr int kSelThreads = 256;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// unsigned key in score order: -0 and +0 alike, NaN below everything
__device__ __forceinline__ uint32_t order_key(float s) {
    if (s != s) return 0u;
    if (s == 0.f) s = 0.f;
    const uint32_t b = __float_as_uint(s);
    return (b >> 31) ? ~b : (b | 0x80000000u);
}

template <int TPQ, int D>
__global__ __launch_bounds__(kSelThreads) void topr_select_kernel(const uint16_t* q, const uint16_t* k, uint64_t* bits,
                                                                  int L, int keep, int qtiles) {
    constexpr int QW = kSelThreads / TPQ;        // queries per workgroup
    constexpr int KPT = 64 / TPQ;                // keys per thread per key tile
    constexpr int NTMAX = 128 / KPT;             // key tiles a thread's registers hold
    constexpr int BPL = 256 / TPQ;               // histogram bins per lane
    constexpr int PIECES = 64 * D / 8 / kSelThreads;   // 16-byte pieces of a K tile per thread
    static_assert(PIECES >= 1, "tile pieces");
    __shared__ __attribute__((aligned(16))) float qs[QW][D];
    __shared__ __attribute__((aligned(16))) float kt[D][64];
    __shared__ uint32_t hist[QW][256];
    __shared__ uint32_t s_digit[QW], s_above[QW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int qi = tid / TPQ, tq = tid % TPQ;
    const int gbase = (lane / TPQ) * TPQ;        // first lane of this query's group in the wave
    const uint64_t gmask = TPQ == 64 ? ~0ull : ((1ull << TPQ) - 1ull);
    const size_t g = blockIdx.x / qtiles;
    const int t0 = (blockIdx.x % qtiles) * QW;
    const int nt = L / 64;

    for (int i = tid; i < QW * D; i += kSelThreads) {
        const int r = i / D, d = i % D;
        qs[r][d] = bf16_bits_to_float(q[(g * L + t0 + r) * D + d]);
    }
    const uint4* kg = (const uint4*)(k + g * (size_t)L * D);
    uint4 pre[PIECES];
    auto fetch = [&](int m) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) pre[p] = kg[(size_t)m * (64 * D / 8) + p * kSelThreads + tid];
    };
    // piece p of the tile: key r = p / (D / 8), columns d0 .. d0 + 7; key r sits
    // at position KPT * (r % TPQ) + r / TPQ
    auto stage = [&]() {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int piece = p * kSelThreads + tid;
            const int r = piece / (D / 8), d0 = (piece % (D / 8)) * 8;
            const int pos = KPT * (r % TPQ) + r / TPQ;
            const uint32_t w[4] = {pre[p].x, pre[p].y, pre[p].z, pre[p].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kt[d0 + 2 * e][pos] = bf16_bits_to_float(w[e] & 0xffffu);
                kt[d0 + 2 * e + 1][pos] = bf16_bits_to_float(w[e] >> 16);
            }
        }
    };

    // ---- exact scores, kept as order keys ----
    uint32_t key[NTMAX * KPT];
    fetch(0);
#pragma unroll
    for (int m = 0; m < NTMAX; ++m) {
        if (m < nt) {
            __syncthreads();                 // previous tile's readers are done
            stage();
            __syncthreads();
            if (m + 1 < nt) fetch(m + 1);    // in flight while this tile is scored
            float acc[KPT];
#pragma unroll
            for (int e = 0; e < KPT; ++e) acc[e] = 0.f;
#pragma unroll 4
            for (int d = 0; d < D; d += 4) {
                const float4 qv = *(const float4*)&qs[qi][d];
                const float qd[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const float* kr = &kt[d + dd][KPT * tq];
#pragma unroll
                    for (int e = 0; e < KPT; ++e) acc[e] = fmaf(qd[dd], kr[e], acc[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < KPT; ++e) key[m * KPT + e] = order_key(acc[e]);
        }
    }

    // ---- radix select of the keep-th largest key ----
    uint32_t prefix = 0;
    int need = keep;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int b = tq; b < 256; b += TPQ) hist[qi][b] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NTMAX * KPT; ++i) {
            if (i / KPT < nt) {
                const uint32_t kk = key[i];
                const bool match = pass == 0 || (kk >> (shift + 8)) == (prefix >> (shift + 8));
                if (match) atomicAdd(&hist[qi][(kk >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        uint32_t h[BPL], own = 0;
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            h[j] = hist[qi][tq * BPL + j];
            own += h[j];
        }
        uint32_t suffix = own;               // this lane's bins and those of higher lanes of the group
#pragma unroll
        for (int off = 1; off < TPQ; off <<= 1) {
            const uint32_t o = __shfl_down(suffix, off, TPQ);
            if (tq + off < TPQ) suffix += o;
        }
        uint32_t above = suffix - own;
#pragma unroll
        for (int j = BPL - 1; j >= 0; --j) {
            if (above < (uint32_t)need && (uint32_t)need <= above + h[j]) {
                s_digit[qi] = (uint32_t)(tq * BPL + j);
                s_above[qi] = above;
            }
            above += h[j];
        }
        __syncthreads();
        prefix |= s_digit[qi] << shift;
        need -= (int)s_above[qi];
        __syncthreads();                     // s_digit / hist are rewritten next pass
    }

    // ---- kept iff key > T, or key == T among the first `need` in index order ----
    const uint32_t T = prefix;
    uint32_t running = 0;
    uint64_t words[NTMAX / TPQ > 0 ? NTMAX / TPQ : 1];
#pragma unroll
    for (int j = 0; j < (NTMAX / TPQ > 0 ? NTMAX / TPQ : 1); ++j) words[j] = 0;
#pragma unroll
    for (int m = 0; m < NTMAX; ++m) {
        if (m < nt) {
            uint64_t word = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint32_t kk = key[m * KPT + e];
                const bool eq = kk == T;
                const uint64_t es = (__ballot(eq) >> gbase) & gmask;
                const uint32_t rank = running + (uint32_t)__popcll(es & ((1ull << tq) - 1ull));
                running += (uint32_t)__popcll(es);
                const bool sel = kk > T || (eq && rank < (uint32_t)need);
                const uint64_t ss = (__ballot(sel) >> gbase) & gmask;
                word |= ss << (TPQ * e);     // key 64m + tq' + TPQ e  ->  bit tq' + TPQ e
            }
            if (tq == m % TPQ) words[m / TPQ] = word;
        }
    }
    uint64_t* out = bits + (g * L + t0 + qi) * (size_t)nt;
#pragma unroll
    for (int j = 0; j < (NTMAX / TPQ > 0 ? NTMAX / TPQ : 1); ++j) {
        const int m = tq + TPQ * j;
        if (m < nt) out[m] = words[j];
    }
}

// Launched with hipExtLaunchKernelGGL: given events, the dispatch itself
// records the kernel's start and stop.
// Key-stationary selection, D = 64, L <= 1024 KPL: one workgroup of 1024
// threads per (batch, head, chunk of queries).  Lane `lane` of wave w holds the
// KPL keys s = (w KPL + j) 64 + lane in registers as packed bf16; the queries
// come in batches of QB, their values as scalar operands, so the in-order
// FMA chains read nothing from LDS.  Each batch's QB queries then share one
// radix select (LDS histograms, a wave per query scans), ties are ranked in
// index order from per-tile counts, and the kept-key word of tile w KPL + j is
// the wave's ballot.
// Inclusive prefix sum over the 64 lanes of a wave by DPP lane moves (no LDS
// round trips): sums of four within each row of 16 from three shifted adds,
// then the rows' halves (shift by 4 into banks 1-3, by 8 into banks 2-3), then
// the rows (lane 15 of each row into the next odd row, lane 31 into rows 2 and
// 3).  Lanes a move leaves without a source add 0.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
    const int xi = (int)x;
    int s = xi + __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xF, 0xF, true);   // row_shr:1
    s += __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xF, 0xF, true);           // row_shr:2
    s += __builtin_amdgcn_update_dpp(0, xi, 0x113, 0xF, 0xF, true);           // row_shr:3
    s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, false);           // row_shr:4, banks 1-3
    s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, false);           // row_shr:8, banks 2-3
    s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);           // row_bcast:15, rows 1, 3
    s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);           // row_bcast:31, rows 2, 3
    return (uint32_t)s;
}

constexpr int kKsThreads = 1024;
constexpr int kKsWaves = kKsThreads / 64;
constexpr int kKsBatch = 8;

template <int KPL>
__global__ __launch_bounds__(kKsThreads) void topr_select_ks_kernel(const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ k,
                                                                    uint64_t* __restrict__ bits, int L, int keep,
                                                                    int chunk, int nchunks) {
    constexpr int D = 64;
    constexpr int QB = kKsBatch;
    constexpr int NTILE = kKsWaves * KPL;          // key tiles a workgroup covers
    // two sets of histograms and scan results, used by alternate passes: a
    // pass's scan clears its own set for the pass after next, so a pass needs
    // no barrier before its atomics and none after its results are read
    __shared__ uint32_t hist[2][QB][256];
    __shared__ uint32_t s_digit[2][QB], s_above[2][QB];
    __shared__ uint32_t s_tie[QB];                  // some keys equal to T are dropped
    __shared__ uint32_t eqc[QB][NTILE];             // keys equal to T per (query, tile), then their prefix
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t g = blockIdx.x / nchunks;
    const int c0 = (blockIdx.x % nchunks) * chunk;
    const int c1 = min(L, c0 + chunk);
    const int nt = L / 64;

    // this lane's keys, packed bf16 pairs
    uint32_t kp[KPL][D / 2];
    bool kvalid[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int m = wave * KPL + j;
        kvalid[j] = m < nt;
        const uint4* src = (const uint4*)(k + (g * L + (size_t)(kvalid[j] ? m : 0) * 64 + lane) * D);
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            const uint4 u = kvalid[j] ? src[c] : make_uint4(0, 0, 0, 0);
            kp[j][4 * c + 0] = u.x; kp[j][4 * c + 1] = u.y; kp[j][4 * c + 2] = u.z; kp[j][4 * c + 3] = u.w;
        }
    }
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int x = tid; x < 2 * QB * 256; x += kKsThreads) (&hist[0][0][0])[x] = 0u;
    __syncthreads();

    for (int t0 = c0; t0 < c1; t0 += QB) {
        constexpr int nq = QB;   // chunks and L are multiples of QB: every batch is full
        // keep the keys packed: without this the compiler converts all of them
        // to fp32 once, ahead of the loop, and runs out of registers
#pragma unroll
        for (int j = 0; j < KPL; ++j)
#pragma unroll
            for (int x = 0; x < D / 2; ++x) asm volatile("" : "+v"(kp[j][x]));
        // ---- exact in-order scores of the batch's queries against this lane's keys ----
        float acc[QB][KPL];
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < KPL; ++j) acc[i][j] = 0.f;
        // the batch's q values are uniform: scalar loads from one base (rows D
        // elements apart), 4 d (2 packed pairs) per chunk, the next chunk's
        // issued before this chunk's FMAs; a scheduling fence per chunk bounds
        // how many are live
        const uint32_t* qbase = (const uint32_t*)(q + (g * L + (size_t)t0) * D);
        uint32_t qa[QB][2], qn[QB][2];
        auto loadq = [&](int c, uint32_t (&dst)[QB][2]) {
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                const uint2 u = *(const uint2*)(qbase + i * (D / 2) + 2 * c);
                dst[i][0] = u.x; dst[i][1] = u.y;
            }
        };
        loadq(0, qa);
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            if (c + 1 < D / 4) loadq(c + 1, qn);
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int hi = 0; hi < 2; ++hi) {
                    float kf[KPL];
#pragma unroll
                    for (int j = 0; j < KPL; ++j) {
                        const uint32_t w = kp[j][2 * c + e];
                        kf[j] = __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
                    }
#pragma unroll
                    for (int i = 0; i < QB; ++i) {
                        const uint32_t w = qa[i][e];
                        const float qv = __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
#pragma unroll
                        for (int j = 0; j < KPL; ++j) acc[i][j] = fmaf(qv, kf[j], acc[i][j]);
                    }
                }
            // this chunk's FMAs all come before this point and the next chunk's
            // after it (the accumulators pass through it), so only two chunks'
            // q values are live and QB x KPL independent chains interleave
#pragma unroll
            for (int i = 0; i < QB; ++i)
#pragma unroll
                for (int j = 0; j < KPL; ++j) asm volatile("" : "+v"(acc[i][j]));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (c + 1 < D / 4) {
#pragma unroll
                for (int i = 0; i < QB; ++i) { qa[i][0] = qn[i][0]; qa[i][1] = qn[i][1]; }
            }
        }
        uint32_t key[QB][KPL];
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < KPL; ++j) key[i][j] = order_key(acc[i][j]);

        // ---- radix select of each query's keep-th largest key ----
        uint32_t prefix[QB];
        int need[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) { prefix[i] = 0; need[i] = keep; }
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            const int hb = pass & 1;
#pragma unroll
            for (int i = 0; i < QB; ++i)
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const uint32_t kk = key[i][j];
                    const bool match = pass == 0 || (kk >> (shift + 8)) == (prefix[i] >> (shift + 8));
                    if (i < nq && kvalid[j] && match) atomicAdd(&hist[hb][i][(kk >> shift) & 255u], 1u);
                }
            __syncthreads();
            if (wave < nq) {
                // one wave per query: lane l owns bins 255 - 4l - b, b = 0 .. 3
                // (lane 0 the highest), read and cleared; the keys above a
                // lane's bins are the prefix sum over the lanes before it
                const int qi = wave;
                uint32_t h[4], own = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    h[b] = hist[hb][qi][255 - 4 * lane - b];
                    own += h[b];
                    hist[hb][qi][255 - 4 * lane - b] = 0u;
                }
                uint32_t above = wave_prefix_sum(own) - own;
                int nd = need[0];
#pragma unroll
                for (int x = 1; x < QB; ++x)
                    if (qi == x) nd = need[x];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if (above < (uint32_t)nd && (uint32_t)nd <= above + h[b]) {
                        s_digit[hb][qi] = (uint32_t)(255 - 4 * lane - b);
                        s_above[hb][qi] = above;
                        // last pass: h[b] keys equal T, and nd - above of them are kept
                        if (pass == 3) s_tie[qi] = (uint32_t)nd - above != h[b];
                    }
                    above += h[b];
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < QB; ++i)
                if (i < nq) {
                    prefix[i] |= s_digit[hb][i] << shift;
                    need[i] -= (int)s_above[hb][i];
                }
        }

        // ---- ties: rank keys equal to T in index order (tile, lane) ----
        // Only needed when some keys equal to T are dropped; with continuous
        // scores T is almost always unique, and every key equal to it is kept.
        bool any_tie = false;
#pragma unroll
        for (int i = 0; i < QB; ++i) any_tie = any_tie || (i < nq && s_tie[i] != 0u);
        if (any_tie) {
#pragma unroll
            for (int i = 0; i < QB; ++i)
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const uint64_t eb = __ballot(i < nq && kvalid[j] && key[i][j] == prefix[i]);
                    if (lane == 0) eqc[i][wave * KPL + j] = (uint32_t)__popcll(eb);
                }
            __syncthreads();
            if (wave < QB) {
                // exclusive prefix of query `wave`'s per-tile counts, one tile per lane
                const uint32_t c = lane < NTILE ? eqc[wave][lane] : 0u;
                uint32_t incl = c;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = __shfl_up(incl, off);
                    if (lane >= off) incl += o;
                }
                if (lane < NTILE) eqc[wave][lane] = incl - c;
            }
            __syncthreads();
        }
        uint64_t myword = 0;
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const uint32_t kk = key[i][j];
                const bool eq = i < nq && kvalid[j] && kk == prefix[i];
                bool take_eq = eq;
                if (any_tie) {
                    const uint64_t eb = __ballot(eq);
                    const uint32_t rank = eqc[i][wave * KPL + j] + (uint32_t)__popcll(eb & lt_mask);
                    take_eq = eq && rank < (uint32_t)need[i];
                }
                const bool sel = i < nq && kvalid[j] && (kk > prefix[i] || take_eq);
                const uint64_t word = __ballot(sel);
                if (lane == i * KPL + j) myword = word;
            }
        // lane i KPL + j writes the word of query i, tile wave KPL + j
        {
            const int i = lane / KPL, j = lane % KPL;
            const int m = wave * KPL + j;
            if (lane < QB * KPL && i < nq && m < nt) bits[(g * L + t0 + i) * (size_t)nt + m] = myword;
        }
        // No barrier here: the next batch writes LDS (its pass 0 histogram,
        // cleared by this batch's pass 2, and eqc) only after barriers that
        // every thread reaches once done with this batch's reads.
    }
}

template <int TPQ, int D>
hipError_t launch_t(const void* q, const void* k, uint64_t* bits, int G, int L, int keep, hipStream_t s,
                    hipEvent_t before, hipEvent_t after) {
    constexpr int QW = kSelThreads / TPQ;
    const int qtiles = L / QW;
    hipExtLaunchKernelGGL((topr_select_kernel<TPQ, D>), dim3((unsigned)((int64_t)G * qtiles)), dim3(kSelThreads), 0,
                          s, before, after, 0, (const uint16_t*)q, (const uint16_t*)k, bits, L, keep, qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topr_select(const void* q, const void* k, uint64_t* bits, int G, int L, int D, int keep,
                              hipStream_t s, hipEvent_t before, hipEvent_t after) {
    if (L % 64 != 0 || L > kMaxTopLen || keep < 1 || keep > L || (D != 64 && D != 128)) return hipErrorInvalidValue;
    if (D == 64 && L <= 2 * kKsThreads) {
        // key-stationary: at most one workgroup per CU (a second round of
        // workgroups would double the time), each over a chunk of queries
        int nchunks = G >= 256 ? 1 : 256 / G;
        int chunk = (L + nchunks - 1) / nchunks;
        chunk = (chunk + kKsBatch - 1) / kKsBatch * kKsBatch;
        nchunks = (L + chunk - 1) / chunk;
        const dim3 grid((unsigned)((int64_t)G * nchunks));
        if (L <= kKsThreads)
            hipExtLaunchKernelGGL((topr_select_ks_kernel<1>), grid, dim3(kKsThreads), 0, s, before, after, 0,
                                  (const uint16_t*)q, (const uint16_t*)k, bits, L, keep, chunk, nchunks);
        else
            hipExtLaunchKernelGGL((topr_select_ks_kernel<2>), grid, dim3(kKsThreads), 0, s, before, after, 0,
                                  (const uint16_t*)q, (const uint16_t*)k, bits, L, keep, chunk, nchunks);
        return hipGetLastError();
    }
    if (L <= 2048)
        return D == 64 ? launch_t<16, 64>(q, k, bits, G, L, keep, s, before, after)
                       : launch_t<16, 128>(q, k, bits, G, L, keep, s, before, after);
    if (L <= 4096)
        return D == 64 ? launch_t<32, 64>(q, k, bits, G, L, keep, s, before, after)
                       : launch_t<32, 128>(q, k, bits, G, L, keep, s, before, after);
    return D == 64 ? launch_t<64, 64>(q, k, bits, G, L, keep, s, before, after)
                   : launch_t<64, 128>(q, k, bits, G, L, keep, s, before, after);
}

}  // namespace bsattn
