// router.hip -- routed-query selection: exact fp64 score q.w and per-head top-k.
//
// SQA page ("Transformer计算效率优化：SQA稀疏注意力机制详解"), section 2.1: a linear
// router scores every query and the top-k queries attend to all keys;
// section 3.2: the router is kept at higher precision than the model.
//
// score[t] = sum_d (double)q[t,d] * (double)w[d], added left to right in d.
// A bf16 x fp32 product has at most 32 significant bits, so each product is
// exact in fp64 and only the additions round: the value is reproducible bit
// for bit by any implementation that adds in the same order (fused or not).
// Rows are ordered by (score descending, row ascending): ties go to the
// lower row.
//
// Two launches.  route_score_kernel: one wave per 64 rows of a (b, h); the
// rows are staged through LDS with coalesced loads, then every lane runs its
// row's sequential fp64 chain and writes the score to the workspace.
// route_select_kernel: one workgroup per (b, h), no sort of the whole row
// set.  Scores become 64-bit keys whose unsigned order is the score order
// (NaN lowest); a 256-bin histogram over the finite range, with a bin index
// that never decreases with the score, finds the bin holding the k-th best
// row; only that bin's rows are sorted, by (key descending, row ascending),
// and its need-th entry is the threshold pair.  A row is routed iff it ranks
// before or at that pair, exactly the top k, and a workgroup scan writes
// those rows in ascending order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../internal.h"

namespace bsattn {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 256;

// ---------------- scores ----------------

// One wave: rows t0 .. t0 + 63 of one (b, h).  LDS row stride D * 2 + 16
// bytes keeps the lanes' 16-byte row reads free of bank conflicts.
template <int D>
__global__ __launch_bounds__(64) void route_score_kernel(const uint16_t* q, const float* w, int L, int n_tiles,
                                                         double* scores) {
    constexpr int kStride = D * 2 + 16;          // bytes per staged row
    constexpr int kPieces = D / 8;               // 16-byte pieces per row
    __shared__ __attribute__((aligned(16))) unsigned char rows[64 * kStride];
    __shared__ __attribute__((aligned(16))) double wd[D];
    const int lane = threadIdx.x;
    const size_t bh = blockIdx.x / n_tiles;
    const int t0 = (blockIdx.x % n_tiles) * 64;
    const int n_rows = min(64, L - t0);
    const uint4* src = (const uint4*)(q + (bh * (size_t)L + t0) * D);
    // every load of the 64 rows is issued before any is stored, so the wave
    // waits for memory once instead of once per 16-byte piece
    uint4 u[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        const int p = lane + 64 * i;
        u[i] = make_uint4(0, 0, 0, 0);
        if (p / kPieces < n_rows) u[i] = src[p];
    }
    float wf[(D + 63) / 64];
#pragma unroll
    for (int i = 0; i < (D + 63) / 64; ++i) wf[i] = lane + 64 * i < D ? w[lane + 64 * i] : 0.f;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        const int p = lane + 64 * i;
        *(uint4*)(rows + (p / kPieces) * kStride + (p % kPieces) * 16) = u[i];
    }
#pragma unroll
    for (int i = 0; i < (D + 63) / 64; ++i)
        if (lane + 64 * i < D) wd[lane + 64 * i] = (double)wf[i];
    __syncthreads();
    if (lane >= n_rows) return;
    const unsigned char* row = rows + lane * kStride;
    double acc = 0.0;
#pragma unroll 4
    for (int c = 0; c < kPieces; ++c) {
        const uint4 u = *(const uint4*)(row + c * 16);
        const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = (double)__uint_as_float(v[e] << 16);
            const double hi = (double)__uint_as_float(v[e] & 0xffff0000u);
            acc = fma(lo, wd[c * 8 + 2 * e], acc);      // the product is exact: same bits as mul then add
            acc = fma(hi, wd[c * 8 + 2 * e + 1], acc);
        }
    }
    scores[bh * (size_t)L + t0 + lane] = acc;
}

// ---------------- selection ----------------

// Unsigned key in score order: +0 and -0 alike, NaN below everything.
__device__ __forceinline__ uint64_t score_key(double s) {
    if (s != s) return 0;
    if (s == 0.0) s = 0.0;
    const uint64_t b = (uint64_t)__double_as_longlong(s);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Bin of a score: 0 for NaN and for s <= lo, 255 for s >= hi, else
// floor((s - lo) * inv) capped at 255.  Each step is monotone, so the bin
// never decreases as the key grows.
__device__ __forceinline__ int score_bin(double s, double lo, double hi, double inv) {
    if (!(s > lo)) return 0;
    if (s >= hi) return kBins - 1;
    const double x = (s - lo) * inv;
    return x >= (double)(kBins - 1) ? kBins - 1 : (int)x;
}

// x ranks before y in (key descending, row ascending)
__device__ __forceinline__ bool ranks_before(uint64_t kx, int rx, uint64_t ky, int ry) {
    return kx > ky || (kx == ky && rx < ry);
}

template <int R>
__global__ __launch_bounds__(kSelThreads) void route_select_kernel(const double* scores, int L, int k, int CP,
                                                                   int32_t* out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    __shared__ int hist[kBins];
    __shared__ double red_lo[kSelWaves], red_hi[kSelWaves];
    __shared__ int wave_tot[kSelWaves];
    __shared__ int s_bin, s_above, s_count;
    __shared__ uint64_t s_tkey;
    __shared__ int s_trow;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = blockIdx.x;
    const double* sp = scores + bh * (size_t)L;

    // this thread's rows: tid * R .. tid * R + R - 1 (ascending across threads)
    double s[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int t = tid * R + j;
        s[j] = t < L ? sp[t] : NAN;
    }
    // finite range
    double lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (isfinite(s[j])) { lo = fmin(lo, s[j]); hi = fmax(hi, s[j]); }
    for (int off = 32; off > 0; off >>= 1) {
        lo = fmin(lo, __shfl_xor(lo, off));
        hi = fmax(hi, __shfl_xor(hi, off));
    }
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    if (lane == 0) { red_lo[wave] = lo; red_hi[wave] = hi; }
    if (tid == 0) s_count = 0;
    __syncthreads();
    lo = red_lo[0]; hi = red_hi[0];
    for (int i = 1; i < kSelWaves; ++i) { lo = fmin(lo, red_lo[i]); hi = fmax(hi, red_hi[i]); }
    const double span = hi - lo;
    const double inv = (hi > lo && isfinite(span)) ? (double)kBins / span : 0.0;

    int bin[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int t = tid * R + j;
        bin[j] = score_bin(s[j], lo, hi, inv);
        if (t < L) atomicAdd(&hist[bin[j]], 1);
    }
    __syncthreads();

    // the bin b with (rows in bins above b) < k <= (rows in bins from b up)
    if (wave == 0) {
        int h[4], own = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { h[i] = hist[lane * 4 + i]; own += h[i]; }
        int suffix = own;                       // rows in this lane's bins and every higher lane's
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_down(suffix, off);
            if (lane + off < 64) suffix += o;
        }
        int above = suffix - own;               // rows in higher lanes' bins
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            if (above < k && k <= above + h[i]) { s_bin = lane * 4 + i; s_above = above; }
            above += h[i];
        }
    }
    __syncthreads();
    const int bsel = s_bin;
    const int need = k - s_above;               // 1 <= need <= rows in bin bsel

    // that bin's rows -> LDS candidates (wave-aggregated slots)
    uint64_t* ckey = (uint64_t*)sm;             // [CP], CP a power of two >= L
    int* crow = (int*)(ckey + CP);              // [CP]
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int t = tid * R + j;
        const bool is = t < L && bin[j] == bsel;
        const uint64_t m = __ballot(is);
        if (m == 0) continue;
        const int leader = __ffsll((unsigned long long)m) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&s_count, __popcll(m));
        base = __shfl(base, leader);
        if (is) {
            const int slot = base + __popcll(m & ((1ull << lane) - 1));
            ckey[slot] = score_key(s[j]);
            crow[slot] = t;
        }
    }
    __syncthreads();
    const int c = s_count;
    int n = 1;
    while (n < c) n <<= 1;
    for (int i = c + tid; i < n; i += kSelThreads) { ckey[i] = 0; crow[i] = 0x7fffffff; }
    __syncthreads();
    // bitonic sort of the n candidates, best first
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n; i += kSelThreads) {
                const int jj = i ^ stride;
                if (jj > i) {
                    const uint64_t ki = ckey[i], kj = ckey[jj];
                    const int ri = crow[i], rj = crow[jj];
                    if (ranks_before(kj, rj, ki, ri) == ((i & size) == 0)) {
                        ckey[i] = kj; ckey[jj] = ki;
                        crow[i] = rj; crow[jj] = ri;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (tid == 0) { s_tkey = ckey[need - 1]; s_trow = crow[need - 1]; }
    __syncthreads();
    const uint64_t tkey = s_tkey;
    const int trow = s_trow;

    // routed iff ranked before or at the threshold pair; write ascending
    int mine = 0;
    bool sel[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int t = tid * R + j;
        const uint64_t key = score_key(s[j]);
        sel[j] = t < L && (key > tkey || (key == tkey && t <= trow));
        mine += sel[j];
    }
    int incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int pos = incl - mine;
    for (int i = 0; i < wave; ++i) pos += wave_tot[i];
    int32_t* op = out + bh * (size_t)k;
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (sel[j] && pos < k) op[pos++] = tid * R + j;   // exactly k rows are routed
}

template <int R>
hipError_t launch_select(const double* scores, int B, int H, int L, int k, int32_t* out, hipStream_t s) {
    int cp = 1;
    while (cp < L) cp <<= 1;
    const size_t lds = (size_t)cp * (sizeof(uint64_t) + sizeof(int));
    hipError_t e = hipFuncSetAttribute((const void*)route_select_kernel<R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_select_kernel<R>, dim3((unsigned)((int64_t)B * H)), dim3(kSelThreads), lds, s, scores,
                       L, k, cp, out);
    return hipGetLastError();
}

}  // namespace

size_t route_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t) {
    return (size_t)B * H * L * sizeof(double);
}

hipError_t launch_route_topk(const void* q, const float* w, int32_t B, int32_t H, int32_t L, int32_t D,
                             int32_t k, int32_t* out, void* workspace, hipStream_t s) {
    double* scores = (double*)workspace;
    const int n_tiles = (L + 63) / 64;
    const dim3 grid((unsigned)((int64_t)B * H * n_tiles));
    if (D == 64)
        hipLaunchKernelGGL(route_score_kernel<64>, grid, dim3(64), 0, s, (const uint16_t*)q, w, L, n_tiles, scores);
    else
        hipLaunchKernelGGL(route_score_kernel<128>, grid, dim3(64), 0, s, (const uint16_t*)q, w, L, n_tiles, scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int R = (L + kSelThreads - 1) / kSelThreads;
    if (R <= 1) return launch_select<1>(scores, B, H, L, k, out, s);
    if (R <= 2) return launch_select<2>(scores, B, H, L, k, out, s);
    if (R <= 4) return launch_select<4>(scores, B, H, L, k, out, s);
    return launch_select<8>(scores, B, H, L, k, out, s);
}

}  // namespace bsattn
