// candidates.hip -- candidate-list attention: the candidate generator and the
// importance evaluation of the Adaptive Sparse Transformer page ("Adapt or
// Perish: 新手入门指南 – Adaptive Sparse Transformer 核心原理与实战").
//
// cand_positions_kernel: a Conv1d of the hidden states x [B, L, C] (k output
// channels, kernel 3, padding 1, bias) predicts k key positions per query.
// The position is the output rounded to the nearest token (ties to even) and
// clamped to [0, L - 1] (NaN -> 0), an integer decision taken from floating
// point, so the sum has one fixed evaluation: fp64, from bias[j], adding the
// products of tap u = 0, 1, 2 in turn and, within a tap, of channel c = 0 ..
// C - 1.  A bf16 x fp32 product is exact in fp64 (fused or not); taps
// outside the sequence add nothing.  A thread runs the chain of one (token,
// output); the fp64 chains are latency-bound (see the kernel and the design
// notes for the variants measured).
//
// cand_attention_kernel: one wave per (batch, head, query).  Lane j < k holds
// candidate position j; a position seen in a lower lane is dropped (the
// candidate set).  Each remaining lane takes the in-order fp32 score q.k of
// its key (products added in order of d from +0, as the top-keep selection
// does), the lanes are ranked by (score descending, position ascending) and
// the first `keep` are kept.  The softmax of scale * score over the kept keys
// then weighs their V rows: every lane owns D/64 output columns and walks the
// kept keys, eight V rows per round of loads, so each row is read once,
// coalesced.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "../internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// One chain per thread: output j of token t, a workgroup holding 256 / kp
// tokens x kp outputs.  The kp lanes of a token read the same x element (one
// cached load) and, with the weights tap-major, k consecutive weights.
constexpr int kPosThreads = 256;

__global__ __launch_bounds__(kPosThreads) void cand_positions_kernel(const uint16_t* __restrict__ x,
                                                                     const float* __restrict__ w,
                                                                     const float* __restrict__ bias, int L, int C,
                                                                     int k, int kp, int32_t* __restrict__ pos) {
    const int T = kPosThreads / kp;
    const int tiles = (L + T - 1) / T;
    const int b = blockIdx.x / tiles;
    const int j = threadIdx.x % kp;
    const int t = (blockIdx.x % tiles) * T + threadIdx.x / kp;
    if (j >= k || t >= L) return;
    const uint16_t* xb = x + (size_t)b * L * C;
    double acc = (double)bias[j];
#pragma unroll 1
    for (int u = 0; u < 3; ++u) {
        const int row = t + u - 1;
        if (row < 0 || row >= L) continue;   // padding: the tap adds nothing
        const uint16_t* xr = xb + (size_t)row * C;
        const float* wu = w + (size_t)u * C * k + j;
#pragma unroll 4
        for (int c = 0; c < C; ++c)
            acc = fma((double)__uint_as_float((uint32_t)xr[c] << 16), (double)wu[(size_t)c * k], acc);
    }
    int p;
    if (acc != acc) p = 0;
    else p = (int)fmin(fmax(rint(acc), 0.0), (double)(L - 1));
    pos[((size_t)b * L + t) * k + j] = p;
}

// unsigned key in score order: -0 and +0 alike, NaN below everything
__device__ __forceinline__ uint32_t order_key(float s) {
    if (s != s) return 0u;
    if (s == 0.f) s = 0.f;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D>
__global__ __launch_bounds__(256) void cand_attention_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ kk,
                                                             const uint16_t* __restrict__ v,
                                                             const int32_t* __restrict__ pos, int H, int L, int k,
                                                             int keep, float scale, uint16_t* __restrict__ out,
                                                             float* __restrict__ lse, int32_t* __restrict__ kept_out,
                                                             int64_t n_queries) {
    constexpr int DL = D / 64;   // output columns per lane
    const int lane = threadIdx.x & 63;
    const int64_t qi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (qi >= n_queries) return;   // the whole wave
    const int t = (int)(qi % L);
    const int64_t g = qi / L;      // b * H + h
    const int b = (int)(g / H);
    const uint16_t* kb = kk + (size_t)g * L * D;
    const uint16_t* vb = v + (size_t)g * L * D;
    // candidate position of this lane (-1: none; positions outside the sequence are ignored)
    int p = lane < k ? pos[((size_t)b * L + t) * k + lane] : -1;
    if (p < 0 || p >= L) p = -1;
    bool valid = p >= 0;
    // (readlane with a loop-uniform lane: a scalar read, not an LDS permute)
    for (int i = 0; i < k; ++i) {   // a position already held by a lower lane is dropped
        const int pi = __builtin_amdgcn_readlane(p, i);
        valid = valid && !(i < lane && pi == p);
    }
    // in-order fp32 score of this lane's key
    const uint16_t* qr = q + ((size_t)g * L + t) * D;
    float s = 0.f;
    if (valid) {
        const uint16_t* kr = kb + (size_t)p * D;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            const u32x4_t qw = *(const u32x4_t*)(qr + 8 * c);
            const u32x4_t kw = *(const u32x4_t*)(kr + 8 * c);
            const uint32_t qe[4] = {qw.x, qw.y, qw.z, qw.w}, ke[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = fmaf(lo16(qe[e]), lo16(ke[e]), s);
                s = fmaf(hi16(qe[e]), hi16(ke[e]), s);
            }
        }
    }
    // rank: valid lanes ahead of this one by (score desc, position asc)
    const uint32_t key = order_key(s);
    int rank = 0;
    const uint64_t vm = __ballot(valid);
    for (int i = 0; i < k; ++i) {
        const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)key, i);
        const int pi = __builtin_amdgcn_readlane(p, i);
        const bool vi = (vm >> i) & 1ull;
        rank += (vi && (ki > key || (ki == key && pi < p))) ? 1 : 0;
    }
    const bool kept = valid && rank < keep;
    const uint64_t km = __ballot(kept);
    // softmax over the kept keys (log2 domain), then their V rows
    const float z = kept ? s * scale * 1.4426950408889634f : -INFINITY;
    float mx = z;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float pw = kept ? exp2f(z - mx) : 0.f;   // mx is finite when any key is kept
    float lsum = pw;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
    float acc[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] = 0.f;
    // the kept keys' V rows, eight at a time: their loads go out together
    constexpr int VB = 8;
    for (uint64_t m = km; m;) {
        int pi[VB];
        float wi[VB];
#pragma unroll
        for (int n = 0; n < VB; ++n) {
            const int i = m ? __builtin_ctzll(m) : 0;
            pi[n] = m ? __builtin_amdgcn_readlane(p, i) : -1;
            wi[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pw), i));
            m &= m - 1;
        }
        uint16_t vv[VB][DL];
#pragma unroll
        for (int n = 0; n < VB; ++n)
#pragma unroll
            for (int e = 0; e < DL; ++e) vv[n][e] = pi[n] >= 0 ? vb[(size_t)pi[n] * D + lane + 64 * e] : (uint16_t)0;
#pragma unroll
        for (int n = 0; n < VB; ++n)
#pragma unroll
            for (int e = 0; e < DL; ++e)
                if (pi[n] >= 0) acc[e] = fmaf(wi[n], __uint_as_float((uint32_t)vv[n][e] << 16), acc[e]);
    }
    // no kept key (every position outside the sequence): O = 0, LSE = -inf
    const float inv = km ? 1.f / lsum : 0.f;
    uint16_t* orow = out + ((size_t)g * L + t) * D;
#pragma unroll
    for (int e = 0; e < DL; ++e) orow[lane + 64 * e] = (uint16_t)(pack2(acc[e] * inv, 0.f) & 0xffffu);
    if (lane == 0) lse[(size_t)g * L + t] = km ? (mx + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
    if (kept_out) {
        // ascending kept positions, -1 past their count
        const int n_kept = __builtin_popcountll(km);
        int slot = 0;
        for (uint64_t m = km; m; m &= m - 1) slot += __builtin_amdgcn_readlane(p, __builtin_ctzll(m)) < p ? 1 : 0;
        int32_t* ko = kept_out + ((size_t)g * L + t) * keep;
        if (kept) ko[slot] = p;
        if (lane >= n_kept && lane < keep) ko[lane] = -1;
    }
}

}  // namespace

hipError_t launch_cand_positions(const void* x, const float* w, const float* bias, int B, int L, int C, int k,
                                 int32_t* pos, hipStream_t s) {
    if (k < 1 || k > kMaxCandidates || C < 1) return hipErrorInvalidValue;
    int kp = 1;
    while (kp < k) kp <<= 1;
    const int T = kPosThreads / kp;
    const int64_t grid = (int64_t)B * ((L + T - 1) / T);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(cand_positions_kernel, dim3((unsigned)grid), dim3(kPosThreads), 0, s, (const uint16_t*)x, w,
                       bias, L, C, k, kp, pos);
    return hipGetLastError();
}

hipError_t launch_cand_attention(const void* q, const void* k, const void* v, const int32_t* pos, int B, int H,
                                 int L, int D, int n_cand, int keep, float scale, void* out, float* lse,
                                 int32_t* kept, hipStream_t s, hipEvent_t before, hipEvent_t after) {
    if (n_cand < 1 || n_cand > kMaxCandidates || keep < 1 || keep > n_cand || (D != 64 && D != 128))
        return hipErrorInvalidValue;
    const int64_t nq = (int64_t)B * H * L;
    const int64_t grid = (nq + 3) / 4;
    if (grid == 0) return hipSuccess;
    // given events, the dispatch records the kernel's own start and stop
    if (D == 64)
        hipExtLaunchKernelGGL(cand_attention_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, before, after, 0,
                              (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pos, H, L, n_cand, keep,
                              scale, (uint16_t*)out, lse, kept, nq);
    else
        hipExtLaunchKernelGGL(cand_attention_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, before, after, 0,
                              (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pos, H, L, n_cand, keep,
                              scale, (uint16_t*)out, lse, kept, nq);
    return hipGetLastError();
}

}  // namespace bsattn
