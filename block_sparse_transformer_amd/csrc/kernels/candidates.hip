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
// outside the sequence add nothing.  cand_positions4_kernel (k % 4 == 0,
// C % 8 == 0) runs the four chains of outputs 4g .. 4g + 3 of one token per
// thread, so that each x value is loaded and converted once for four fused
// multiply-adds; cand_positions_kernel runs one chain per thread otherwise.
//
// The importance evaluation keeps, per (batch, head, query), the `keep` best
// distinct candidates by the in-order fp32 score q.k of their keys (products
// added in order of d from +0, as the top-keep selection does), the lower
// position first on equal scores; the softmax of scale * score over the kept
// keys then weighs their V rows.  Two kernels compute it:
// * cand_attention2_kernel (k <= 32): two queries per wave, one candidate per
//   lane; the ranking is a bitonic sort within each half-wave (see there);
// * cand_attention_kernel (k up to 64): one wave per query.  Lane j < k holds
//   candidate position j; a position seen in a lower lane is dropped, and each
//   lane counts the lanes ahead of it.  Every lane owns D/64 output columns
//   and walks the kept keys, eight V rows per round of loads, so each row is
//   read once, coalesced.
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));


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

// Four outputs per thread (k % 4 == 0, C % 8 == 0, x and w 16-byte aligned): thread
// (token t, group g) runs the chains of outputs 4g .. 4g + 3, each in the same
// fixed order as above.  Per step of eight channels it loads the eight x
// values of the row once (16 bytes, one conversion each, shared by the four
// chains) and the four weights of each channel as one float4.
__global__ __launch_bounds__(kPosThreads) void cand_positions4_kernel(const uint16_t* __restrict__ x,
                                                                      const float* __restrict__ w,
                                                                      const float* __restrict__ bias, int L, int C,
                                                                      int k, int gp, int32_t* __restrict__ pos) {
    const int T = kPosThreads / gp;   // tokens per workgroup, gp lanes (output groups) per token
    const int tiles = (L + T - 1) / T;
    const int b = blockIdx.x / tiles;
    const int g = threadIdx.x % gp;
    const int t = (blockIdx.x % tiles) * T + threadIdx.x / gp;
    if (4 * g >= k || t >= L) return;
    const uint16_t* xb = x + (size_t)b * L * C;
    double acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = (double)bias[4 * g + i];
#pragma unroll 1
    for (int u = 0; u < 3; ++u) {
        const int row = t + u - 1;
        if (row < 0 || row >= L) continue;   // padding: the tap adds nothing
        const uint16_t* xr = xb + (size_t)row * C;
        const float* wu = w + (size_t)u * C * k + 4 * g;
#pragma unroll 2
        for (int c0 = 0; c0 < C; c0 += 8) {
            const u32x4_t xv = *(const u32x4_t*)(xr + c0);
            float4 wv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = *(const float4*)(wu + (size_t)(c0 + i) * k);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double xd = (double)((i & 1) ? hi16(xw[i >> 1]) : lo16(xw[i >> 1]));
                acc[0] = fma(xd, (double)wv[i].x, acc[0]);
                acc[1] = fma(xd, (double)wv[i].y, acc[1]);
                acc[2] = fma(xd, (double)wv[i].z, acc[2]);
                acc[3] = fma(xd, (double)wv[i].w, acc[3]);
            }
        }
    }
    int32_t* pr = pos + ((size_t)b * L + t) * k + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = acc[i];
        pr[i] = a != a ? 0 : (int)fmin(fmax(rint(a), 0.0), (double)(L - 1));
    }
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

// The value of lane (j ^ X) of the same half-wave (ds_swizzle, bit-mask mode:
// and-mask 31, or-mask 0, xor-mask X).
template <int X>
__device__ __forceinline__ uint32_t swz_xor(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (X << 10));
}

// One compare-exchange stage of a bitonic sort, descending, over the 32 lanes
// of each half-wave: lane j meets lane j ^ X, and of the pair the lane with
// bit B (the highest bit of X) clear keeps the larger value.  The comparison
// is one ballot; the lanes' side is a constant lane mask.
template <int X>
__device__ __forceinline__ uint64_t bitonic_cx(uint64_t v) {
    constexpr int B = X >= 16 ? 16 : X >= 8 ? 8 : X >= 4 ? 4 : X >= 2 ? 2 : 1;
    constexpr uint32_t low32 = B == 16 ? 0x0000ffffu : B == 8 ? 0x00ff00ffu : B == 4 ? 0x0f0f0f0fu
                             : B == 2 ? 0x33333333u : 0x55555555u;   // lanes j with bit B clear
    constexpr uint64_t low = ((uint64_t)low32 << 32) | low32;
    const uint32_t lo = swz_xor<X>((uint32_t)v), hi = swz_xor<X>((uint32_t)(v >> 32));
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    const uint64_t gt = __builtin_amdgcn_ballot_w64(v > o);
    return __builtin_amdgcn_inverse_ballot_w64(~(gt ^ low)) ? v : o;   // larger to the low side
}

// Sort of the 32 values of each half-wave, descending (lane 0 the largest):
// for each block size, a mirrored stage (j meets the lane at the same distance
// from the block's other end) and then the halving stages.
__device__ __forceinline__ uint64_t bitonic_sort32(uint64_t v) {
    v = bitonic_cx<1>(v);
    v = bitonic_cx<3>(v);
    v = bitonic_cx<1>(v);
    v = bitonic_cx<7>(v);
    v = bitonic_cx<2>(v);
    v = bitonic_cx<1>(v);
    v = bitonic_cx<15>(v);
    v = bitonic_cx<4>(v);
    v = bitonic_cx<2>(v);
    v = bitonic_cx<1>(v);
    v = bitonic_cx<31>(v);
    v = bitonic_cx<8>(v);
    v = bitonic_cx<4>(v);
    v = bitonic_cx<2>(v);
    return bitonic_cx<1>(v);
}

// Sum over the 32 lanes of each half-wave.
__device__ __forceinline__ float half_sum(float x) {
    x += __uint_as_float(swz_xor<16>(__float_as_uint(x)));
    x += __uint_as_float(swz_xor<8>(__float_as_uint(x)));
    x += __uint_as_float(swz_xor<4>(__float_as_uint(x)));
    x += __uint_as_float(swz_xor<2>(__float_as_uint(x)));
    x += __uint_as_float(swz_xor<1>(__float_as_uint(x)));
    return x;
}

// Two queries per wave, for k <= 32: half-wave hq = lane / 32 holds query
// 2 w + hq and its lane j = lane % 32 candidate j.  Each lane computes the
// in-order fp32 score of its candidate (the same products and order as the
// one-query kernel), then the half-wave sorts the pairs (order key of the
// score, position) descending -- score first, the lower position first on
// equal scores -- with a bitonic network of lane swaps.  Repeats of a
// position carry equal pairs, so they become neighbours and all but the first
// drop out; a lane's rank is the number of distinct candidates before it, and
// the first `keep` are kept.  The largest kept score is then in lane 0 of the
// half.  Each lane owns D / 32 output columns and walks the kept keys of its
// half, V rows read whole by the 32 lanes.
template <int D>
__global__ __launch_bounds__(256) void cand_attention2_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ kk,
                                                              const uint16_t* __restrict__ v,
                                                              const int32_t* __restrict__ pos, int H, int L, int k,
                                                              int keep, float scale, uint16_t* __restrict__ out,
                                                              float* __restrict__ lse, int32_t* __restrict__ kept_out,
                                                              int n_groups) {
    constexpr int DH = D / 32;   // output columns per lane
    const int lane = threadIdx.x & 63;
    const int hq = lane >> 5, j = lane & 31;
    // Workgroup i runs on XCD i % 8, and XCD x takes the groups x, x + 8, ...:
    // a group's K and V, which its queries gather, stay in one XCD's L2.
    const int tb_per_group = (L + 7) / 8;   // workgroups (eight queries each) per group
    const int xcd = blockIdx.x % kXcds, jw = blockIdx.x / kXcds;
    const int g = xcd + kXcds * (jw / tb_per_group);   // b * H + h
    if (g >= n_groups) return;
    const int t0 = (jw % tb_per_group) * 8 + (threadIdx.x >> 6) * 2;
    if (t0 >= L) return;             // the whole wave
    const int t = t0 + hq;
    const bool live = t < L;         // the second half of the last wave may be past the end
    const int b = g / H;
    const int64_t qi = (int64_t)g * L + (live ? t : t0);   // row of Q, O and LSE
    const int64_t prow = (int64_t)b * L + (live ? t : t0); // row of the positions
    const uint16_t* kb = kk + (size_t)g * L * D;
    const uint16_t* vb = v + (size_t)g * L * D;
    int p = (live && j < k) ? pos[(size_t)prow * k + j] : -1;
    if (p < 0 || p >= L) p = -1;
    // in-order fp32 score of this lane's key
    float s = 0.f;
    if (p >= 0) {
        const uint16_t* qr = q + (size_t)qi * D;
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
    // sort (order key, complement of the position) descending; no candidate:
    // key 0 and the largest position, below every candidate
    const uint32_t pk = p >= 0 ? (uint32_t)p : 0x7fffffffu;
    uint64_t sv = ((uint64_t)(p >= 0 ? order_key(s) : 0u) << 32) | (uint32_t)~pk;
    sv = bitonic_sort32(sv);
    const uint32_t key = (uint32_t)(sv >> 32);
    const int ps = (int)~(uint32_t)sv;           // position of this lane's pair after the sort
    const bool valid = ps != 0x7fffffff;
    const int prev = __shfl_up(ps, 1);           // the pair before (lane j - 1 of the half for j > 0)
    const bool distinct = valid && !(j > 0 && prev == ps);
    const uint32_t dm = (uint32_t)(__ballot(distinct) >> (32 * hq));
    const int rank = __builtin_popcount(dm & ((1u << j) - 1u));
    const bool kept = distinct && rank < keep;
    // the score back from its order key (exact, -0 aside; a NaN stays a NaN)
    const float ss = __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
    const float z = kept ? ss * scale * 1.4426950408889634f : -INFINITY;
    const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 0));
    const float m1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 32));
    const float m = hq ? m1 : m0;                // the largest kept score of the half (lane 0 of the half)
    const float pw = kept ? __builtin_amdgcn_exp2f(z - m) : 0.f;   // z - m <= 0
    const float lsum = half_sum(pw);
    // the kept V rows of both halves, four at a time
    const uint64_t km = __ballot(kept);
    uint32_t mlo = (uint32_t)km, mhi = (uint32_t)(km >> 32);
    float acc[DH];
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] = 0.f;
    constexpr int VB = 4;
    while (mlo | mhi) {
        int pi[VB];
        float wi[VB];
#pragma unroll
        for (int n = 0; n < VB; ++n) {
            const int il = mlo ? __builtin_ctz(mlo) : 0, ih = mhi ? 32 + __builtin_ctz(mhi) : 32;
            const int pl = mlo ? __builtin_amdgcn_readlane(ps, il) : -1;
            const int ph = mhi ? __builtin_amdgcn_readlane(ps, ih) : -1;
            const float wl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), il));
            const float wh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), ih));
            pi[n] = hq ? ph : pl;
            wi[n] = hq ? wh : wl;
            mlo &= mlo - 1u;
            mhi &= mhi - 1u;
        }
        uint32_t vv[VB][DH / 2 > 0 ? DH / 2 : 1];
#pragma unroll
        for (int n = 0; n < VB; ++n) {
            if (pi[n] >= 0) {
                const uint16_t* vr = vb + (size_t)pi[n] * D + DH * j;
                if constexpr (DH == 2) {
                    vv[n][0] = *(const uint32_t*)vr;
                } else {
                    const u32x2_t w2 = *(const u32x2_t*)vr;
                    vv[n][0] = w2.x;
                    vv[n][1] = w2.y;
                }
            } else {
#pragma unroll
                for (int e = 0; e < DH / 2; ++e) vv[n][e] = 0u;
            }
        }
#pragma unroll
        for (int n = 0; n < VB; ++n)
            if (pi[n] >= 0)
#pragma unroll
                for (int e = 0; e < DH / 2; ++e) {
                    acc[2 * e] = fmaf(wi[n], lo16(vv[n][e]), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(wi[n], hi16(vv[n][e]), acc[2 * e + 1]);
                }
    }
    if (!live) return;
    const bool any = ((km >> (32 * hq)) & 0xffffffffull) != 0;
    // no kept key (every position outside the sequence): O = 0, LSE = -inf
    const float inv = any ? 1.f / lsum : 0.f;
    uint16_t* orow = out + (size_t)qi * D + DH * j;
    if constexpr (DH == 2) {
        *(uint32_t*)orow = pack2(acc[0] * inv, acc[1] * inv);
    } else {
        u32x2_t w2;
        w2.x = pack2(acc[0] * inv, acc[1] * inv);
        w2.y = pack2(acc[2] * inv, acc[3] * inv);
        *(u32x2_t*)orow = w2;
    }
    if (j == 0) lse[qi] = any ? (m + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
    if (kept_out) {
        // ascending kept positions, -1 past their count
        const uint32_t hm = (uint32_t)(km >> (32 * hq));
        const int n_kept = __builtin_popcount(hm);
        int slot = 0;
        for (uint32_t mm = hm; mm; mm &= mm - 1u) slot += __shfl(ps, 32 * hq + __builtin_ctz(mm)) < ps ? 1 : 0;
        int32_t* ko = kept_out + (size_t)qi * keep;
        if (kept) ko[slot] = ps;
        if (j >= n_kept && j < keep) ko[j] = -1;
    }
}

}  // namespace

hipError_t launch_cand_positions(const void* x, const float* w, const float* bias, int B, int L, int C, int k,
                                 int32_t* pos, hipStream_t s) {
    if (k < 1 || k > kMaxCandidates || C < 1) return hipErrorInvalidValue;
    if (k % 4 == 0 && C % 8 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)w & 15) == 0) {
        int gp = 1;
        while (gp < k / 4) gp <<= 1;
        const int T = kPosThreads / gp;
        const int64_t grid = (int64_t)B * ((L + T - 1) / T);
        if (grid == 0) return hipSuccess;
        hipLaunchKernelGGL(cand_positions4_kernel, dim3((unsigned)grid), dim3(kPosThreads), 0, s, (const uint16_t*)x,
                           w, bias, L, C, k, gp, pos);
        return hipGetLastError();
    }
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
    const int64_t groups = (int64_t)B * H;
    const int64_t grid2 = (int64_t)kXcds * ((groups + kXcds - 1) / kXcds) * ((L + 7) / 8);   // two queries per wave
    if (n_cand <= 32 && grid2 < ((int64_t)1 << 31)) {
        if (D == 64)
            hipExtLaunchKernelGGL(cand_attention2_kernel<64>, dim3((unsigned)grid2), dim3(256), 0, s, before, after, 0,
                                  (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pos, H, L, n_cand, keep,
                                  scale, (uint16_t*)out, lse, kept, (int)groups);
        else
            hipExtLaunchKernelGGL(cand_attention2_kernel<128>, dim3((unsigned)grid2), dim3(256), 0, s, before, after,
                                  0, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pos, H, L, n_cand,
                                  keep, scale, (uint16_t*)out, lse, kept, (int)groups);
        return hipGetLastError();
    }
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
