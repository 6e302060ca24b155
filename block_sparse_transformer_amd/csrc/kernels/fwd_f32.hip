// fwd_f32.hip -- block-sparse attention forward with fp32 inputs and fp32 arithmetic.
//
// Same definition as the bf16 path (Adaptive Sparse Transformer page, the
// SparseAttention formula, masked scores at -inf; one softmax over the union
// of the BigBird patterns) for fp32 tensors, where the result must stay
// within fp32 rounding of the exact value.  This path favours plainness over
// speed: one wave per 64-row query block, one lane per query row, K/V staged
// through LDS in 32-key halves and read as broadcasts, scores by sequential
// fp32 FMA, exact-rate expf.  Every row, global rows included, is walked by a
// single workgroup (no split, no merge).
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

template <int D, int MASK>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const FwdArgs a, const int32_t* row_ptr) {
    __shared__ float Ks[32][D];
    __shared__ float Vs[32][D];
    const int tid = threadIdx.x;
    const int rows = a.H * a.nb;
    const int row = blockIdx.x % rows;
    const int b = blockIdx.x / rows;
    const int h = row / a.nb;
    const int qblk = row % a.nb;
    const size_t bh = (size_t)b * a.H + h;
    const int tq = qblk * 64 + tid;
    const float* qp = (const float*)a.q + (bh * a.L + tq) * D;
    const float* kp = (const float*)a.k + bh * (size_t)a.L * D;
    const float* vp = (const float*)a.v + bh * (size_t)a.L * D;

    int valid = a.L;
    if (MASK == MASK_PAD) valid = min(max(a.valid_len[b], 0), a.L);

    float q[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; d += 4) {
        const float4 x = *(const float4*)(qp + d);
        q[d] = x.x; q[d + 1] = x.y; q[d + 2] = x.z; q[d + 3] = x.w;
        acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const int c0 = row_ptr[row], c1 = row_ptr[row + 1];
    for (int c = c0; c < c1; ++c) {
        const int j = a.col_idx[c];
        if (j * 64 >= valid) break;   // ascending row: the rest is padding
        for (int half = 0; half < 2; ++half) {
            const int key0 = j * 64 + half * 32;
            __syncthreads();
            for (int e = tid * 4; e < 32 * D; e += 64 * 4) {
                const int kk = e / D, d = e % D;
                *(float4*)&Ks[kk][d] = *(const float4*)(kp + (size_t)(key0 + kk) * D + d);
                *(float4*)&Vs[kk][d] = *(const float4*)(vp + (size_t)(key0 + kk) * D + d);
            }
            __syncthreads();
            float s[32];
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < 32; ++kk) {
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) dot = fmaf(q[d], Ks[kk][d], dot);
                s[kk] = (MASK == MASK_PAD && key0 + kk >= valid) ? -INFINITY : dot * a.scale;
                mx = fmaxf(mx, s[kk]);
            }
            const float mnew = fmaxf(m, mx);
            const float muse = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = expf(m - muse);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
            for (int kk = 0; kk < 32; ++kk) {
                const float p = expf(s[kk] - muse);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vs[kk][d], acc[d]);
            }
            m = mnew;
        }
    }
    float* orow = (float*)a.out + (bh * a.L + tq) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4)
        *(float4*)(orow + d) = make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
    a.lse[bh * a.L + tq] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D, int MASK>
hipError_t launch_t(const FwdArgs& a, const int32_t* row_ptr, hipStream_t s) {
    const int64_t grid = (int64_t)a.B * a.H * a.nb;
    hipLaunchKernelGGL((fwd_f32_kernel<D, MASK>), dim3((unsigned)grid), dim3(64), 0, s, a, row_ptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, const int32_t* row_ptr, int head_dim, int mask, hipStream_t s,
                          hipEvent_t before, hipEvent_t after) {
    hipError_t e;
    if (before && (e = hipEventRecord(before, s)) != hipSuccess) return e;
    if (head_dim == 64)
        e = mask == MASK_PAD ? launch_t<64, MASK_PAD>(a, row_ptr, s) : launch_t<64, MASK_NONE>(a, row_ptr, s);
    else
        e = mask == MASK_PAD ? launch_t<128, MASK_PAD>(a, row_ptr, s) : launch_t<128, MASK_NONE>(a, row_ptr, s);
    if (e != hipSuccess) return e;
    if (after && (e = hipEventRecord(after, s)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace bsattn
