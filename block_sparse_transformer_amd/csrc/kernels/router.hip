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
//
// One workgroup of 1024 threads per (b, h): scores into LDS, a bitonic sort
// by (score descending, row ascending) -- ties go to the lower row -- then a
// second bitonic sort of the k winners by row index so the output is
// ascending.  L <= 8192 keeps both arrays in LDS (96 KB).
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ double bf16_to_double(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

__global__ __launch_bounds__(kThreads) void route_topk_kernel(const uint16_t* q, const float* w, int L,
                                                              int D, int k, int NP, int KP, int32_t* out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    double* sc = (double*)sm;              // [NP]
    int* ix = (int*)(sc + NP);             // [NP]
    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;
    const uint16_t* qp = q + bh * (size_t)L * D;

    for (int t = tid; t < NP; t += kThreads) {
        double acc = -INFINITY;
        if (t < L) {
            acc = 0.0;
            const uint16_t* row = qp + (size_t)t * D;
            for (int d0 = 0; d0 < D; d0 += 8) {
                const uint4 u = *(const uint4*)(row + d0);
                const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = acc + bf16_to_double(wv[e] & 0xffffu) * (double)w[d0 + 2 * e];
                    acc = acc + bf16_to_double(wv[e] >> 16) * (double)w[d0 + 2 * e + 1];
                }
            }
        }
        sc[t] = acc;
        ix[t] = t;
    }
    __syncthreads();

    // Bitonic sort into "best first": x before y iff sx > sy or (sx == sy and ix < iy).
    // Padding entries (score -inf, index >= L) sort after every real row.
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < NP; i += kThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const double si = sc[i], sj = sc[j];
                    const int ii = ix[i], ij = ix[j];
                    const bool j_first = sj > si || (sj == si && ij < ii);
                    const bool forward = (i & size) == 0;
                    if (j_first == forward) {
                        sc[i] = sj; sc[j] = si;
                        ix[i] = ij; ix[j] = ii;
                    }
                }
            }
            __syncthreads();
        }
    }

    // The k winners, sorted ascending by row (reusing the score area as int storage).
    int* win = (int*)sc;   // [KP]
    for (int i = tid; i < KP; i += kThreads) win[i] = i < k ? ix[i] : 0x7fffffff;
    __syncthreads();
    for (int size = 2; size <= KP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < KP; i += kThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const int a = win[i], c = win[j];
                    const bool forward = (i & size) == 0;
                    if ((c < a) == forward) { win[i] = c; win[j] = a; }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < k; i += kThreads) out[bh * k + i] = win[i];
}

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

hipError_t launch_route_topk(const void* q, const float* w, int32_t B, int32_t H, int32_t L, int32_t D,
                             int32_t k, int32_t* out, hipStream_t s) {
    const int NP = next_pow2(L);
    const int KP = next_pow2(k);
    const size_t lds = (size_t)NP * (sizeof(double) + sizeof(int));
    hipError_t e = hipFuncSetAttribute((const void*)route_topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)((int64_t)B * H)), dim3(kThreads), lds, s,
                       (const uint16_t*)q, w, L, D, k, NP, KP, out);
    return hipGetLastError();
}

}  // namespace bsattn
