// layer.hip -- the element-wise steps of the attention layer around the
// block-sparse attention (primer page, "BERT稀疏注意力机制入门指南：原理、实现与性能优化",
// section PyTorch 实现基础稀疏注意力, the SparseAttention module): the qkv
// projection's bias and the split of its width-3C rows into per-head Q, K, V
// (read as (3, H, D)), the concatenation of the heads' outputs back to rows of
// width C, and the output projection's bias.  The two projections themselves
// are plain GEMMs done by rocBLAS.  All three kernels are HBM-bound copies;
// each thread moves 8 consecutive features (16 bytes of bf16) so that every
// access is a full 16-byte vector.
#include <hip/hip_runtime.h>

#include "../internal.h"

namespace bsattn {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 fp32 + 8 bf16 bias -> 8 bf16, one rounding.
__device__ __forceinline__ u32x4_t add_bias8(const float* src, const uint16_t* bias) {
    const float4 a = *(const float4*)src;
    const float4 b = *(const float4*)(src + 4);
    const u32x4_t bb = *(const u32x4_t*)bias;
    u32x4_t r;
    r.x = pack_bf16x2(a.x + bf16_lo(bb.x), a.y + bf16_hi(bb.x));
    r.y = pack_bf16x2(a.z + bf16_lo(bb.y), a.w + bf16_hi(bb.y));
    r.z = pack_bf16x2(b.x + bf16_lo(bb.z), b.y + bf16_hi(bb.z));
    r.w = pack_bf16x2(b.z + bf16_lo(bb.w), b.w + bf16_hi(bb.w));
    return r;
}

// qkv32 [B*L, 3C] fp32 + b_qkv -> q, k, v [B, H, L, D] bf16.  Thread = 8 features.
__global__ __launch_bounds__(256) void split_heads_kernel(const float* qkv32, const uint16_t* b_qkv,
                                                          uint16_t* q, uint16_t* k, uint16_t* v,
                                                          int B, int L, int H, int D) {
    const int C = H * D;
    const size_t n8 = (size_t)B * L * 3 * C / 8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const size_t row = i / (3 * C / 8);             // b * L + t
    const int col = (int)(i % (3 * C / 8)) * 8;     // in [0, 3C)
    const int s = col / C, h = (col % C) / D, d = col % D;
    const size_t b = row / L, t = row % L;
    uint16_t* dst = s == 0 ? q : (s == 1 ? k : v);
    *(u32x4_t*)(dst + ((b * H + h) * L + t) * D + d) = add_bias8(qkv32 + row * 3 * C + col, b_qkv + col);
}

// O [B, H, L, D] bf16 -> o2 [B*L, C] bf16 (heads concatenated in order).
__global__ __launch_bounds__(256) void merge_heads_kernel(const uint16_t* o, uint16_t* o2, int B, int L, int H,
                                                          int D) {
    const int C = H * D;
    const size_t n8 = (size_t)B * L * C / 8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const size_t row = i / (C / 8);
    const int col = (int)(i % (C / 8)) * 8;
    const int h = col / D, d = col % D;
    const size_t b = row / L, t = row % L;
    *(u32x4_t*)(o2 + row * C + col) = *(const u32x4_t*)(o + ((b * H + h) * L + t) * D + d);
}

// out32 [B*L, C] fp32 + b_proj -> out [B*L, C] bf16.
__global__ __launch_bounds__(256) void bias_out_kernel(const float* out32, const uint16_t* b_proj, uint16_t* out,
                                                       size_t rows, int C) {
    const size_t n8 = rows * C / 8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const int col = (int)(i % (C / 8)) * 8;
    *(u32x4_t*)(out + i * 8) = add_bias8(out32 + i * 8, b_proj + col);
}

unsigned blocks_for(size_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_split_heads(const float* qkv32, const void* b_qkv, void* q, void* k, void* v, int B, int L,
                              int H, int D, hipStream_t s) {
    const size_t n8 = (size_t)B * L * 3 * H * D / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(split_heads_kernel, dim3(blocks_for(n8)), dim3(256), 0, s, qkv32, (const uint16_t*)b_qkv,
                       (uint16_t*)q, (uint16_t*)k, (uint16_t*)v, B, L, H, D);
    return hipGetLastError();
}

hipError_t launch_merge_heads(const void* o, void* o2, int B, int L, int H, int D, hipStream_t s) {
    const size_t n8 = (size_t)B * L * H * D / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_heads_kernel, dim3(blocks_for(n8)), dim3(256), 0, s, (const uint16_t*)o,
                       (uint16_t*)o2, B, L, H, D);
    return hipGetLastError();
}

hipError_t launch_bias_out(const float* out32, const void* b_proj, void* out, size_t rows, int C, hipStream_t s) {
    const size_t n8 = rows * C / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(bias_out_kernel, dim3(blocks_for(n8)), dim3(256), 0, s, out32, (const uint16_t*)b_proj,
                       (uint16_t*)out, rows, C);
    return hipGetLastError();
}

}  // namespace bsattn
