// layout_build.hip -- the block layout rule evaluated on the device.
//
// One thread per (head, query block) row runs the same integer rule as the
// host builder (layout_rule.h: BigBird page, section 核心实现), so the device
// CSR can be compared with the host CSR bit for bit.  Counts go to
// row_ptr[1..], a single-workgroup scan turns them into offsets, and a third
// pass fills col_idx.
#include <hip/hip_runtime.h>

#include "../internal.h"

namespace bsattn {
namespace {

constexpr int kScanThreads = 1024;

// kind 0: rule rows on 64-token blocks; 1: token band; 2: rule on 32-token
// blocks (two rule rows per tile row); 3: rule on 128-token blocks (each rule
// row and column spans two tiles)
__global__ void count_kernel(const RowRule rule, int kind, int H, int nb, int band, int32_t* row_ptr) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= H * nb) return;
    const int h = r / nb, i = r % nb;
    int n;
    if (kind == 0) n = rule_row_count(rule, h, i);
    else if (kind == 1) n = band_row_fill(nb, kBlock, band, i, nullptr);
    else if (kind == 2) n = sub_tile_row(rule, h, i, nullptr, nullptr);
    else n = wide_tile_row_fill(rule, h, i, nullptr);
    row_ptr[r + 1] = n;
    if (r == 0) row_ptr[0] = 0;
}

// In-place inclusive scan of row_ptr[1..n] by one workgroup.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* row_ptr, int n) {
    __shared__ int32_t part[kScanThreads];
    const int tid = threadIdx.x;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int s = 1 + tid * per;
    const int e = min(n + 1, s + per);
    int32_t sum = 0;
    for (int x = s; x < e; ++x) sum += row_ptr[x];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = tid > 0 ? part[tid - 1] : 0;
    for (int x = s; x < e; ++x) {
        run += row_ptr[x];
        row_ptr[x] = run;
    }
}

__global__ void fill_kernel(const RowRule rule, int kind, int H, int nb, int band, const int32_t* row_ptr,
                            int32_t* col_idx, uint8_t* subs) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= H * nb) return;
    const int h = r / nb, i = r % nb;
    int32_t* out = col_idx + row_ptr[r];
    if (kind == 0) {
        rule_row_fill(rule, h, i, out);
    } else if (kind == 1) {
        band_row_fill(nb, kBlock, band, i, out);
    } else if (kind == 2) {
        sub_tile_row(rule, h, i, out, subs + row_ptr[r]);
    } else {
        wide_tile_row_fill(rule, h, i, out);
    }
}

}  // namespace

hipError_t launch_layout_build(const RowRule& rule, int kind, int32_t H, int32_t nb, int32_t band,
                               int32_t* row_ptr, int32_t* col_idx, uint8_t* subs, hipStream_t s) {
    const int rows = H * nb;
    const int threads = 128;
    const int grid = (rows + threads - 1) / threads;
    hipLaunchKernelGGL(count_kernel, dim3(grid), dim3(threads), 0, s, rule, kind, H, nb, band, row_ptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, row_ptr, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(threads), 0, s, rule, kind, H, nb, band, row_ptr, col_idx,
                       subs);
    return hipGetLastError();
}

}  // namespace bsattn
