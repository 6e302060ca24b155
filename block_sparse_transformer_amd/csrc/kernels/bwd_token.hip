// bwd_token.hip -- backward of the token-granular pattern: the pairs that the
// band and the global rows leave out.
//
// What is differentiated (BigBird page, its code example and the 核心实现
// section, token-granular: query t sees key s iff t or s is a global token,
// |t - s| <= w, or s is one of t's random tokens; the gradients are those of
// bwd_bf16.hip).  The band pairs and the global rows' pairs run through the
// MFMA passes of bwd_bf16.hip, the global rows as routed tiles shared by every
// (batch, head) group.  What remains, for every non-global row t, is a short
// list of extra keys: the global tokens outside t's band, and t's random
// tokens.  Those pairs are added here, to the bf16 gradients the MFMA passes
// wrote (one more rounding, 2^-9 relative):
//   * tok_dq_extra_kernel: dQ[t] += scale * sum_s dS[t,s] k_s over the extra
//     keys of each non-global row;
//   * tok_dkv_global_kernel, then tok_dkv_global_sum_kernel: for each global
//     key s, dK[s] += scale * sum_t dS[t,s] q_t and dV[s] += sum_t P[t,s] dO_t
//     over the non-global rows outside s's band, a few keys per workgroup
//     sharing the row loads, in row chunks whose fp32 partials the sum kernel
//     adds;
//   * tok_dkv_links_kernel: the same sums for each key s over the rows whose
//     random tokens hold s (the lists transposed on the host).
// P = exp(scale q.k - LSE) from the forward's LSE and dS = P (dO.v - delta),
// with delta = rowsum(dO * O) from the dQ pass.  Random tokens are never
// global, so the two dK/dV kernels write disjoint keys and every output
// element has one writer.
//
// Eight lanes per row (or key), D/8 columns each; the dot products are
// reduced over the eight lanes by shuffles.  These pairs are few (about
// n_global + r per row) and scattered: the kernels are gathers, bound by L2
// latency rather than by arithmetic, so their loads go out four keys (rows)
// at a time, and the global keys, the same for every row, are held on chip.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBatch = 4;   // keys (rows) whose slices are loaded together

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DP consecutive bf16 at element offset `off` of `base`, as fp32 (16-byte aligned).
template <int DP>
__device__ __forceinline__ void load_slice(const void* base, size_t off, float (&v)[DP]) {
    const u32x4_t* p = (const u32x4_t*)((const uint16_t*)base + off);
#pragma unroll
    for (int c = 0; c < DP / 8; ++c) {
        const u32x4_t w = p[c];
        const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * c + 2 * i] = lo16(e[i]);
            v[8 * c + 2 * i + 1] = hi16(e[i]);
        }
    }
}

// v[d] + add[d] * f, rounded back to bf16, at element offset `off` of `base`.
template <int DP>
__device__ __forceinline__ void add_slice(void* base, size_t off, const float (&add)[DP], float f) {
    u32x4_t* p = (u32x4_t*)((uint16_t*)base + off);
#pragma unroll
    for (int c = 0; c < DP / 8; ++c) {
        const u32x4_t w = p[c];
        const uint32_t e[4] = {w.x, w.y, w.z, w.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = pack2(fmaf(add[8 * c + 2 * i], f, lo16(e[i])), fmaf(add[8 * c + 2 * i + 1], f, hi16(e[i])));
        p[c] = u32x4_t{o[0], o[1], o[2], o[3]};
    }
}

// The value of another lane of the same row of 16, by a DPP lane move (no
// LDS round trip, unlike a shuffle through ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the eight lanes of a row (lanes 8k .. 8k + 7 of the wave, all
// active together): lane ^ 1 and lane ^ 2 within the quad, then the other
// quad's sum through the half-row mirror (lane i meets lane 7 - i).  Every
// lane ends with the same value (each step adds the same two numbers on both
// sides).
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_move<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_move<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_move<0x141>(x);   // row_half_mirror
    return x;
}

template <int DP>
__device__ __forceinline__ float dot(const float (&x)[DP], const float (&y)[DP]) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DP; ++d) s = fmaf(x[d], y[d], s);
    return s;
}

// Groups are dealt to XCDs as in the forward (workgroup i runs on XCD i % 8,
// and XCD x takes groups x, x + 8, ...), so a group's K and V, read by the
// gathers, stay in one XCD's L2.  Returns false past the last group.
__device__ __forceinline__ bool group_of(const BwdArgs& a, int per_group, int& g, int& rest) {
    const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    g = x + kXcds * (j / per_group);
    rest = j % per_group;
    return g < a.B * a.H;
}

// dQ of the extra keys of each non-global row: 32 rows per workgroup.  The
// global keys are the same for every row of the group: their K and V rows are
// staged in LDS, 64 keys at a time, and read from there.
template <int D>
__global__ __launch_bounds__(256) void tok_dq_extra_kernel(const BwdArgs a) {
    constexpr int DP = D / 8;
    __shared__ __attribute__((aligned(16))) uint16_t kvs[2][64][D];
    __shared__ int gs[64];
    const int tid = threadIdx.x, part = tid & 7;
    int g, rest;
    if (!group_of(a, a.L / 32, g, rest)) return;   // the whole workgroup
    const int t = rest * 32 + (tid >> 3);
    const size_t row = (size_t)g * a.L + t;
    const float lse = a.lse[row];
    // global rows come from the routed pass; rows with no key have nothing to add
    const bool live = a.tok_global[t] == 0 && lse != -INFINITY;
    const size_t gb = (size_t)g * a.L * D + part * DP;
    float qv[DP], dov[DP], acc[DP];
    load_slice<DP>(a.q, gb + (size_t)t * D, qv);
    load_slice<DP>(a.dout, gb + (size_t)t * D, dov);
    const float delta = a.delta[row];
    const float nl = -lse * kLog2e;
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = 0.f;
    bool used = false;
    // keys ids[0 .. kBatch) (-1: none); the same for the row's eight lanes
    auto visit = [&](const int (&ids)[kBatch]) {
        float kv[kBatch][DP], vv[kBatch][DP];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (ids[i] >= 0) {
                load_slice<DP>(a.k, gb + (size_t)ids[i] * D, kv[i]);
                load_slice<DP>(a.v, gb + (size_t)ids[i] * D, vv[i]);
            }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (ids[i] >= 0) {
                const float sc = group_sum(dot<DP>(qv, kv[i]));
                const float dp = group_sum(dot<DP>(dov, vv[i]));
                const float ds = exp2f(fmaf(sc, a.scale_log2, nl)) * (dp - delta);
#pragma unroll
                for (int d = 0; d < DP; ++d) acc[d] = fmaf(ds, kv[i][d], acc[d]);
                used = true;
            }
    };
    // the global keys outside the row's band, staged 64 at a time
    for (int c0 = 0; c0 < a.n_g; c0 += 64) {
        const int nc = min(64, a.n_g - c0);
        __syncthreads();   // the previous chunk's readers are done
        for (int e = tid; e < nc * (D / 8); e += 256) {
            const int key = e / (D / 8), piece = e % (D / 8);
            const int s = a.gtok[c0 + key];
            const size_t off = ((size_t)g * a.L + s) * D + 8 * piece;
            *(u32x4_t*)&kvs[0][key][8 * piece] = *(const u32x4_t*)((const uint16_t*)a.k + off);
            *(u32x4_t*)&kvs[1][key][8 * piece] = *(const u32x4_t*)((const uint16_t*)a.v + off);
            if (piece == 0) gs[key] = s;
        }
        __syncthreads();
        if (!live) continue;
        for (int key = 0; key < nc; ++key) {
            const int s = gs[key];
            if (abs(t - s) <= a.band) continue;   // inside the band: the band pass has it
            float kv[DP], vv[DP];
#pragma unroll
            for (int c = 0; c < DP / 8; ++c) {
                const u32x4_t wk = *(const u32x4_t*)&kvs[0][key][part * DP + 8 * c];
                const u32x4_t wv = *(const u32x4_t*)&kvs[1][key][part * DP + 8 * c];
                const uint32_t ek[4] = {wk.x, wk.y, wk.z, wk.w}, ev[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kv[8 * c + 2 * i] = lo16(ek[i]);
                    kv[8 * c + 2 * i + 1] = hi16(ek[i]);
                    vv[8 * c + 2 * i] = lo16(ev[i]);
                    vv[8 * c + 2 * i + 1] = hi16(ev[i]);
                }
            }
            const float sc = group_sum(dot<DP>(qv, kv));
            const float dp = group_sum(dot<DP>(dov, vv));
            const float ds = exp2f(fmaf(sc, a.scale_log2, nl)) * (dp - delta);
#pragma unroll
            for (int d = 0; d < DP; ++d) acc[d] = fmaf(ds, kv[d], acc[d]);
            used = true;
        }
    }
    if (!live) return;
    // the random tokens
    const int32_t* lk = a.links + ((size_t)(g % a.H) * a.L + t) * a.n_links;
    for (int j0 = 0; j0 < a.n_links; j0 += kBatch) {
        int ids[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) ids[i] = j0 + i < a.n_links ? lk[j0 + i] : -1;
        visit(ids);
    }
    if (used) add_slice<DP>(a.dq, gb + (size_t)t * D, acc, a.scale);
}

// dK, dV of the global keys from the non-global rows outside their band: one
// workgroup per (group, GK global keys, row chunk), 32 rows at a time; each
// row's q and dO slices are loaded once for its GK keys.  Writes the chunk's
// fp32 partials.
template <int D>
__global__ __launch_bounds__(256) void tok_dkv_global_kernel(const BwdArgs a) {
    constexpr int DP = D / 8, GK = tok_global_keys_per_wg(D);
    constexpr int RB = D == 64 ? kBatch : kBatch / 2;   // rows loaded together (registers)
    __shared__ float red[4][8][2 * DP];
    const int tid = threadIdx.x, part = tid & 7, slot = tid >> 3, lane = tid & 63, wave = tid >> 6;
    const int n_kc = (a.n_g + GK - 1) / GK;
    int g, rest;
    if (!group_of(a, n_kc * a.g_chunks, g, rest)) return;   // the whole workgroup
    const int kc = rest / a.g_chunks, ch = rest % a.g_chunks;
    const int rows_per = (a.L + a.g_chunks - 1) / a.g_chunks;
    const int r0 = ch * rows_per, r1 = min(a.L, r0 + rows_per);
    const size_t gb = (size_t)g * a.L * D + part * DP;
    int sk[GK];
    float kv[GK][DP], vv[GK][DP], ak[GK][DP], av[GK][DP];
#pragma unroll
    for (int e = 0; e < GK; ++e) {
        const int c = kc * GK + e;
        sk[e] = c < a.n_g ? a.gtok[c] : -1;
        const int s = sk[e] < 0 ? 0 : sk[e];
        load_slice<DP>(a.k, gb + (size_t)s * D, kv[e]);
        load_slice<DP>(a.v, gb + (size_t)s * D, vv[e]);
#pragma unroll
        for (int d = 0; d < DP; ++d) ak[e][d] = av[e][d] = 0.f;
    }
    for (int t0 = r0 + slot; t0 < r1; t0 += 32 * RB) {
        int ts[RB];
        float qv[RB][DP], dov[RB][DP], nl[RB], delta[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int t = t0 + 32 * i;
            ts[i] = (t < r1 && a.tok_global[t] == 0) ? t : -1;
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (ts[i] >= 0) {
                const size_t row = (size_t)g * a.L + ts[i];
                load_slice<DP>(a.q, gb + (size_t)ts[i] * D, qv[i]);
                load_slice<DP>(a.dout, gb + (size_t)ts[i] * D, dov[i]);
                const float lse = a.lse[row];
                nl[i] = lse == -INFINITY ? -INFINITY : -lse * kLog2e;   // -inf: the row has no key
                delta[i] = a.delta[row];
            }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (ts[i] >= 0 && nl[i] != -INFINITY) {
#pragma unroll
                for (int e = 0; e < GK; ++e) {
                    if (sk[e] < 0 || abs(ts[i] - sk[e]) <= a.band) continue;   // no key, or inside its band
                    const float sc = group_sum(dot<DP>(qv[i], kv[e]));
                    const float dp = group_sum(dot<DP>(dov[i], vv[e]));
                    const float p = exp2f(fmaf(sc, a.scale_log2, nl[i]));
                    const float ds = p * (dp - delta[i]);
#pragma unroll
                    for (int d = 0; d < DP; ++d) {
                        ak[e][d] = fmaf(ds, qv[i][d], ak[e][d]);
                        av[e][d] = fmaf(p, dov[i][d], av[e][d]);
                    }
                }
            }
    }
    // per key: the wave's eight row slots (lanes part + 8 i), then the four waves
#pragma unroll
    for (int e = 0; e < GK; ++e) {
#pragma unroll
        for (int d = 0; d < DP; ++d)
#pragma unroll
            for (int m = 8; m < 64; m <<= 1) {
                ak[e][d] += __shfl_xor(ak[e][d], m);
                av[e][d] += __shfl_xor(av[e][d], m);
            }
        if (lane < 8)
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                red[wave][lane][d] = ak[e][d];
                red[wave][lane][DP + d] = av[e][d];
            }
        __syncthreads();
        if (tid < 8 && sk[e] >= 0) {
            const int c = kc * GK + e;
            float* dst = a.ws_g + (((size_t)g * a.n_g + c) * a.g_chunks + ch) * 2 * D;
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                dst[tid * DP + d] = (red[0][tid][d] + red[1][tid][d]) + (red[2][tid][d] + red[3][tid][d]);
                dst[D + tid * DP + d] =
                    (red[0][tid][DP + d] + red[1][tid][DP + d]) + (red[2][tid][DP + d] + red[3][tid][DP + d]);
            }
        }
        __syncthreads();   // red is rewritten for the next key
    }
}

// The global keys' chunk partials, added into dK and dV: one workgroup per
// (group, global key), two columns per thread.
template <int D>
__global__ __launch_bounds__(64) void tok_dkv_global_sum_kernel(const BwdArgs a) {
    const int g = blockIdx.x / a.n_g, c = blockIdx.x % a.n_g;
    const int d = 2 * (int)threadIdx.x;
    if (d >= D) return;
    const int s = a.gtok[c];
    const float* src = a.ws_g + ((size_t)g * a.n_g + c) * a.g_chunks * 2 * D + d;
    float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
    for (int ch = 0; ch < a.g_chunks; ++ch) {
        k0 += src[(size_t)ch * 2 * D];
        k1 += src[(size_t)ch * 2 * D + 1];
        v0 += src[(size_t)ch * 2 * D + D];
        v1 += src[(size_t)ch * 2 * D + D + 1];
    }
    const size_t off = ((size_t)g * a.L + s) * D + d;
    uint32_t* pk = (uint32_t*)((uint16_t*)a.dk + off);
    uint32_t* pv = (uint32_t*)((uint16_t*)a.dv + off);
    const uint32_t wk = *pk, wv = *pv;
    *pk = pack2(fmaf(k0, a.scale, lo16(wk)), fmaf(k1, a.scale, hi16(wk)));
    *pv = pack2(lo16(wv) + v0, hi16(wv) + v1);
}

// dK, dV of each key from the rows whose random tokens hold it: 32 keys per
// workgroup; keys that no row links to are left alone.
template <int D>
__global__ __launch_bounds__(256) void tok_dkv_links_kernel(const BwdArgs a) {
    constexpr int DP = D / 8;
    const int tid = threadIdx.x, part = tid & 7;
    int g, rest;
    if (!group_of(a, a.L / 32, g, rest)) return;
    const int s = rest * 32 + (tid >> 3);
    const int32_t* tp = a.tptr + (size_t)(g % a.H) * (a.L + 1) + s;
    const int p0 = tp[0], p1 = tp[1];
    if (p0 == p1) return;
    const size_t gb = (size_t)g * a.L * D + part * DP;
    float kv[DP], vv[DP], ak[DP], av[DP];
    load_slice<DP>(a.k, gb + (size_t)s * D, kv);
    load_slice<DP>(a.v, gb + (size_t)s * D, vv);
#pragma unroll
    for (int d = 0; d < DP; ++d) ak[d] = av[d] = 0.f;
    for (int i0 = p0; i0 < p1; i0 += kBatch) {
        int ts[kBatch];
        float qv[kBatch][DP], dov[kBatch][DP], lse[kBatch], delta[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) ts[i] = i0 + i < p1 ? a.trows[i0 + i] : -1;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (ts[i] >= 0) {
                const size_t row = (size_t)g * a.L + ts[i];
                load_slice<DP>(a.q, gb + (size_t)ts[i] * D, qv[i]);
                load_slice<DP>(a.dout, gb + (size_t)ts[i] * D, dov[i]);
                lse[i] = a.lse[row];
                delta[i] = a.delta[row];
            }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (ts[i] >= 0 && lse[i] != -INFINITY) {
                const float sc = group_sum(dot<DP>(qv[i], kv));
                const float dp = group_sum(dot<DP>(dov[i], vv));
                const float p = exp2f(fmaf(sc, a.scale_log2, -lse[i] * kLog2e));
                const float ds = p * (dp - delta[i]);
#pragma unroll
                for (int d = 0; d < DP; ++d) {
                    ak[d] = fmaf(ds, qv[i][d], ak[d]);
                    av[d] = fmaf(p, dov[i][d], av[d]);
                }
            }
    }
    add_slice<DP>(a.dk, gb + (size_t)s * D, ak, a.scale);
    add_slice<DP>(a.dv, gb + (size_t)s * D, av, 1.f);
}

template <int D>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    const int64_t groups = (int64_t)a.B * a.H;
    const int64_t gpad = (groups + kXcds - 1) / kXcds * kXcds;   // whole rounds of XCDs
    if (a.n_g > 0 || a.n_links > 0) {
        hipLaunchKernelGGL(tok_dq_extra_kernel<D>, dim3((unsigned)(gpad * (a.L / 32))), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.n_g > 0) {
        constexpr int GK = tok_global_keys_per_wg(D);
        const int64_t n_kc = (a.n_g + GK - 1) / GK;
        hipLaunchKernelGGL(tok_dkv_global_kernel<D>, dim3((unsigned)(gpad * n_kc * a.g_chunks)), dim3(256), 0, s,
                           a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(tok_dkv_global_sum_kernel<D>, dim3((unsigned)(groups * a.n_g)), dim3(64), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.n_links > 0) {
        hipLaunchKernelGGL(tok_dkv_links_kernel<D>, dim3((unsigned)(gpad * (a.L / 32))), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_tok_bwd_extra(const BwdArgs& a, int head_dim, hipStream_t s) {
    if (a.L % 64 != 0 || (a.n_g > 0 && (!a.gtok || !a.ws_g || a.g_chunks < 1)) ||
        (a.n_links > 0 && (!a.links || !a.tptr || !a.trows)))
        return hipErrorInvalidValue;
    return head_dim == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace bsattn
