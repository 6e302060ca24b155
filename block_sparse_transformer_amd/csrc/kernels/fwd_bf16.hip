// fwd_bf16.hip -- block-sparse attention forward, bf16 in/out, bf16 MFMA with fp32 accumulation.
//
// What is computed (Adaptive Sparse Transformer page, the SparseAttention
// formula; masked scores are -inf): for every query row, softmax over the
// allowed keys of scale * q.k, times V.  Attention runs only on the non-zero
// 64x64 blocks of the block-CSR layout (SQA page, "Transformer计算效率优化：SQA稀疏
// 注意力机制详解", section 3.1: FlashAttention-style computation restricted to
// non-zero blocks; section 5: 64x64 blocks held in on-chip memory).
//
// Design for gfx950 (CDNA4, wave64, 160 KB LDS per CU):
//  * One workgroup = 2 waves = one 64-row query tile; wave w owns rows
//    32w..32w+31.  The tile walks its CSR row of key blocks.
//  * K and V tiles are double-buffered in LDS: the global loads of tile t+1
//    are issued into registers before tile t is computed, and written to the
//    other LDS buffer afterwards; one barrier per tile.  K is stored
//    row-major (padded rows, conflict-free 16-byte reads); V is stored
//    transposed (Vt[d][key]) so that the PV contraction over keys reads
//    contiguous keys.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the 32x32 accumulator gives each lane 16
//    keys of ONE query, so the row max/sum are in-lane reductions plus a
//    single exchange between the two half-waves.  The same registers,
//    rounded to bf16, are directly the B operand of O^T = V^T P^T (the order
//    of the contraction index is free as long as A and B agree).
//  * Online softmax in the log2 domain: p = exp2(s*scale*log2e - m) with a
//    single FMA feeding v_exp_f32; running max m and per-half partial sums.
//  * Rows longer than 16 blocks (global rows, routed tiles) are split into
//    chunks; each chunk writes a normalised fp32 partial and its LSE, and
//    merge_kernel combines them by log-sum-exp.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // native vector: stays in registers
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8_t pack_bf16x8(const f32x16_t& s, int base) {
    u32x4_t u;
    u.x = pack_bf16x2(s[base + 0], s[base + 1]);
    u.y = pack_bf16x2(s[base + 2], s[base + 3]);
    u.z = pack_bf16x2(s[base + 4], s[base + 5]);
    u.w = pack_bf16x2(s[base + 6], s[base + 7]);
    return as_bf16x8(u);
}


// Layout constants shared by the kernel and its tile helpers.
template <int D>
struct Tile {
    static constexpr int KS = D + 8;     // LDS K row stride (bf16 elements): conflict-free 16-byte reads
    static constexpr int VS = 64 + 4;    // LDS Vt row stride (bf16 elements): conflict-free 8-byte reads
    static constexpr int KT = 64 * KS;   // K tile (elements)
    static constexpr int VT = D * VS;    // Vt tile (elements)
    static constexpr int KLD = D / 16;   // 16-byte K pieces per thread per tile (128 threads)
    static constexpr int VLD = D / 64;   // (4 keys x 8 d) V units per thread per tile
};

// Issue the global loads of key block j into registers.  K: 16-byte pieces,
// consecutive threads on consecutive pieces of a row.  V: thread owns 4
// consecutive keys x 8 consecutive d, ready for the transposed LDS store.
template <int D>
__device__ __forceinline__ void tile_gload(const uint16_t* kp, const uint16_t* vp, int j, int tid,
                                           u32x4_t (&kr)[Tile<D>::KLD], u32x4_t (&vr)[Tile<D>::VLD][4]) {
    const uint16_t* kt = kp + (size_t)j * 64 * D;
#pragma unroll
    for (int r = 0; r < Tile<D>::KLD; ++r) {
        const int id = tid + 128 * r;
        const int row = id / (D / 8), cc = id % (D / 8);
        kr[r] = *(const u32x4_t*)(kt + row * D + cc * 8);
    }
    const uint16_t* vt = vp + (size_t)j * 64 * D;
#pragma unroll
    for (int u = 0; u < Tile<D>::VLD; ++u) {
        const int uid = tid + 128 * u;
        const int kg = uid % 16, dc = uid / 16;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) vr[u][rr] = *(const u32x4_t*)(vt + (4 * kg + rr) * D + 8 * dc);
    }
}

// Write the staged tile to one LDS buffer: K row-major, V transposed (Vt[d][key]).
template <int D>
__device__ __forceinline__ void tile_lstore(uint16_t* Ks, int tid, const u32x4_t (&kr)[Tile<D>::KLD],
                                            const u32x4_t (&vr)[Tile<D>::VLD][4]) {
    uint16_t* Vt = Ks + Tile<D>::KT;
#pragma unroll
    for (int r = 0; r < Tile<D>::KLD; ++r) {
        const int id = tid + 128 * r;
        const int row = id / (D / 8), cc = id % (D / 8);
        *(u32x4_t*)(Ks + row * Tile<D>::KS + cc * 8) = kr[r];
    }
#pragma unroll
    for (int u = 0; u < Tile<D>::VLD; ++u) {
        const int uid = tid + 128 * u;
        const int kg = uid % 16, dc = uid / 16;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            // dword m4 of key row rr holds d = 8dc+2m4 (low half) and 8dc+2m4+1 (high half)
            const uint32_t w0 = vr[u][0][m4], w1 = vr[u][1][m4];
            const uint32_t w2 = vr[u][2][m4], w3 = vr[u][3][m4];
            u32x2_t lo, hi;
            lo.x = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
            lo.y = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            hi.x = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            hi.y = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            *(u32x2_t*)(Vt + (8 * dc + 2 * m4) * Tile<D>::VS + 4 * kg) = lo;
            *(u32x2_t*)(Vt + (8 * dc + 2 * m4 + 1) * Tile<D>::VS + 4 * kg) = hi;
        }
    }
}

template <int D, int MASK>
__global__ __launch_bounds__(128) void fwd_bf16_kernel(const FwdArgs a) {
    constexpr int KS = Tile<D>::KS, VS = Tile<D>::VS, KT = Tile<D>::KT, VT = Tile<D>::VT;
    constexpr int KLD = Tile<D>::KLD, VLD = Tile<D>::VLD;
    constexpr int NC = D / 16;       // 16-wide contraction chunks of Q K^T
    constexpr int NDB = D / 32;      // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int rloc = wave * 32 + ql;

    // ---- decode the work unit: routed tiles first, then the explicit items ----
    int b, h, qblk = 0, cb, ce, slot, rt = 0;
    bool routed;
    const int n_routed_units = a.n_routed > 0 ? a.B * a.H * a.n_rt * a.r_chunks : 0;
    if ((int)blockIdx.x < n_routed_units) {
        int r = blockIdx.x;
        const int c = r % a.r_chunks;
        r /= a.r_chunks;
        rt = r % a.n_rt;
        r /= a.n_rt;
        h = r % a.H;
        b = r / a.H;
        cb = c * a.r_chunk_tiles;
        ce = min(a.nb, cb + a.r_chunk_tiles);
        slot = a.r_slot_base + ((b * a.H + h) * a.n_rt + rt) * a.r_chunks + c;
        routed = true;
    } else {
        const int u = blockIdx.x - n_routed_units;
        const WorkItem it = a.items[u / a.B];
        b = u % a.B;
        h = it.row / a.nb;
        qblk = it.row % a.nb;
        cb = it.col_begin;
        ce = it.col_end;
        slot = it.slot < 0 ? -1 : b * a.n_slots + it.slot;
        routed = false;
    }
    const size_t bh = (size_t)b * a.H + h;

    int tq;   // query token of this lane's row (-1: unused row of a ragged routed tile)
    if (!routed) {
        tq = qblk * 64 + rloc;
    } else {
        const int kk = rt * 64 + rloc;
        tq = kk < a.n_routed ? a.routed_rows[bh * a.n_routed + kk] : -1;
        if (tq >= a.L) tq = -1;   // out-of-range routed rows are skipped, never dereferenced
    }

    int valid = a.L;
    if (MASK == MASK_PAD) {
        valid = min(max(a.valid_len[b], 0), a.L);
        // rows are ascending: drop the trailing blocks that start at or past the valid length
        while (ce > cb && a.col_idx[ce - 1] * 64 >= valid) --ce;
    }

    const uint16_t* qp = (const uint16_t*)a.q + bh * (size_t)a.L * D;
    const uint16_t* kp = (const uint16_t*)a.k + bh * (size_t)a.L * D;
    const uint16_t* vp = (const uint16_t*)a.v + bh * (size_t)a.L * D;

    // Q^T fragments, the B operand of S^T = K Q^T: lane (ql, hh) holds Q[row][16c + 8hh .. +7].
    bf16x8_t qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        u32x4_t u = {0u, 0u, 0u, 0u};
        if (tq >= 0) u = *(const u32x4_t*)(qp + (size_t)tq * D + 16 * c + 8 * hh);
        qf[c] = as_bf16x8(u);
    }

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m = -INFINITY;   // running max of scaled scores (log2 units)
    float l = 0.f;         // running partial sum over this half-wave's keys

    u32x4_t kr[KLD];
    u32x4_t vr[VLD][4];
    const int n = ce - cb;
    if (n > 0) {
        tile_gload<D>(kp, vp, routed ? cb : a.col_idx[cb], tid, kr, vr);
        tile_lstore<D>(smem, tid, kr, vr);
    }
    __syncthreads();

    for (int t = 0; t < n; ++t) {
        const int j = routed ? cb + t : a.col_idx[cb + t];
        if (t + 1 < n) tile_gload<D>(kp, vp, routed ? cb + t + 1 : a.col_idx[cb + t + 1], tid, kr, vr);
        const uint16_t* Ks = smem + (t & 1) * (KT + VT);
        const uint16_t* Vt = Ks + KT;

        // S^T (keys x queries): s0 keys 0..31, s1 keys 32..63 of the tile.
        f32x16_t s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bf16x8_t k0 = as_bf16x8(*(const u32x4_t*)(Ks + ql * KS + 16 * c + 8 * hh));
            const bf16x8_t k1 = as_bf16x8(*(const u32x4_t*)(Ks + (32 + ql) * KS + 16 * c + 8 * hh));
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[c], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[c], s1, 0, 0, 0);
        }
        // accumulator register i holds key 8*(i/4) + 4*hh + (i%4) (+32 for s1)
        if (MASK == MASK_PAD) {
            if (j * 64 + 64 > valid) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * 64 + 8 * (i / 4) + 4 * hh + (i % 4);
                    if (key >= valid) s0[i] = -INFINITY;
                    if (key + 32 >= valid) s1[i] = -INFINITY;
                }
            }
        }
        if (MASK == MASK_BAND) {
            if (!routed) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * 64 + 8 * (i / 4) + 4 * hh + (i % 4);
                    if (abs(tq - key) > a.band) s0[i] = -INFINITY;
                    if (abs(tq - key - 32) > a.band) s1[i] = -INFINITY;
                }
            }
        }

        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx * a.scale_log2);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - muse);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], a.scale_log2, -muse));
            s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], a.scale_log2, -muse));
            ps += s0[i] + s1[i];
        }
        l = l * alpha + ps;
        m = mnew;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

        // P^T fragments: MFMA c2 covers keys 16c2..16c2+15; element e of lane half hh is
        // key 16c2 + 8(e/4) + 4hh + e%4.
        bf16x8_t pf[4];
        pf[0] = pack_bf16x8(s0, 0);
        pf[1] = pack_bf16x8(s0, 8);
        pf[2] = pack_bf16x8(s1, 0);
        pf[3] = pack_bf16x8(s1, 8);
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const uint16_t* vrow = Vt + (32 * db + ql) * VS + 16 * c2 + 4 * hh;
                const u32x2_t lo = *(const u32x2_t*)vrow;
                const u32x2_t hi = *(const u32x2_t*)(vrow + 8);
                const u32x4_t lh = {lo.x, lo.y, hi.x, hi.y};
                const bf16x8_t va = as_bf16x8(lh);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[c2], o[db], 0, 0, 0);
            }
        }
        if (t + 1 < n) tile_lstore<D>(smem + ((t + 1) & 1) * (KT + VT), tid, kr, vr);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    if (tq < 0) return;
    if (slot < 0) {
        uint16_t* orow = (uint16_t*)a.out + (bh * a.L + tq) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                u32x2_t w;
                w.x = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
                w.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                *(u32x2_t*)(orow + d0) = w;
            }
        if (hh == 0) a.lse[bh * a.L + tq] = lse_v;
    } else {
        float* orow = a.ws_o + ((size_t)slot * 64 + rloc) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hh;
                *(float4*)(orow + d0) = make_float4(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv,
                                                    o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
            }
        if (hh == 0) a.ws_lse[(size_t)slot * 64 + rloc] = lse_v;
    }
}

// Combine the chunk partials of split rows: LSE = logsumexp_c LSE_c,
// O = sum_c exp(LSE_c - LSE) O_c.  A chunk with no allowed key has LSE_c = -inf
// and weight 0; a row with none at all gets O = 0, LSE = -inf.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const FwdArgs a) {
    constexpr int DP = D / 4;   // d values per thread
    const int row = threadIdx.x >> 2;
    const int part = threadIdx.x & 3;
    int b, h, first, nch, tq;
    const int n_routed_units = a.n_routed > 0 ? a.B * a.H * a.n_rt : 0;
    if ((int)blockIdx.x < n_routed_units) {
        int r = blockIdx.x;
        const int rt = r % a.n_rt;
        r /= a.n_rt;
        h = r % a.H;
        b = r / a.H;
        first = a.r_slot_base + ((b * a.H + h) * a.n_rt + rt) * a.r_chunks;
        nch = a.r_chunks;
        const int kk = rt * 64 + row;
        tq = kk < a.n_routed ? a.routed_rows[((size_t)b * a.H + h) * a.n_routed + kk] : -1;
        if (tq >= a.L) tq = -1;
    } else {
        const int u = blockIdx.x - n_routed_units;
        const MergeItem mi = a.merges[u / a.B];
        b = u % a.B;
        h = mi.row / a.nb;
        first = b * a.n_slots + mi.first_slot;
        nch = mi.n_chunks;
        tq = (mi.row % a.nb) * 64 + row;
    }
    if (tq < 0) return;
    const size_t bh = (size_t)b * a.H + h;
    float mx = -INFINITY;
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, a.ws_lse[(size_t)(first + c) * 64 + row]);
    uint16_t* orow = (uint16_t*)a.out + (bh * a.L + tq) * D + part * DP;
    if (mx == -INFINITY) {
#pragma unroll
        for (int d = 0; d < DP; d += 2) *(uint32_t*)(orow + d) = 0u;
        if (part == 0) a.lse[bh * a.L + tq] = -INFINITY;
        return;
    }
    float acc[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = 0.f;
    float wsum = 0.f;
    for (int c = 0; c < nch; ++c) {
        const float w = expf(a.ws_lse[(size_t)(first + c) * 64 + row] - mx);
        wsum += w;
        const float* src = a.ws_o + ((size_t)(first + c) * 64 + row) * D + part * DP;
#pragma unroll
        for (int d = 0; d < DP; d += 4) {
            const float4 x = *(const float4*)(src + d);
            acc[d + 0] += w * x.x;
            acc[d + 1] += w * x.y;
            acc[d + 2] += w * x.z;
            acc[d + 3] += w * x.w;
        }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int d = 0; d < DP; d += 2) *(uint32_t*)(orow + d) = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
    if (part == 0) a.lse[bh * a.L + tq] = mx + logf(wsum);
}

template <int D, int MASK>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
    const int64_t n_routed_units = a.n_routed > 0 ? (int64_t)a.B * a.H * a.n_rt * a.r_chunks : 0;
    const int64_t grid = (int64_t)a.n_items * a.B + n_routed_units;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK>), dim3((unsigned)grid), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before,
                           hipEvent_t after) {
    hipError_t e;
    if (before && (e = hipEventRecord(before, s)) != hipSuccess) return e;
    if (head_dim == 64) {
        e = mask == MASK_PAD ? launch_fwd_t<64, MASK_PAD>(a, s)
          : mask == MASK_BAND ? launch_fwd_t<64, MASK_BAND>(a, s)
                              : launch_fwd_t<64, MASK_NONE>(a, s);
    } else {
        e = mask == MASK_PAD ? launch_fwd_t<128, MASK_PAD>(a, s)
          : mask == MASK_BAND ? launch_fwd_t<128, MASK_BAND>(a, s)
                              : launch_fwd_t<128, MASK_NONE>(a, s);
    }
    if (e != hipSuccess) return e;
    if (after && (e = hipEventRecord(after, s)) != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_merge_bf16(const FwdArgs& a, int head_dim, hipStream_t s) {
    const int64_t n_routed_units = a.n_routed > 0 ? (int64_t)a.B * a.H * a.n_rt : 0;
    const int64_t grid = (int64_t)a.n_merges * a.B + n_routed_units;
    if (grid == 0) return hipSuccess;
    if (head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((merge_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bsattn
