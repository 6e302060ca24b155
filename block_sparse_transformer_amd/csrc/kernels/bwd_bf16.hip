// bwd_bf16.hip -- block-sparse attention backward, bf16 in/out, bf16 MFMA with fp32 accumulation.
//
// What is computed: the gradients of the forward in fwd_bf16.hip (the
// SparseAttention formula of the Adaptive Sparse Transformer page, "Adapt or
// Perish: 新手入门指南 – Adaptive Sparse Transformer 核心原理与实战", with
// masked scores at -inf) with respect to Q, K and V for an upstream dO.  The
// pages train these models (SQA page, "Transformer计算效率优化：SQA稀疏注意力机制详解",
// sections 2.2 and 3.2) but print no backward; it is the derivative of the
// forward.  With P = exp(scale * q.k - LSE) on the allowed entries of a
// non-zero 64x64 block (0 elsewhere):
//
//     delta = rowsum(dO * O)
//     dV    = P^T dO                 dP = dO V^T
//     dS    = P * (dP - delta)
//     dQ    = scale * dS K           dK = scale * dS^T Q
//
// P is recomputed from the saved LSE; nothing of size L x L is stored.
//
// Design for gfx950:
//  * Two passes, each with one workgroup (2 waves) per row or column of the
//    block layout, so that every output is accumulated in registers and
//    written once, with no atomics: the dQ pass walks the key blocks of a
//    query block's row; the dK/dV pass walks the query blocks whose rows hold
//    a key block (the layout transposed on the host).  Rows and columns
//    longer than 16 blocks (global rows and columns) are split into chunks;
//    each chunk writes an fp32 partial and a small launch adds them up.
//  * delta = rowsum(dO * O) is formed in the dQ pass, from the dO half-rows
//    its lanes already load, and stored for the dK/dV pass that follows.
//  * All products are v_mfma_f32_32x32x16_bf16 with the output transposed so
//    that a lane owns one row of the pass's own block (a query in the dQ pass,
//    a key in the dK/dV pass) and holds 16 entries of the other side in its
//    registers.  Those registers, rounded to bf16, are directly the B operand
//    of the next product (the order of a contraction index is free as long as
//    both operands agree), and the A operand of that product is the staged
//    tile read transposed by ds_read_b64_tr_b16.  Tiles sit row-major in LDS
//    with 16-byte pieces XOR-swizzled by the row, read both row-wise
//    (ds_read_b128) and transposed.
//  * In the dK/dV pass each lane's 16 registers belong to 16 different
//    queries, each with its own LSE and delta.  They enter as the initial
//    accumulator of the score and dP products (-LSE/scale and -delta per
//    row), so no per-register statistics have to be held.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kBT = 128;   // 2 waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Physical 16-byte piece of logical piece `piece` in row `row` (an involution).
__device__ __forceinline__ int swz(int row, int piece) { return piece ^ (row & 7); }

// Copy of a 64 x D bf16 tile (row-major, contiguous) into LDS, swizzled, in
// two halves: load the tile's pieces into registers (issued before the
// current tile's products, so the loads run behind them), then store them to
// LDS once the current tile is done.
template <int D>
struct TileRegs {
    static constexpr int R = 64 * (D / 8) / kBT;
    u32x4_t v[R];
};
template <int D>
__device__ __forceinline__ void fetch_tile(TileRegs<D>& t, const uint16_t* src, int tid) {
    constexpr int P = D / 8;
#pragma unroll
    for (int r = 0; r < TileRegs<D>::R; ++r) {
        const int p = tid + r * kBT;
        t.v[r] = *(const u32x4_t*)(src + (p / P) * D + (p % P) * 8);
    }
}
template <int D>
__device__ __forceinline__ void commit_tile(uint16_t* lds, const TileRegs<D>& t, int tid) {
    constexpr int P = D / 8;
#pragma unroll
    for (int r = 0; r < TileRegs<D>::R; ++r) {
        const int p = tid + r * kBT;
        const int row = p / P, c = p % P;
        *(u32x4_t*)(lds + row * D + swz(row, c) * 8) = t.v[r];
    }
}

// Row-wise MFMA operand: 8 consecutive elements of `row`, logical piece `piece`.
template <int D>
__device__ __forceinline__ bf16x8_t rd_row(const uint16_t* lds, int row, int piece) {
    return as_bf16x8(*(const u32x4_t*)(lds + row * D + swz(row, piece) * 8));
}

// Transposed MFMA A operand from a row-major tile Y (rows = contraction index):
// chunk c covers rows 16c .. 16c + 15 in the order of the packed B operand
// (lane half hh holds rows 16c + 4hh + {0..3, 8..11}), columns 32db .. 32db + 31.
template <int D>
__device__ __forceinline__ bf16x8_t rd_tr(const uint16_t* lds, int c, int db, int hh, int gi, int gsel) {
    const int d0 = 32 * db + 16 * gsel + 4 * (gi & 3);
    const int r0 = 16 * c + 4 * hh + (gi >> 2);
    const int r1 = r0 + 8;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(lds + r0 * D + swz(r0, d0 >> 3) * 8 + (d0 & 7)));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(lds + r1 * D + swz(r1, d0 >> 3) * 8 + (d0 & 7)));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    const u32x4_t lh = {l2.x, l2.y, h2.x, h2.y};
    return as_bf16x8(lh);
}

// Pack contraction chunk c (16 rows of a 64-row output pair blk[2]) as a B operand.
__device__ __forceinline__ bf16x8_t pack_chunk(const f32x16_t (&blk)[2], int c) {
    const f32x16_t& x = blk[c >> 1];
    const int o = 8 * (c & 1);
    u32x4_t u;
    u.x = pack_bf16x2(x[o + 0], x[o + 1]);
    u.y = pack_bf16x2(x[o + 2], x[o + 3]);
    u.z = pack_bf16x2(x[o + 4], x[o + 5]);
    u.w = pack_bf16x2(x[o + 6], x[o + 7]);
    return as_bf16x8(u);
}

// Write a lane's transposed accumulator (register i of block db <-> column
// 32db + 8(i/4) + 4hh + i%4) as row `t` of a bf16 tensor or of an fp32 partial.
template <int D>
__device__ __forceinline__ void store_row(const f32x16_t (&acc)[D / 32], float mul, uint16_t* bf_row,
                                          float* f32_row, int hh) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * db + 8 * gq + 4 * hh;
            if (bf_row) {
                u32x2_t w;
                w.x = pack_bf16x2(acc[db][4 * gq + 0] * mul, acc[db][4 * gq + 1] * mul);
                w.y = pack_bf16x2(acc[db][4 * gq + 2] * mul, acc[db][4 * gq + 3] * mul);
                *(u32x2_t*)(bf_row + d) = w;
            } else {
                *(float4*)(f32_row + d) = make_float4(acc[db][4 * gq] * mul, acc[db][4 * gq + 1] * mul,
                                                      acc[db][4 * gq + 2] * mul, acc[db][4 * gq + 3] * mul);
            }
        }
}

// An item's list entries, one per lane, loaded once: entry e of the item is
// then a lane read (v_readlane) instead of a memory round trip in front of the
// next tile's loads.  Items longer than a wave read the list directly.
struct ItemList {
    int32_t first, n, idx;
    uint32_t sub;
    __device__ __forceinline__ bool in_regs() const { return n <= 64; }
};
// Debug builds (BSATTN_DEBUG): a list entry at or past `limit` sets bit 16 of
// *a.dbg and reads as block 0; release builds compile this to nothing.
__device__ __forceinline__ int dbg_entry(const BwdArgs& a, int v, int limit) {
#ifdef BSATTN_DEBUG
    if (v < 0 || v >= limit) {
        atomicOr(a.dbg, 16u);
        v = 0;
    }
#endif
    return v;
}
__device__ __forceinline__ ItemList load_list(const BwdArgs& a, const BwdItem& item, bool with_sub, int limit) {
    ItemList l;
    l.first = item.begin;
    l.n = item.end - item.begin;
    const int lane = threadIdx.x & 63;
    const bool mine = lane < l.n;
    l.idx = mine ? dbg_entry(a, a.idx[item.begin + lane], limit) : 0;
    l.sub = with_sub && mine ? (uint32_t)a.idx_sub[item.begin + lane] : 0u;
    return l;
}
__device__ __forceinline__ int list_idx(const BwdArgs& a, const ItemList& l, int e, int limit) {
    return l.in_regs() ? __builtin_amdgcn_readlane(l.idx, e - l.first) : dbg_entry(a, a.idx[e], limit);
}
__device__ __forceinline__ int list_sub(const BwdArgs& a, const ItemList& l, int e) {
    return l.in_regs() ? (int)__builtin_amdgcn_readlane(l.sub, e - l.first) : (int)a.idx_sub[e];
}

// Workgroup -> (batch entry, head, item).  Workgroups are dealt round-robin
// to the 8 XCDs; XCD x takes the (b, h) groups x, x + 8, ... one after the
// other, so that the tiles a group's items read stay in that XCD's L2.
__device__ __forceinline__ bool take_item(const BwdArgs& a, int& b, int& h, int& blk, BwdItem& item) {
    const int x = blockIdx.x % kXcds;
    const int k = blockIdx.x / kXcds;
    const int g = x + kXcds * (k / a.items_per_head);
    if (g >= a.B * a.H) return false;
    b = g / a.H;
    h = g % a.H;
    item = a.items[(size_t)h * a.items_per_head + k % a.items_per_head];
    if (item.head_blk < 0) return false;
#ifdef BSATTN_DEBUG
    // debug builds: an item out of bounds sets bit 8 of *a.dbg and is skipped
    if (item.head_blk / a.nb != h || item.begin > item.end || item.begin < 0 || item.slot < -1 ||
        item.slot >= a.n_slots) {
        atomicOr(a.dbg, 8u);
        return false;
    }
#endif
    blk = item.head_blk % a.nb;
    return true;
}

// dQ pass: workgroup = (item, batch entry); wave w owns queries 32w .. 32w + 31
// of query block `blk`, each lane one query.
template <int D, int MASK>
__global__ __launch_bounds__(kBT) void bwd_dq_kernel(const BwdArgs a) {
    constexpr int NC = D / 16, NDB = D / 32, TILE = 64 * D;
    __shared__ __attribute__((aligned(1024))) uint16_t kt[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vt[TILE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ql = lane & 31, hh = lane >> 5, gi = lane & 15, gsel = (lane >> 4) & 1;
    int b, h, blk;
    BwdItem item;
    if (!take_item(a, b, h, blk, item)) return;
    const size_t grp = (size_t)b * a.H + h;
    const size_t gbase = grp * a.L * D;
    // this lane's query: row 32 wave + ql of query block blk, or (MASK_ROUTED_Q)
    // of routed tile blk, whose rows are gathered from routed_rows (-1: none)
    int t = blk * 64 + wave * 32 + ql;
    if (MASK == MASK_ROUTED_Q) {
        const int kk = t;
        t = kk < a.n_routed ? a.routed_rows[grp * a.routed_stride + kk] : -1;
        if (t >= a.L) t = -1;
    }

    bf16x8_t qf[NC], dof[NC];
    u32x4_t ug[NC], uo[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const size_t off = gbase + (size_t)max(t, 0) * D + 16 * c + 8 * hh;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        qf[c] = as_bf16x8(t >= 0 ? *(const u32x4_t*)((const uint16_t*)a.q + off) : zero);
        ug[c] = t >= 0 ? *(const u32x4_t*)((const uint16_t*)a.dout + off) : zero;
        uo[c] = t >= 0 ? *(const u32x4_t*)((const uint16_t*)a.out + off) : zero;
        dof[c] = as_bf16x8(ug[c]);
    }
    const float lse = t >= 0 ? a.lse[grp * a.L + t] : -INFINITY;
    const float nl2 = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
    const int valid = MASK == MASK_PAD ? min(max(a.valid_len[b], 0), a.L) : a.L;
    const float c2 = a.scale_log2;

    f32x16_t dqa[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqa[db][i] = 0.f;

    // key block of list entry e: the layout's row list, or (routed tiles) every block in order
    const ItemList lst = MASK == MASK_ROUTED_Q ? ItemList{item.begin, 0, 0, 0u} : load_list(a, item, MASK == MASK_SUB, a.nb);
#ifdef BSATTN_DEBUG
    if (MASK == MASK_ROUTED_Q && item.end > a.nb) {   // a routed tile's entries are the key blocks themselves
        atomicOr(a.dbg, 16u);
        item.end = item.begin;
    }
#endif
    auto key_block = [&](int e) -> int { return MASK == MASK_ROUTED_Q ? e : list_idx(a, lst, e, a.nb); };
    TileRegs<D> kr, vr;
    if (item.begin < item.end) {
        const int j0 = key_block(item.begin);
        fetch_tile<D>(kr, (const uint16_t*)a.k + gbase + (size_t)j0 * TILE, tid);
        fetch_tile<D>(vr, (const uint16_t*)a.v + gbase + (size_t)j0 * TILE, tid);
    }
    // delta = rowsum(dO * O) for this lane's query (lanes l and l + 32 hold the
    // two halves of the row), formed once the first tile's loads are out; the
    // dK/dV pass, which runs after this one, reads it (every item of a row
    // writes the same value)
    float dl = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dl = fmaf(bf16_to_f32(uo[c][e] & 0xffffu), bf16_to_f32(ug[c][e] & 0xffffu), dl);
            dl = fmaf(bf16_to_f32(uo[c][e] >> 16), bf16_to_f32(ug[c][e] >> 16), dl);
        }
    dl += __shfl_xor(dl, 32);
    if (hh == 0 && t >= 0) a.delta[grp * a.L + t] = dl;
    for (int e = item.begin; e < item.end; ++e) {
        const int j = key_block(e);
        // 32-token blocks: key halves this wave's query half may see
        const int sub = MASK == MASK_SUB ? list_sub(a, lst, e) >> (2 * wave) : 3;
        // band layouts: a tile whose farthest (query, key) pair is inside the band needs no mask
        const bool band_cut = MASK == MASK_BAND && 64 * abs(blk - j) + 63 > a.band;
        __syncthreads();   // the previous tile's reads are done
        commit_tile<D>(kt, kr, tid);
        commit_tile<D>(vt, vr, tid);
        __syncthreads();
        if (e + 1 < item.end) {   // the next tile's loads run behind this tile's products
            const int jn = key_block(e + 1);
            fetch_tile<D>(kr, (const uint16_t*)a.k + gbase + (size_t)jn * TILE, tid);
            fetch_tile<D>(vr, (const uint16_t*)a.v + gbase + (size_t)jn * TILE, tid);
        }
        // S^T = K Q^T and dP^T = V dO^T: block kb holds keys 32kb .. 32kb + 31
        f32x16_t s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(kt, 32 * kb + ql, 2 * c + hh), qf[c], s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(vt, 32 * kb + ql, 2 * c + hh), dof[c], dp[kb], 0, 0, 0);
            }
        }
        // dS^T = P^T * (dP^T - delta), P^T = exp2(s * scale * log2e - LSE * log2e)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, nl2));
                if (MASK == MASK_PAD && j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4) >= valid) p = 0.f;
                if (MASK == MASK_SUB && !((sub >> kb) & 1)) p = 0.f;
                if (MASK == MASK_BAND && band_cut && abs(t - (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4))) > a.band)
                    p = 0.f;
                s[kb][i] = p * (dp[kb][i] - dl);
            }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8_t u = pack_chunk(s, c);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(kt, c, db, hh, gi, gsel), u, dqa[db], 0, 0, 0);
        }
    }
    if (item.slot < 0) {
        if (t >= 0) store_row<D>(dqa, a.scale, (uint16_t*)a.dq + gbase + (size_t)t * D, nullptr, hh);
    } else {
        float* row = a.ws_dq + (((size_t)b * a.n_slots + item.slot) * 64 + wave * 32 + ql) * D;
        store_row<D>(dqa, a.scale, nullptr, row, hh);
    }
}

// dK/dV pass: workgroup = (item, batch entry); wave w owns keys 32w .. 32w + 31
// of key block `blk`, each lane one key.
template <int D, int MASK>
__global__ __launch_bounds__(kBT) void bwd_dkdv_kernel(const BwdArgs a) {
    constexpr int NC = D / 16, NDB = D / 32, TILE = 64 * D;
    __shared__ __attribute__((aligned(1024))) uint16_t qt[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t ot[TILE];   // dO tile
    __shared__ __attribute__((aligned(16))) float nlse[64];       // -LSE / scale (-inf: row sees no key)
    __shared__ __attribute__((aligned(16))) float ndel[64];       // -delta
    __shared__ __attribute__((aligned(16))) int qtok[64];         // query token of each row (-1: none)

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kl = lane & 31, hh = lane >> 5, gi = lane & 15, gsel = (lane >> 4) & 1;
    int b, h, blk;
    BwdItem item;
    if (!take_item(a, b, h, blk, item)) return;
    const size_t grp = (size_t)b * a.H + h;
    const size_t gbase = grp * a.L * D;
    const int key = blk * 64 + wave * 32 + kl;

    bf16x8_t kf[NC], vf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kf[c] = as_bf16x8(*(const u32x4_t*)((const uint16_t*)a.k + gbase + (size_t)key * D + 16 * c + 8 * hh));
        vf[c] = as_bf16x8(*(const u32x4_t*)((const uint16_t*)a.v + gbase + (size_t)key * D + 16 * c + 8 * hh));
    }
    const bool key_ok = MASK == MASK_PAD ? key < min(max(a.valid_len[b], 0), a.L) : true;
    const float c2 = a.scale_log2;

    f32x16_t dka[NDB], dva[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dka[db][i] = dva[db][i] = 0.f;

    TileRegs<D> qr, orr;
    float lse_r = 0.f, del_r = 0.f;
    int tok_r = 0;
    // token of row `row` of query entry ib: query block ib, or (ib >= nb, MASK_BAND_ROUTED)
    // row `row` of routed tile ib - nb (-1 past the routed rows)
    auto row_token = [&](int ib, int row) -> int {
        if (MASK != MASK_BAND_ROUTED || ib < a.nb) return ib * 64 + row;
        const int kk = (ib - a.nb) * 64 + row;
        const int t = kk < a.n_routed ? a.routed_rows[grp * a.routed_stride + kk] : -1;
        return t < a.L ? t : -1;
    };
    auto fetch = [&](int ib) {
        if (MASK == MASK_BAND_ROUTED && ib >= a.nb) {
            // a routed tile: its rows gathered, missing rows zero
            constexpr int P = D / 8;
#pragma unroll
            for (int r = 0; r < TileRegs<D>::R; ++r) {
                const int p = tid + r * kBT;
                const int t = row_token(ib, p / P);
                const size_t off = gbase + (size_t)max(t, 0) * D + (p % P) * 8;
                const u32x4_t zero = {0u, 0u, 0u, 0u};
                qr.v[r] = t >= 0 ? *(const u32x4_t*)((const uint16_t*)a.q + off) : zero;
                orr.v[r] = t >= 0 ? *(const u32x4_t*)((const uint16_t*)a.dout + off) : zero;
            }
        } else {
            fetch_tile<D>(qr, (const uint16_t*)a.q + gbase + (size_t)ib * TILE, tid);
            fetch_tile<D>(orr, (const uint16_t*)a.dout + gbase + (size_t)ib * TILE, tid);
        }
        if (tid < 64) {
            tok_r = row_token(ib, tid);
            const size_t r = grp * a.L + (size_t)max(tok_r, 0);
            lse_r = tok_r >= 0 ? a.lse[r] : -INFINITY;
            del_r = tok_r >= 0 ? a.delta[r] : 0.f;
        }
    };
    // query blocks, and (MASK_BAND_ROUTED) routed tiles nb + r
    const int qlimit = a.nb + (MASK == MASK_BAND_ROUTED ? (a.n_routed + 63) / 64 : 0);
    const ItemList lst = load_list(a, item, MASK == MASK_SUB, qlimit);
    if (item.begin < item.end) fetch(list_idx(a, lst, item.begin, qlimit));
    for (int e = item.begin; e < item.end; ++e) {
        // 32-token blocks: query halves that may see this wave's key half
        const int sub = MASK == MASK_SUB ? list_sub(a, lst, e) >> wave : 15;
        // band layouts: query block ib, masked per pair unless the whole tile is inside the band
        const int ib = list_idx(a, lst, e, qlimit);
        const bool routed_entry = MASK == MASK_BAND_ROUTED && ib >= a.nb;
        const bool band_cut = (MASK == MASK_BAND || MASK == MASK_BAND_ROUTED) && !routed_entry &&
                              64 * abs(blk - ib) + 63 > a.band;
        __syncthreads();
        commit_tile<D>(qt, qr, tid);
        commit_tile<D>(ot, orr, tid);
        if (tid < 64) {
            nlse[tid] = lse_r == -INFINITY ? -INFINITY : -lse_r / a.scale;
            ndel[tid] = -del_r;
            qtok[tid] = tok_r;
        }
        __syncthreads();
        if (e + 1 < item.end) fetch(list_idx(a, lst, e + 1, qlimit));   // behind this tile's products
        // S = Q K^T - LSE/scale and dP = dO V^T - delta: block qb holds queries 32qb .. 32qb + 31,
        // register i <-> query 32qb + 8(i/4) + 4hh + i%4
        f32x16_t s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 l4 = *(const float4*)(nlse + 32 * qb + 8 * g4 + 4 * hh);
                const float4 d4 = *(const float4*)(ndel + 32 * qb + 8 * g4 + 4 * hh);
                s[qb][4 * g4 + 0] = l4.x; s[qb][4 * g4 + 1] = l4.y; s[qb][4 * g4 + 2] = l4.z; s[qb][4 * g4 + 3] = l4.w;
                dp[qb][4 * g4 + 0] = d4.x; dp[qb][4 * g4 + 1] = d4.y; dp[qb][4 * g4 + 2] = d4.z; dp[qb][4 * g4 + 3] = d4.w;
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(qt, 32 * qb + kl, 2 * c + hh), kf[c], s[qb], 0, 0, 0);
                dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(ot, 32 * qb + kl, 2 * c + hh), vf[c], dp[qb], 0, 0, 0);
            }
        }
        // P = exp2(S * scale * log2e), dS = P * (dP - delta)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            // routed tiles: a pair counts here only outside the band (the band entries hold the rest)
            int tk[16];
            if (MASK == MASK_BAND_ROUTED && routed_entry) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int4 t4 = *(const int4*)(qtok + 32 * qb + 8 * g4 + 4 * hh);
                    tk[4 * g4 + 0] = t4.x; tk[4 * g4 + 1] = t4.y; tk[4 * g4 + 2] = t4.z; tk[4 * g4 + 3] = t4.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(s[qb][i] * c2);
                if (!key_ok) p = 0.f;
                if (MASK == MASK_SUB && !((sub >> (2 * qb)) & 1)) p = 0.f;
                if ((MASK == MASK_BAND || MASK == MASK_BAND_ROUTED) && band_cut &&
                    abs(ib * 64 + 32 * qb + 8 * (i / 4) + 4 * hh + (i % 4) - key) > a.band)
                    p = 0.f;
                if (MASK == MASK_BAND_ROUTED && routed_entry && (tk[i] < 0 || abs(tk[i] - key) <= a.band)) p = 0.f;
                s[qb][i] = p;
                dp[qb][i] *= p;
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8_t up = pack_chunk(s, c);
            const bf16x8_t ud = pack_chunk(dp, c);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(ot, c, db, hh, gi, gsel), up, dva[db], 0, 0, 0);
                dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(qt, c, db, hh, gi, gsel), ud, dka[db], 0, 0, 0);
            }
        }
    }
    if (item.slot < 0) {
        store_row<D>(dka, a.scale, (uint16_t*)a.dk + gbase + (size_t)key * D, nullptr, hh);
        store_row<D>(dva, 1.f, (uint16_t*)a.dv + gbase + (size_t)key * D, nullptr, hh);
    } else {
        const size_t r = (((size_t)b * a.n_slots + item.slot) * 64 + wave * 32 + kl) * D;
        store_row<D>(dka, a.scale, nullptr, a.ws_dk + r, hh);
        store_row<D>(dva, 1.f, nullptr, a.ws_dv + r, hh);
    }
}

// Sum of a split row's (column's) fp32 partials into the bf16 output block.
// One workgroup per (split, batch entry, 1024-element slice of the 64 x D
// block); each thread owns 4 elements and issues its chunks' loads together.
template <int D>
__global__ __launch_bounds__(256) void bwd_sum_kernel(const BwdArgs a, int which) {
    constexpr int SLICES = 64 * D / 1024;
    const int slice = blockIdx.x % SLICES;
    const int rest = blockIdx.x / SLICES;
    const int si = rest / a.B, b = rest % a.B;
    const BwdSum sm = a.sums[si];
    const int h = sm.head_blk / a.nb, blk = sm.head_blk % a.nb;
    const size_t out_base = (((size_t)b * a.H + h) * a.L + (size_t)blk * 64) * D;
    const int x = slice * 1024 + threadIdx.x * 4;
    const int n_out = which == 0 ? 1 : 2;
    for (int o = 0; o < n_out; ++o) {
        const float* ws = which == 0 ? a.ws_dq : (o == 0 ? a.ws_dk : a.ws_dv);
        uint16_t* dst = (uint16_t*)(which == 0 ? a.dq : (o == 0 ? a.dk : a.dv)) + out_base;
        const float* src = ws + ((size_t)b * a.n_slots + sm.first_slot) * 64 * D + x;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int ch = 0;
        for (; ch + 4 <= sm.n_chunks; ch += 4) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *(const float4*)(src + (size_t)(ch + u) * 64 * D);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
            }
        }
        for (; ch < sm.n_chunks; ++ch) {
            const float4 v = *(const float4*)(src + (size_t)ch * 64 * D);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        u32x2_t w;
        w.x = pack_bf16x2(acc.x, acc.y);
        w.y = pack_bf16x2(acc.z, acc.w);
        *(u32x2_t*)(dst + x) = w;
    }
}

// Sum of a routed tile's dQ partials into the dQ rows of its routed tokens.
// One workgroup per (tile, batch entry, 1024-element slice of the 64 x D block).
template <int D>
__global__ __launch_bounds__(256) void bwd_routed_sum_kernel(const BwdArgs a) {
    constexpr int SLICES = 64 * D / 1024;
    const int slice = blockIdx.x % SLICES;
    const int rest = blockIdx.x / SLICES;
    const int si = rest / a.B, b = rest % a.B;
    const BwdSum sm = a.sums[si];
    const int h = sm.head_blk / a.nb, r = sm.head_blk % a.nb;
    const size_t grp = (size_t)b * a.H + h;
    const int x = slice * 1024 + threadIdx.x * 4;
    const int kk = r * 64 + x / D;
    if (kk >= a.n_routed) return;
    const int t = a.routed_rows[grp * a.routed_stride + kk];
    if (t < 0 || t >= a.L) return;
    const float* src = a.ws_dq + ((size_t)b * a.n_slots + sm.first_slot) * 64 * D + x;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ch = 0; ch < sm.n_chunks; ++ch) {
        const float4 v = *(const float4*)(src + (size_t)ch * 64 * D);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    u32x2_t w;
    w.x = pack_bf16x2(acc.x, acc.y);
    w.y = pack_bf16x2(acc.z, acc.w);
    *(u32x2_t*)((uint16_t*)a.dq + (grp * a.L + t) * D + x % D) = w;
}

template <int D, int MASK>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
    const int64_t groups = (int64_t)a.B * a.H;
    const int64_t grid = (groups + kXcds - 1) / kXcds * kXcds * a.items_per_head;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, MASK>), dim3((unsigned)grid), dim3(kBT), 0, s, a);
    return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s, hipEvent_t before, hipEvent_t after) {
    const int64_t groups = (int64_t)a.B * a.H;
    const int64_t grid = (groups + kXcds - 1) / kXcds * kXcds * a.items_per_head;
    if (grid == 0) return hipSuccess;
    // given events, the dispatch records the kernel's own start and stop
    hipExtLaunchKernelGGL((bwd_dkdv_kernel<D, MASK>), dim3((unsigned)grid), dim3(kBT), 0, s, before, after, 0, a);
    return hipGetLastError();
}

}  // namespace

#ifdef BSATTN_DEBUG
// Debug builds: the word the backward kernels report list errors into.
__device__ uint32_t g_bwd_dbg_word;

// Clear the word, run `launch` with it, read it back (synchronising the
// stream); a set bit is reported as a device-side assert.
template <class F>
hipError_t debug_launch(const BwdArgs& a, hipStream_t s, F&& launch) {
    uint32_t* dw = nullptr;
    hipError_t e = hipGetSymbolAddress((void**)&dw, HIP_SYMBOL(g_bwd_dbg_word));
    if (e != hipSuccess) return e;
    static const uint32_t zero = 0;
    if ((e = hipMemcpyAsync(dw, &zero, sizeof(zero), hipMemcpyHostToDevice, s)) != hipSuccess) return e;
    BwdArgs ad = a;
    ad.dbg = dw;
    if ((e = launch(ad)) != hipSuccess) return e;
    uint32_t flag = 0;
    if ((e = hipMemcpyAsync(&flag, dw, sizeof(flag), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    return flag ? hipErrorAssert : hipSuccess;
}
#endif

static hipError_t launch_bwd_dq_impl(const BwdArgs& a, int head_dim, int mask, hipStream_t s) {
    if (mask == MASK_ROUTED_Q)
        return head_dim == 64 ? launch_dq_t<64, MASK_ROUTED_Q>(a, s) : launch_dq_t<128, MASK_ROUTED_Q>(a, s);
    if (head_dim == 64)
        return mask == MASK_PAD   ? launch_dq_t<64, MASK_PAD>(a, s)
             : mask == MASK_SUB   ? launch_dq_t<64, MASK_SUB>(a, s)
             : mask == MASK_BAND  ? launch_dq_t<64, MASK_BAND>(a, s)
                                  : launch_dq_t<64, MASK_NONE>(a, s);
    return mask == MASK_PAD   ? launch_dq_t<128, MASK_PAD>(a, s)
         : mask == MASK_SUB   ? launch_dq_t<128, MASK_SUB>(a, s)
         : mask == MASK_BAND  ? launch_dq_t<128, MASK_BAND>(a, s)
                              : launch_dq_t<128, MASK_NONE>(a, s);
}

static hipError_t launch_bwd_dkdv_impl(const BwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before,
                                       hipEvent_t after) {
    if (mask == MASK_BAND_ROUTED)
        return head_dim == 64 ? launch_dkdv_t<64, MASK_BAND_ROUTED>(a, s, before, after)
                              : launch_dkdv_t<128, MASK_BAND_ROUTED>(a, s, before, after);
    if (head_dim == 64)
        return mask == MASK_PAD   ? launch_dkdv_t<64, MASK_PAD>(a, s, before, after)
             : mask == MASK_SUB   ? launch_dkdv_t<64, MASK_SUB>(a, s, before, after)
             : mask == MASK_BAND  ? launch_dkdv_t<64, MASK_BAND>(a, s, before, after)
                                  : launch_dkdv_t<64, MASK_NONE>(a, s, before, after);
    return mask == MASK_PAD   ? launch_dkdv_t<128, MASK_PAD>(a, s, before, after)
         : mask == MASK_SUB   ? launch_dkdv_t<128, MASK_SUB>(a, s, before, after)
         : mask == MASK_BAND  ? launch_dkdv_t<128, MASK_BAND>(a, s, before, after)
                              : launch_dkdv_t<128, MASK_NONE>(a, s, before, after);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int mask, hipStream_t s) {
#ifdef BSATTN_DEBUG
    return debug_launch(a, s, [&](const BwdArgs& ad) { return launch_bwd_dq_impl(ad, head_dim, mask, s); });
#else
    return launch_bwd_dq_impl(a, head_dim, mask, s);
#endif
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before,
                           hipEvent_t after) {
#ifdef BSATTN_DEBUG
    return debug_launch(a, s, [&](const BwdArgs& ad) {
        return launch_bwd_dkdv_impl(ad, head_dim, mask, s, before, after);
    });
#else
    return launch_bwd_dkdv_impl(a, head_dim, mask, s, before, after);
#endif
}

hipError_t launch_bwd_routed_sum(const BwdArgs& a, int head_dim, hipStream_t s) {
    const int64_t grid = (int64_t)a.n_sums * a.B * (64 * head_dim / 1024);
    if (grid == 0) return hipSuccess;
    if (head_dim == 64) hipLaunchKernelGGL((bwd_routed_sum_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_routed_sum_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_sum(const BwdArgs& a, int head_dim, int which, hipStream_t s) {
    const int64_t grid = (int64_t)a.n_sums * a.B * (64 * head_dim / 1024);
    if (grid == 0) return hipSuccess;
    if (head_dim == 64) hipLaunchKernelGGL((bwd_sum_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, a, which);
    else hipLaunchKernelGGL((bwd_sum_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, a, which);
    return hipGetLastError();
}

}  // namespace bsattn
