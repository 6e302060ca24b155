// fwd_bf16.hip -- block-sparse attention forward, bf16 in/out, bf16 MFMA with fp32 accumulation.
//
// What is computed (Adaptive Sparse Transformer page, "Adapt or Perish: 新手入门指南 –
// Adaptive Sparse Transformer 核心原理与实战", the SparseAttention formula; masked
// scores are -inf): for every query row, softmax over the allowed keys of
// scale * q.k, times V.  Attention runs only on the non-zero 64x64 blocks of
// the block-CSR layout (SQA page, "Transformer计算效率优化：SQA稀疏注意力机制详解",
// section 3.1: FlashAttention-style computation restricted to non-zero
// blocks; section 5: 64x64 blocks staged in on-chip memory).
//
// Design for gfx950 (CDNA4: wave64, 4 SIMDs and 160 KB LDS per CU, 8 XCDs):
//  * One workgroup = 2 waves = one 64-row query tile walking its list of key
//    blocks; wave w owns query rows 32w..32w+31 against all 64 keys of every
//    key tile.  The list (at most 64 blocks) is read once into a VGPR and
//    each step takes its block index with v_readlane.
//  * K and V tiles travel global -> LDS by direct LDS loads
//    (global_load_lds_dwordx4, issued from inline asm so that only the
//    pipeline's explicit waits govern them): no staging registers, no LDS
//    store instructions.  Tiles are row-major in LDS with the 16-byte pieces of
//    every row XOR-swizzled so that both readers are bank-conflict free:
//    K through ds_read_b128 (A operand of S^T = K Q^T), V through
//    ds_read_b64_tr_b16, whose 16-lane transpose hands each lane 4
//    consecutive keys of one d column -- exactly the A operand of
//    O^T = V^T P^T, with no transpose pass over V.
//  * Two LDS stages: the loads of the next tile are in flight while the
//    current one is computed (a third stage cost more in occupancy than it
//    gained in latency hiding).  Every step waits
//    with an explicit vmcnt for its own tile only and passes a plain
//    s_barrier (a fenced __syncthreads would wait for all loads in flight).
//  * Scores are computed transposed with v_mfma_f32_32x32x16_bf16: each lane
//    holds 16 keys of ONE query per 32x32 block, so row reductions are in-lane
//    plus one v_permlane32_swap between half-waves.  The same registers,
//    rounded to bf16, are the B operand of the PV product (the order of a
//    contraction index is free as long as both operands agree).
//  * Online softmax in the log2 domain, p = exp2(s*scale*log2e - m): one FMA
//    into v_exp_f32 (half rate on gfx950).  The running max m is only raised
//    when a tile's max exceeds it by more than kLazyMax (so p <= 2^kLazyMax,
//    harmless in fp32 and bf16), which skips the O rescale on almost every
//    tile.  Row sums add the fp32 probabilities (v_dot2c_f32_bf16 on the bf16
//    P gave wrong sums on gfx950 in testing, so it is not used).
//  * Rows longer than 16 blocks (global rows, routed tiles) are split into
//    chunks run by different workgroups; each writes a normalised fp32
//    partial and its LSE, and a small second launch merges them by
//    log-sum-exp.  (Merging inside the attention kernel by the last chunk to
//    arrive needs device-scope release/acquire fences, which on gfx950 write
//    back and invalidate the XCD's L2 and slowed every resident workgroup.)
//  * Scheduling: workgroups are dealt round-robin to the 8 XCDs; workgroup i
//    runs on XCD i%8, and the kernel maps it to the (i/8)-th unit of the
//    (batch, head) groups assigned to that XCD, so every group's K/V is read
//    by one XCD and stays in its L2.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // native vectors stay in registers
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;   // log2 units: p never exceeds 2^8
constexpr int kThreads = 128;      // 2 waves per workgroup

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// Combine a value across the two half-waves (lanes l and l^32).
// v_permlane32_swap exchanges one half of its first operand with the other
// half of its second; with x in both, the two results hold x from the lower
// and from the upper half-wave in every lane, in some order -- so their max
// and their sum are the pairwise max and sum whatever the order.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: outstanding direct-to-LDS loads
// of later tiles stay in flight (each wave has already waited for its own
// loads of the tile about to be read).  The empty asm keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D>
struct Geo {
    static constexpr int PIECES = D / 8;                 // 16-byte pieces per K/V row
    static constexpr int TILE = 64 * D;                  // bf16 elements of one K or V tile
    static constexpr int LPT = 64 * PIECES / kThreads;   // direct loads per thread per K (or V) tile
    static constexpr int NC = D / 16;                    // 16-wide contraction chunks of S^T
    static constexpr int NDB = D / 32;                   // 32-row blocks of O^T
};

// One direct global -> LDS load of 16 bytes per lane from sbase + voff: lane
// i's bytes land at LDS byte address lds + 16 i (sbase and lds are
// wave-uniform SGPR values, voff a per-lane byte offset).  Written as inline
// asm so that the compiler does not track it: the only waits on these loads
// are the explicit vmcnt waits of the pipeline (the compiler's own LDS-DMA
// alias tracking inserts full drains at loop headers).  The instruction
// writes no register; M0 is saved and restored around it, with the wait
// state M0 needs before an LDS load.
__device__ __forceinline__ void lds_load16(uint32_t voff, const void* sbase, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)LDS_PTR(p);
}

// Physical position of a 16-byte piece inside its row (XOR is an involution,
// so the same map converts logical <-> physical).
__device__ __forceinline__ int swz_k(int row, int piece) { return piece ^ (row & 7); }
__device__ __forceinline__ int swz_v(int row, int piece) { return piece ^ ((row & 3) << 1); }

// Direct loads of key block j into one LDS stage [K tile | V tile].  Each wave
// instruction fills 1 KB of LDS contiguously (lane i -> +16 i); lane i loads
// the global piece that the swizzle places at that slot, and the 8 (16) lanes
// covering one row read the whole 128 (256) byte row.  Per-lane byte offsets
// are fixed for the whole walk (koffs/voffs); the tile base and the LDS
// destination are scalars, so a load costs no vector ALU work.
template <int D>
__device__ __forceinline__ void issue_tile(const uint16_t* kp, const uint16_t* vp, int j,
                                           const uint32_t (&koffs)[Geo<D>::LPT],
                                           const uint32_t (&voffs)[Geo<D>::LPT], uint32_t lds_wave) {
    using Gm = Geo<D>;
    const uint16_t* kt = kp + (size_t)j * 64 * D;
    const uint16_t* vt = vp + (size_t)j * 64 * D;
#pragma unroll
    for (int r = 0; r < Gm::LPT; ++r) {
        lds_load16(koffs[r], kt, lds_wave + r * kThreads * 16);
        lds_load16(voffs[r], vt, lds_wave + 2 * Gm::TILE + r * kThreads * 16);
    }
}

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(const FwdArgs a) {
    using Gm = Geo<D>;
    constexpr int NC = Gm::NC, NDB = Gm::NDB, TILE = Gm::TILE;
    __shared__ __attribute__((aligned(1024))) uint16_t st0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t st1[2 * TILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int rloc = wave * 32 + ql;  // this lane's query row within the tile

    // ---- decode: XCD x = blockIdx % 8 runs groups g = x, x+8, ... in order ----
    const int G = a.B * a.H;
    const int nru = a.n_routed > 0 ? a.n_rt * a.r_chunks : 0;   // routed units per group
    const int per_group = nru + a.items_per_head;
    const int x = blockIdx.x % kXcds;
    const int p = blockIdx.x / kXcds;
    const int g = x + kXcds * (p / per_group);
    const int it = p % per_group;
    if (g >= G) return;
    const int b = g / a.H, h = g % a.H;

    int qblk = 0, cb, ce, slot, rt = 0;
    bool routed;
    if (it < nru) {
        rt = it / a.r_chunks;
        const int c = it % a.r_chunks;
        cb = c * a.r_chunk_tiles;
        ce = min(a.nb, cb + a.r_chunk_tiles);
        slot = a.r_slot_base + (g * a.n_rt + rt) * a.r_chunks + c;
        routed = true;
    } else {
        const WorkItem wi = a.items[h * a.items_per_head + (it - nru)];
        if (wi.row < 0) return;
        qblk = wi.row % a.nb;
        cb = wi.col_begin;
        ce = wi.col_end;
        slot = wi.slot < 0 ? -1 : b * a.n_slots + wi.slot;
        routed = false;
    }
    const size_t bh = (size_t)g;

    auto query_token = [&](int r) -> int {   // token of tile row r (-1: unused routed row)
        if (!routed) return qblk * 64 + r;
        const int kk = rt * 64 + r;
        const int t = kk < a.n_routed ? a.routed_rows[bh * a.n_routed + kk] : -1;
        return (t >= a.L) ? -1 : t;          // out-of-range rows are skipped, never dereferenced
    };
    const int tq = query_token(rloc);

    // Key blocks of this item, one per lane (<= 64 by construction of the schedule).
    int n = ce - cb;
    const int colv = lane < n ? (routed ? cb + lane : a.col_idx[cb + lane]) : 0;
    int valid = a.L;
    if (MASK == MASK_PAD) {
        valid = min(max(a.valid_len[b], 0), a.L);
        // ascending blocks: keep those that start before the valid length
        n = __builtin_popcountll(__ballot(lane < n && colv * 64 < valid));
    }
    auto tile_of = [&](int t) -> int { return __builtin_amdgcn_readlane(colv, t); };

    const uint16_t* qp = (const uint16_t*)a.q + bh * (size_t)a.L * D;
    const uint16_t* kp = (const uint16_t*)a.k + bh * (size_t)a.L * D;
    const uint16_t* vp = (const uint16_t*)a.v + bh * (size_t)a.L * D;

    // Q^T fragments (B operand of S^T): lane (ql, hh) holds Q[row][16c + 8hh .. +7].
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
    float m = -INFINITY;   // running (lazily raised) max of scaled scores, log2 units
    float l = 0.f;         // sum of this lane's probabilities
    const float c2 = a.scale_log2;

    // Per-lane LDS offsets (elements) of the fragment reads, fixed for the whole walk.
    int koff[2][NC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int row = 32 * kb + ql;
            koff[kb][c] = row * D + swz_k(row, 2 * c + hh) * 8;
        }
    // V: the 16-lane transpose read gives lane i of group G, value e, the
    // element (i & 3) of source lane 4e + (i >> 2).  Source lane i therefore
    // points at key row 16c + 8e2 + 4hh + (i >> 2), columns 32db + 16(G & 1) + 4(i & 3) .. +3,
    // and receives V[16c + 8e2 + 4hh + e][32db + ql] for e = 0..3.
    const int gi = lane & 15, gsel = (lane >> 4) & 1;
    int voff[4][NDB][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int row = 16 * c + 8 * e2 + 4 * hh + (gi >> 2);
                const int d0 = 32 * db + 16 * gsel + 4 * (gi & 3);
                voff[c][db][e2] = row * D + swz_v(row, d0 >> 3) * 8 + (d0 & 7);
            }

    // Direct-load byte offsets of this thread's pieces (fixed for the whole walk)
    // and the wave's LDS destinations in each stage.
    uint32_t koffs[Gm::LPT], voffs[Gm::LPT];
#pragma unroll
    for (int r = 0; r < Gm::LPT; ++r) {
        const int slot = r * kThreads + tid;
        const int row = slot / Gm::PIECES, q = slot % Gm::PIECES;
        koffs[r] = (uint32_t)(row * D + swz_k(row, q) * 8) * 2u;
        voffs[r] = (uint32_t)(row * D + swz_v(row, q) * 8) * 2u;
    }
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(wave * 64 * 16);
    const uint32_t lds0 = lds_addr(st0) + wave_lds, lds1 = lds_addr(st1) + wave_lds;

    auto compute = [&](int t, const uint16_t* Ks) {
        const uint16_t* Vs = Ks + TILE;
        const int j = tile_of(t);
        // S^T (keys x queries): s[kb] register i <-> key 32kb + 8(i/4) + 4hh + i%4.
        bf16x8_t kf[2][NC];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c) kf[kb][c] = as_bf16x8(*(const u32x4_t*)(Ks + koff[kb][c]));
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][c], qf[c], s[kb], 0, 0, 0);
        if (MASK == MASK_PAD) {
            if (j * 64 + 64 > valid) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4) >= valid) s[kb][i] = -INFINITY;
            }
        }
        if (MASK == MASK_BAND) {
            if (!routed) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (abs(tq - (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4))) > a.band)
                            s[kb][i] = -INFINITY;
            }
        }
        // V^T fragments for the PV product, read while the softmax runs.
        bf16x8_t va[4][NDB];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(Vs + voff[c][db][0]));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(Vs + voff[c][db][1]));
                const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                const u32x4_t lh = {l2.x, l2.y, h2.x, h2.y};
                va[c][db] = as_bf16x8(lh);
            }

        float mx = __builtin_fmaxf(__builtin_fmaxf(s[0][0], s[0][1]), s[1][0]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[0][i]), s[0][i + 1]);
#pragma unroll
        for (int i = 1; i < 15; i += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[1][i]), s[1][i + 1]);
        mx = __builtin_fmaxf(mx, s[1][15]);
        mx = pair_max(mx) * c2;
        const bool raise = mx > m + kLazyMax;
        if (__ballot(raise) != 0) {          // wave-uniform: rescale only when some row's max jumped
            const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.f;   // 0 when m was -inf
            const float mn = raise ? mx : m;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            m = mn;
        }
        const float muse = m == -INFINITY ? 0.f : m;

        // P^T fragments: pf[c] (c = 0..3) element e <-> key 16c + 8(e/4) + 4hh + e%4.
        bf16x8_t pf[4];
        float ls[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u32x4_t u;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[c / 2][8 * (c % 2) + 2 * e], c2, -muse));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[c / 2][8 * (c % 2) + 2 * e + 1], c2, -muse));
                u[e] = pack_bf16x2(p0, p1);
                acc += p0 + p1;
            }
            ls[c] = acc;
            pf[c] = as_bf16x8(u);
        }
        l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c][db], pf[c], o[db], 0, 0, 0);
    };

    // ---- pipelined walk over the key blocks ----
    // The block list and Q must be in registers before the first load
    // addresses and MFMAs; waiting here once keeps the compiler from placing
    // conservative full waits inside the pipeline.  The prologue loads are
    // unconditional (lanes past the list hold block 0, a valid address).
    wait_vmcnt<0>();
    issue_tile<D>(kp, vp, tile_of(0), koffs, voffs, lds0);
    // step t: tile t sits in stage t%2; the loads of tile t+1 go to the other
    // stage, whose last reader (step t-1) is behind the barrier.
    auto step = [&](int t, const uint16_t* cur, uint32_t nxt) {
        wait_vmcnt<0>();
        stage_barrier();
        if (t + 1 < n) issue_tile<D>(kp, vp, tile_of(t + 1), koffs, voffs, nxt);
        compute(t, cur);
    };
    for (int t = 0; t < n; t += 2) {
        step(t, st0, lds1);
        if (t + 1 < n) step(t + 1, st1, lds0);
    }
    wait_vmcnt<0>();   // no direct-to-LDS load may outlive the workgroup

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
    const float lt = pair_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    if (tq >= 0) {
        // O^T register i of block db <-> d = 32db + 8(i/4) + 4hh + i%4
        if (slot < 0) {
            uint16_t* orow = (uint16_t*)a.out + (bh * a.L + tq) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2_t w;
                    w.x = pack_bf16x2(o[db][4 * gq + 0] * inv, o[db][4 * gq + 1] * inv);
                    w.y = pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
                    *(u32x2_t*)(orow + 32 * db + 8 * gq + 4 * hh) = w;
                }
            if (hh == 0) a.lse[bh * a.L + tq] = lse_v;
        } else {
            float* orow = a.ws_o + ((size_t)slot * 64 + rloc) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(float4*)(orow + 32 * db + 8 * gq + 4 * hh) =
                        make_float4(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                                    o[db][4 * gq + 3] * inv);
            if (hh == 0) a.ws_lse[(size_t)slot * 64 + rloc] = lse_v;
        }
    }
}

// Merge of a split row (global rows, routed tiles): the chunks of the row
// wrote fp32 partials normalised over their own keys plus their LSE; the row's
// LSE is the log-sum-exp of the chunk LSEs and O the LSE-weighted mean of the
// partial outputs.  A chunk with no allowed key has LSE -inf and weight 0; a
// row with no allowed key at all gets O = 0, LSE = -inf.  Runs as its own
// launch after the attention kernel, so stream order makes the partials
// visible without any device-scope fence.  One workgroup per split row,
// four threads per query row, each owning D/4 columns.
template <int D>
__global__ __launch_bounds__(256) void merge_bf16_kernel(const FwdArgs a) {
    constexpr int DP = D / 4;
    const int u = blockIdx.x;
    const int tid = threadIdx.x;
    const int row = tid >> 2, part = tid & 3;
    int first, nch, t;
    size_t bh;
    if (u < a.B * a.n_merges) {
        const int b = u / a.n_merges;
        const MergeItem mi = a.merges[u % a.n_merges];
        bh = (size_t)b * a.H + mi.row / a.nb;
        first = b * a.n_slots + mi.first_slot;
        nch = mi.n_chunks;
        t = (mi.row % a.nb) * 64 + row;
    } else {
        const int v = u - a.B * a.n_merges;
        const int g = v / a.n_rt, rt = v % a.n_rt;
        bh = (size_t)g;
        first = a.r_slot_base + (g * a.n_rt + rt) * a.r_chunks;
        nch = a.r_chunks;
        const int kk = rt * 64 + row;
        t = kk < a.n_routed ? a.routed_rows[bh * a.n_routed + kk] : -1;
        if (t >= a.L) t = -1;   // out-of-range rows are skipped, never dereferenced
    }
    if (t < 0) return;
    const float* lse_p = a.ws_lse + (size_t)first * 64 + row;
    float mxl = -INFINITY;
    for (int c = 0; c < nch; ++c) mxl = __builtin_fmaxf(mxl, lse_p[(size_t)c * 64]);
    uint16_t* orow = (uint16_t*)a.out + (bh * a.L + t) * D + part * DP;
    if (mxl == -INFINITY) {
#pragma unroll
        for (int d = 0; d < DP; d += 2) *(uint32_t*)(orow + d) = 0u;
        if (part == 0) a.lse[bh * a.L + t] = -INFINITY;
        return;
    }
    float acc[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = 0.f;
    float wsum = 0.f;
    for (int c = 0; c < nch; ++c) {
        const float w = expf(lse_p[(size_t)c * 64] - mxl);
        wsum += w;
        const float* src = a.ws_o + ((size_t)(first + c) * 64 + row) * D + part * DP;
#pragma unroll
        for (int d = 0; d < DP; d += 4) {
            const float4 v4 = *(const float4*)(src + d);
            acc[d] += w * v4.x;
            acc[d + 1] += w * v4.y;
            acc[d + 2] += w * v4.z;
            acc[d + 3] += w * v4.w;
        }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int d = 0; d < DP; d += 4) {
        u32x2_t w2;
        w2.x = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
        w2.y = pack_bf16x2(acc[d + 2] * inv, acc[d + 3] * inv);
        *(u32x2_t*)(orow + d) = w2;
    }
    if (part == 0) a.lse[bh * a.L + t] = mxl + logf(wsum);
}

template <int D, int MASK>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
    const int64_t G = (int64_t)a.B * a.H;
    const int64_t nru = a.n_routed > 0 ? (int64_t)a.n_rt * a.r_chunks : 0;
    const int64_t grid = kXcds * ((G + kXcds - 1) / kXcds) * (nru + a.items_per_head);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
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
    const int64_t units = (int64_t)a.B * a.n_merges + (a.n_routed > 0 ? (int64_t)a.B * a.H * a.n_rt : 0);
    if (units == 0) return hipSuccess;
    if (head_dim == 64)
        hipLaunchKernelGGL(merge_bf16_kernel<64>, dim3((unsigned)units), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(merge_bf16_kernel<128>, dim3((unsigned)units), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bsattn
