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
// Two attention kernels share the pieces below.  fwd_bf16_d64_kernel (D = 64)
// runs one workgroup of eight waves per CU, each wave owning a whole 64-row
// query tile and its own list of units; it is described where it is defined.
// fwd_bf16_kernel<D> (D = 128, and the template at any D) runs two-wave
// workgroups:
//  * One workgroup = 2 waves = one 64-row query tile walking its list of key
//    blocks; wave w owns query rows 32w..32w+31 against all 64 keys of every
//    key tile.
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
//    current one is computed.  Every step waits with an explicit vmcnt for
//    its own tile only and passes a plain s_barrier (a fenced __syncthreads
//    would wait for all loads in flight).
//  * Scores are computed transposed with v_mfma_f32_32x32x16_bf16: each lane
//    holds 16 keys of ONE query per 32x32 block, so row reductions are in-lane
//    plus one v_permlane32_swap between half-waves.  The same registers,
//    rounded to bf16, are the B operand of the PV product (the order of a
//    contraction index is free as long as both operands agree).
//  * Online softmax in the log2 domain, p = exp2(s*scale*log2e - m): one FMA
//    into v_exp_f32.  The running max m is taken from the first tile of a
//    unit and afterwards raised only when half a tile's probabilities sum
//    past kSumCap in some lane (then O and l are rescaled and that half is
//    redone), so the per-tile row max and the O rescale are skipped on almost
//    every tile and no probability overflows.  Row sums add the fp32
//    probabilities: v_dot2c_f32_bf16 would add two products per instruction,
//    but of the bf16-rounded probabilities, which moves LSE by up to 2^-9
//    relative on a row with one dominant key -- more than the LSE tolerance.
//  * Rows longer than the chunk size (global rows, routed tiles) are split
//    into chunks run by different workgroups; each writes a normalised fp32
//    partial and its LSE, and a small second launch merges them by
//    log-sum-exp.  (Merging inside the attention kernel by the last chunk to
//    arrive needs device-scope release/acquire fences, which on gfx950 write
//    back and invalidate the XCD's L2 and slowed every resident workgroup.)
//  * Both kernels have STRIDED instances for the attention layer: Q, K and V
//    are read in place from the qkv projection's token-major output and O is
//    written as the concatenated heads, at the strides FwdArgs gives.
//  * Scheduling: workgroups are dealt round-robin to the 8 XCDs; workgroup i
//    runs on XCD i%8, and its list holds units of the (batch, head) groups
//    assigned to that XCD, so every group's K/V is read by one XCD and stays
//    in its L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

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
// A lane's 16 probabilities of half a tile may sum to at most this before the
// running max is raised.  Besides preventing overflow it keeps a dominant
// probability near 1, where its bf16 rounding is exact or small.
constexpr float kSumCap = 256.0f;
// Finite stand-in for the running max of a row that has met no key yet (the
// D = 64 kernel): any finite score then has an infinite probability, which
// trips the kSumCap test, and exp2(kNoMax - m) is 0 for every finite m.
constexpr float kNoMax = -1e30f;
constexpr int kThreads = 128;      // 2 waves per workgroup

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}
// The two bf16 of a packed pair as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// Four direct global -> LDS loads of 16 bytes per lane: load r reads
// sbase + voff[r] + imm_r and writes LDS byte address m0v + imm_r + 16 lane,
// imm_r = 2048 r - 4096 (the instruction offset moves both addresses, so the
// four 2 KB pieces land at m0v - 4096 .. m0v + 4095 with one M0 setting).
// Written as inline asm so that the compiler does not track the loads: the
// only waits on them are the explicit vmcnt waits of the pipeline (the
// compiler's own LDS-DMA alias tracking inserts full drains at loop headers).
// The instructions write no register; M0 is saved and restored around them,
// with the wait state M0 needs before an LDS load.
__device__ __forceinline__ void lds_load16x4(const uint32_t (&voff)[4], const void* sbase, uint32_t m0v) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6 offset:-4096\n\t"
        "global_load_lds_dwordx4 %2, %6 offset:-2048\n\t"
        "global_load_lds_dwordx4 %3, %6\n\t"
        "global_load_lds_dwordx4 %4, %6 offset:2048\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(m0v), "s"(sbase)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)LDS_PTR(p);
}

// Physical position of a 16-byte piece inside its row (XOR is an involution,
// so the same map converts logical <-> physical).
__device__ __forceinline__ int swz_k(int row, int piece) { return piece ^ (row & 7); }
__device__ __forceinline__ int swz_v(int row, int piece) { return piece ^ ((row & 3) << 1); }

// Direct loads of one K (or V) tile -- key block j -- into an LDS buffer.
// Each wave instruction fills 2 KB of LDS contiguously (lane i -> +16 i,
// the two waves interleaved 1 KB apart); lane i loads the global piece that
// the swizzle places at that slot, so the lanes covering one row read the
// whole 128 (256) byte row.  Per-lane byte offsets are fixed for the whole
// walk; the tile base and the LDS destination are scalars, so a tile costs
// no vector ALU work.
template <int D>
__device__ __forceinline__ void issue_half(const uint16_t* base, int j, const uint32_t (&offs)[Geo<D>::LPT],
                                           uint32_t lds_wave) {
    static_assert(Geo<D>::LPT % 4 == 0, "loads come in groups of four");
    const uint16_t* t = base + (size_t)j * 64 * D;
#pragma unroll
    for (int r = 0; r < Geo<D>::LPT; r += 4) {
        const uint32_t o4[4] = {offs[r], offs[r + 1], offs[r + 2], offs[r + 3]};
        lds_load16x4(o4, t, lds_wave + r * kThreads * 16 + 4096);
    }
}

// One wave's share of a 64 x 128 tile (rows rs bytes apart, t pointing at the
// wave's first row): load r = 0..7 reads rows 8r .. 8r + 3 after t, the lane's
// row and piece given by the byte offset lo, and lands at LDS
// lds + 2048 r + 16 lane.  Two groups of four loads with one M0 setting each;
// every load of a group has its own scalar base, less its instruction offset
// (which also moves the LDS destination), so any row stride works.
__device__ __forceinline__ void issue_rows128(const char* t, uint32_t rs, uint32_t lo, uint32_t lds) {
    const int64_t step = 8 * (int64_t)rs - 2048;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const char* s0 = t + (int64_t)g * 32 * rs + 4096;
        const char* s1 = s0 + step;
        const char* s2 = s1 + step;
        const char* s3 = s2 + step;
        uint32_t saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %3 offset:-4096\n\t"
            "global_load_lds_dwordx4 %1, %4 offset:-2048\n\t"
            "global_load_lds_dwordx4 %1, %5\n\t"
            "global_load_lds_dwordx4 %1, %6 offset:2048\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(lo), "s"(lds + 8192u * g + 4096u), "s"(s0), "s"(s1), "s"(s2), "s"(s3)
            : "memory");
    }
}

// s_waitcnt lgkmcnt(0) with the other counters left alone, after every LDS
// access before it in program order.
__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Row t of (b, h) group bh of the bf16 output O: contiguous [B, H, L, D], or
// at the strides of the attention layer's concatenated heads.
__device__ __forceinline__ uint16_t* o_row(const FwdArgs& a, size_t bh, int t, int D) {
    if (a.strided)
        return (uint16_t*)a.out + (int64_t)(bh / a.H) * a.o_bs + (int64_t)(bh % a.H) * a.o_hs + (int64_t)t * a.o_ts;
    return (uint16_t*)a.out + (bh * a.L + t) * D;
}

__device__ __forceinline__ int tile_j(int e) { return e & kTileJ; }
__device__ __forceinline__ int tile_unit(int e) { return (e >> kTileUnitShift) & (kMaxBinUnits - 1); }
// allowed 32 x 32 sub-blocks of a tile: bit 2a + b, query half a, key half b
__device__ __forceinline__ int tile_sub(int e) { return (e >> kTileSubShift) & 15; }

// Debug builds (BSATTN_DEBUG) check the schedule as the kernels walk it: list
// lengths, unit records and tile entries.  A bad value sets a bit of *a.dbg
// and is replaced by one that stays in bounds, so the walk goes on and the
// host reports the error after the launch.  Release builds compile to nothing.
__device__ __forceinline__ void dbg_lengths(const FwdArgs& a, int& nu, int& nt) {
#ifdef BSATTN_DEBUG
    if (nu > kMaxBinUnits || nt > kMaxBinTiles) {
        atomicOr(a.dbg, 4u);
        nu = min(nu, kMaxBinUnits);
        nt = min(nt, kMaxBinTiles);
    }
#endif
}
__device__ __forceinline__ int4 dbg_unit(const FwdArgs& a, int4 r) {
#ifdef BSATTN_DEBUG
    const bool group_ok = r.z >= 0 && r.z < a.B * a.H;
    const bool row_ok = r.x >= 0 ? r.x < a.nb && r.y >= -1 && r.y < a.n_slots
                                 : (-1 - r.x) < a.n_rt && r.y >= 0 && r.y < a.r_chunks;
    if (!group_ok || !row_ok) {
        atomicOr(a.dbg, 1u);
        r = make_int4(0, -1, 0, r.w);
    }
#endif
    return r;
}
__device__ __forceinline__ int dbg_tile(const FwdArgs& a, int e, int nu, bool gathered) {
#ifdef BSATTN_DEBUG
    const int limit = a.nb + (gathered ? a.n_gt : 0);
    if (tile_j(e) >= limit || ((e >> kTileUnitShift) & 127) >= nu) {
        atomicOr(a.dbg, 2u);
        e &= kTileFirst | kTileLast | (15 << kTileSubShift);
    }
#endif
    return e;
}

// STRIDED: Q, K, V and O at the FwdArgs strides (the attention layer's layout)
template <int D, int MASK, bool STRIDED = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(const FwdArgs a) {
    using Gm = Geo<D>;
    constexpr int NC = Gm::NC, NDB = Gm::NDB, TILE = Gm::TILE;
    // D = 128 walks its list with one K and one V buffer (see below); other
    // widths with a ring of two tiles each.
    constexpr int NBUF = D == 128 ? 1 : 2;
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf[NBUF * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vbuf[NBUF * TILE];
    __shared__ int flat[kMaxBinTiles];
    __shared__ int s_count;
    __shared__ __attribute__((aligned(16))) int gtok_s[MASK == MASK_TOKEN ? kMaxTokGlobal : 4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int rloc = wave * 32 + ql;  // this lane's query row within the tile

    // ---- this workgroup: bin `bin` of XCD x = blockIdx % 8 (workgroups are
    // dealt round-robin to the XCDs).  The bins of an XCD share the units --
    // rows, chunks of split rows, routed tiles -- of the (batch, head) groups
    // that XCD serves, packed so that all bins walk the groups in the same
    // order: the K/V working set of the XCD stays near one group and hits in
    // its L2.  The grid is sized to be resident at once.
    const int x = blockIdx.x % kXcds;
    const int bin = blockIdx.x / kXcds;
    const int bi = x * a.n_bins + bin;
    const int up0 = a.unit_ptr[bi];
    const int tp0 = a.tile_ptr[bi];
    int nu = a.unit_ptr[bi + 1] - up0;   // <= 64
    int nt = a.tile_ptr[bi + 1] - tp0;   // <= kMaxBinTiles
    dbg_lengths(a, nu, nt);
    if (nu <= 0) return;

    // Unit table, lane k describing unit k: kind >= 0 query block of a layout
    // row, kind < 0 routed tile -1-kind; slot -1 writes O/LSE, >= 0 a partial;
    // g its (batch, head) group; valid its batch entry's key length.
    int u_kind = 0, u_slot = -1, u_g = 0, u_valid = a.L;
    if (lane < nu) {
        const int4 r = dbg_unit(a, a.units[up0 + lane]);
        const int ub = r.z / a.H;
        u_kind = r.x;
        u_g = r.z;
        if (r.x >= 0) u_slot = r.y < 0 ? -1 : ub * a.n_slots + r.y;
        else u_slot = a.r_slot_base + (r.z * a.n_rt + (-1 - r.x)) * a.r_chunks + r.y;
        if (MASK == MASK_PAD) u_valid = min(max(a.valid_len[ub], 0), a.L);
    }
    auto rd = [](int v, int k) -> int { return __builtin_amdgcn_readlane(v, k); };
    // row stride of Q, K and V (elements), and a group's first row
    const int64_t RS = STRIDED ? a.qkv_ts : D;
    auto gbase = [&](const void* t, int g) -> const uint16_t* {
        if (STRIDED) return (const uint16_t*)t + (int64_t)(g / a.H) * a.qkv_bs + (int64_t)(g % a.H) * a.qkv_hs;
        return (const uint16_t*)t + (size_t)g * a.L * D;
    };
    // K (V) tile j of group g: a block of the sequence, or (token layouts,
    // j >= nb) a gathered tile of the global tokens' keys
    auto ktile = [&](int g, int j) -> const uint16_t* {
        if (MASK == MASK_TOKEN && j >= a.nb) return a.kg + ((size_t)g * a.n_gt + (j - a.nb)) * TILE;
        return gbase(a.k, g) + (size_t)j * 64 * RS;
    };
    auto vtile = [&](int g, int j) -> const uint16_t* {
        if (MASK == MASK_TOKEN && j >= a.nb) return a.vg + ((size_t)g * a.n_gt + (j - a.nb)) * TILE;
        return gbase(a.v, g) + (size_t)j * 64 * RS;
    };

    // token of this lane's query row in a unit of kind `kind`, group g (-1: unused routed row)
    auto query_token = [&](int kind, int g) -> int {
        if (kind >= 0) return kind * 64 + rloc;
        const int kk = (-1 - kind) * 64 + rloc;
        const int t = kk < a.n_routed ? a.routed_rows[(size_t)g * a.routed_stride + kk] : -1;
        return (t >= a.L) ? -1 : t;          // out-of-range rows are skipped, never dereferenced
    };
    // Q^T fragments of a row (B operand of S^T): lane (ql, hh) holds Q[t][16c + 8hh .. +7].
    auto load_q = [&](int t, int g, bf16x8_t (&qf)[NC]) {
        const uint16_t* qp = gbase(a.q, g);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (t >= 0) u = *(const u32x4_t*)(qp + (size_t)t * RS + 16 * c + 8 * hh);
            qf[c] = as_bf16x8(u);
        }
    };
    // Write a unit's result: O row (bf16) and LSE, or an fp32 partial and its LSE.
    auto store_unit = [&](int slot, int t, int g, int r, const f32x16_t (&ov)[NDB], float inv, float lse_v) {
        if (t < 0) return;
        const size_t bh = (size_t)g;
        // O^T register i of block db <-> d = 32db + 8(i/4) + 4hh + i%4
        if (slot < 0) {
            uint16_t* orow = STRIDED ? o_row(a, bh, t, D) : (uint16_t*)a.out + (bh * a.L + t) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2_t w;
                    w.x = pack_bf16x2(ov[db][4 * gq + 0] * inv, ov[db][4 * gq + 1] * inv);
                    w.y = pack_bf16x2(ov[db][4 * gq + 2] * inv, ov[db][4 * gq + 3] * inv);
                    *(u32x2_t*)(orow + 32 * db + 8 * gq + 4 * hh) = w;
                }
            if (hh == 0) a.lse[bh * a.L + t] = lse_v;
        } else {
            float* orow = a.ws_o + ((size_t)slot * 64 + r) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(float4*)(orow + 32 * db + 8 * gq + 4 * hh) =
                        make_float4(ov[db][4 * gq] * inv, ov[db][4 * gq + 1] * inv, ov[db][4 * gq + 2] * inv,
                                    ov[db][4 * gq + 3] * inv);
            if (hh == 0) a.ws_lse[(size_t)slot * 64 + r] = lse_v;
        }
    };

    // ---- the bin's tile list -> LDS.  With a key-padding mask, tiles that
    // start at or past the valid length are dropped (a unit's blocks ascend, so
    // it keeps a prefix) and a unit left with no tile is written as empty
    // (O = 0, LSE = -inf) right here.
    int F = nt;
    uint64_t empty_units = 0;
    if (MASK == MASK_TOKEN)
        for (int i = tid; i < a.n_gt * 64; i += kThreads) gtok_s[i] = a.gtok[i];
    if (MASK != MASK_PAD) {
        for (int i = tid; i < nt; i += kThreads) flat[i] = dbg_tile(a, a.tiles[tp0 + i], nu, MASK == MASK_TOKEN);
    } else {
        // both waves scan the list (wave 0 writes it) and write their half of empty units
        int kept_total = 0;
        for (int base = 0; base < nt; base += 64) {
            const int i = base + lane;
            const int e = i < nt ? dbg_tile(a, a.tiles[tp0 + i], nu, MASK == MASK_TOKEN) : 0;
            const int en = i + 1 < nt ? dbg_tile(a, a.tiles[tp0 + i + 1], nu, MASK == MASK_TOKEN) : 0;
            const int valid = __shfl(u_valid, tile_unit(e));   // the tile's unit's key length
            const bool keep = i < nt && tile_j(e) * 64 < valid;
            const bool keep_next = i + 1 < nt && !(e & kTileLast) && tile_j(en) * 64 < valid;
            const uint64_t km = __ballot(keep);
            const int pos = kept_total + __builtin_popcountll(km & ((1ull << lane) - 1ull));
            if (wave == 0 && keep) flat[pos] = keep_next ? (e & ~kTileLast) : (e | kTileLast);
            const uint64_t em = __ballot(i < nt && (e & kTileFirst) && !keep);
            for (uint64_t mm = em; mm; mm &= mm - 1) empty_units |= 1ull << tile_unit(rd(e, __builtin_ctzll(mm)));
            kept_total += __builtin_popcountll(km);
        }
        F = kept_total;
        const f32x16_t zero[NDB] = {};
        for (uint64_t mm = empty_units; mm; mm &= mm - 1) {
            const int u = __builtin_ctzll(mm);
            const int g = rd(u_g, u);
            store_unit(rd(u_slot, u), query_token(rd(u_kind, u), g), g, rloc, zero, 0.f, -INFINITY);
        }
    }
    __syncthreads();
    if (F == 0) return;
    // units with at least one tile (those without were written above)
    const uint64_t live_units = (nu >= 64 ? ~0ull : ((1ull << nu) - 1ull)) & ~empty_units;

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
    // Direct-load byte offsets of this thread's pieces, and the wave's LDS
    // destinations in each ring buffer.
    uint32_t koffs[Gm::LPT], voffs[Gm::LPT];
#pragma unroll
    for (int r = 0; r < Gm::LPT; ++r) {
        const int sl = r * kThreads + tid;
        const int row = sl / Gm::PIECES, q = sl % Gm::PIECES;
        // minus the instruction offset 2048 (r % 4) - 4096 that the load adds
        koffs[r] = (uint32_t)(row * RS + swz_k(row, q) * 8) * 2u + 4096u - 2048u * (r % 4);
        voffs[r] = (uint32_t)(row * RS + swz_v(row, q) * 8) * 2u + 4096u - 2048u * (r % 4);
    }
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(wave * 64 * 16);
    const uint32_t kl0 = lds_addr(kbuf) + wave_lds, vl0 = lds_addr(vbuf) + wave_lds;

    const float c2 = a.scale_log2;
    f32x16_t o[NDB];
    float m = -INFINITY;   // running (lazily raised) max of scaled scores, log2 units
    float l = 0.f;         // sum of this lane's probabilities
    auto reset = [&]() {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        m = -INFINITY;
        l = 0.f;
    };

    // K fragments of the tile at Ks (A operand of S^T = K Q^T).
    auto kread = [&](const uint16_t* Ks, bf16x8_t (&kf)[2][NC]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c) kf[kb][c] = as_bf16x8(*(const u32x4_t*)(Ks + koff[kb][c]));
    };
    // S^T = K Q^T: s[kb] register i <-> key 32kb + 8(i/4) + 4hh + i%4.
    auto smma = [&](const bf16x8_t (&kf)[2][NC], const bf16x8_t (&q)[NC], f32x16_t (&s)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][c], q[c], s[kb], 0, 0, 0);
    };
    // V^T fragments of the tile at Vs (A operand of O^T = V^T P^T).
    auto vread = [&](const uint16_t* Vs, bf16x8_t (&va)[4][NDB]) {
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
    };
    // Row max of a tile's scores in log2 units (pair of lanes = one query row).
    auto tile_max = [&](const f32x16_t (&s)[2]) -> float {
        float mx = __builtin_fmaxf(__builtin_fmaxf(s[0][0], s[0][1]), s[1][0]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[0][i]), s[0][i + 1]);
#pragma unroll
        for (int i = 1; i < 15; i += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[1][i]), s[1][i + 1]);
        mx = __builtin_fmaxf(mx, s[1][15]);
        return pair_max(mx) * c2;
    };
    // Online softmax, first half: mask the tile's scores (key block j); on the
    // first tile of a unit take the running max from the tile itself.  Later
    // tiles keep the running max m as it is: the max is raised only when a
    // tile's probabilities grow too large (see softmax_pv), which on typical
    // rows happens rarely -- so no per-tile max is computed.
    // MASK_BITS: kept-key words of this lane's query for tiles f, f + 1, f + 2
    // (loaded two steps ahead, so the step's own memory wait covers them)
    uint64_t wbits_cur = 0, wbits_n1 = 0, wbits_n2 = 0;
    auto load_bits = [&](int e) -> uint64_t {
        const int u = tile_unit(e);
        const int g = rd(u_g, u);
        const int t = rd(u_kind, u) * 64 + rloc;
        return a.keep_bits[((size_t)g * a.L + t) * a.nb + tile_j(e)];
    };
    auto softmax_prep = [&](int e, int kind, int tq, int valid, f32x16_t (&s)[2], bool first) {
        const int j = tile_j(e);
        if (MASK == MASK_SUB) {
            // 32-token blocks: this wave holds query half `wave` of the tile
            const int sub = tile_sub(e);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (!((sub >> (2 * wave + kb)) & 1))
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kb][i] = -INFINITY;
        }
        if (MASK == MASK_PAD) {
            if (j * 64 + 64 > valid) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4) >= valid) s[kb][i] = -INFINITY;
            }
        }
        if (MASK == MASK_BAND || MASK == MASK_TOKEN) {
            // a tile whose farthest (query, key) pair is inside the band needs no mask
            if (kind >= 0 && j < a.nb && 64 * abs(kind - j) + 63 > a.band) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (abs(tq - (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4))) > a.band)
                            s[kb][i] = -INFINITY;
            }
        }
        if (MASK == MASK_TOKEN && kind >= 0 && j >= a.nb) {
            // gathered global keys: padding (-1) and keys the band already covers drop out
            const int* gt = gtok_s + (j - a.nb) * 64;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int4 gv = *(const int4*)(gt + 32 * kb + 8 * g4 + 4 * hh);
                    const int gs[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gs[e] < 0 || abs(tq - gs[e]) <= a.band) s[kb][4 * g4 + e] = -INFINITY;
                }
        }
        if (MASK == MASK_BITS) {
            // this lane's query keeps key 32 kb + 8 (i / 4) + 4 hh + i % 4 iff its bit is set
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint32_t w = kb == 0 ? (uint32_t)wbits_cur : (uint32_t)(wbits_cur >> 32);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((w >> (8 * (i / 4) + 4 * hh + (i % 4))) & 1u)) s[kb][i] = -INFINITY;
            }
        }
        if (first) m = tile_max(s);   // o = 0 and l = 0 here
    };
    // Online softmax, second half, for the key chunks c0, c0 + 1 (16 keys each):
    // P = exp2(s * c2 - m) as the bf16 B operand of the PV product (pf[c]
    // element e <-> key 16c + 8(e/4) + 4hh + e%4), row sums in fp32.  If the
    // chunks' probabilities sum past kSumCap in some lane (or a row whose max
    // is still -inf meets a finite score), the running max is raised to the
    // tile's max, O and l are rescaled -- they hold only contributions made
    // with the old max -- and the chunks are redone.  So every probability
    // stays below kSumCap and nothing overflows.
    auto softmax_exp = [&](const f32x16_t (&s)[2], auto c0, u32x4_t (&u)[2]) {
        constexpr int C0 = decltype(c0)::value;
        float lsum;
        auto chunks = [&]() {
            const float muse = m == -INFINITY ? 0.f : m;
            float acc[8];
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = C0 + k;
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[c / 2][8 * (c % 2) + 2 * e], c2, -muse));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[c / 2][8 * (c % 2) + 2 * e + 1], c2, -muse));
                    u[k][e] = pack_bf16x2(p0, p1);
                    acc[4 * k + e] = p0 + p1;
                }
            lsum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
        };
        chunks();
        const bool bad = lsum > kSumCap || (m == -INFINITY && lsum > 0.f);
        if (__ballot(bad) != 0) {          // wave-uniform, rare
            const float mx = tile_max(s);
            const bool raise = mx > m;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.f;   // 0 when m was -inf
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            m = raise ? mx : m;
            chunks();
        }
        l += lsum;
    };
    // O^T += V^T P^T for the key chunks c0, c0 + 1.
    auto pv = [&](const bf16x8_t (&va)[4][NDB], auto c0, const u32x4_t (&u)[2]) {
        constexpr int C0 = decltype(c0)::value;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[C0 + k][db], as_bf16x8(u[k]), o[db], 0, 0, 0);
    };

    if constexpr (D == 128) {
        // ---- one K and one V buffer, two waves per SIMD ----
        // At D = 128 a tile is 32 KB (K and V); with one buffer of each the
        // workgroup holds 34 KB of LDS and at most 256 registers per wave, so
        // four workgroups fit a CU and every SIMD runs two waves, which cover
        // each other's waits.  Step f: wait for this wave's loads of tile f,
        // then a barrier (the other wave's half has landed); read all K
        // fragments, issue the score MFMAs, read all V fragments (into the
        // registers the K fragments leave); a second barrier (both waves hold
        // their fragments), after which the loads of tile f + 1 go into the
        // same buffers while the softmax and the PV product of tile f run.  On
        // a unit's last tile Q is free once the score MFMAs are issued, and
        // the next unit's Q is loaded into the same registers.
        auto tile_g = [&](int e) -> int { return rd(u_g, tile_unit(e)); };
        const int wrow = __builtin_amdgcn_readfirstlane(4 * wave);   // the wave's rows 8r + wrow .. +3
        const int lr = lane >> 4;
        const uint32_t lo_k = (uint32_t)((lr * RS + swz_k(wrow + lr, lane & 15) * 8) * 2);
        const uint32_t lo_v = (uint32_t)((lr * RS + swz_v(wrow + lr, lane & 15) * 8) * 2);
        const uint32_t rsb = (uint32_t)(RS * 2);
        const uint32_t kl = lds_addr(kbuf) + 256u * wrow, vl = lds_addr(vbuf) + 256u * wrow;
        auto issue_tile = [&](const uint16_t* t, uint32_t lo, uint32_t lds) {
            issue_rows128((const char*)(t + (int64_t)wrow * RS), rsb, lo, lds);
        };
        // Fragment offsets as a few base registers plus constants (instruction
        // offsets): K chunk c >= 4 sits 64 elements after chunk c - 4 of the
        // same row (the swizzle permutes pieces within groups of eight), and
        // V column block db >= 2 sits 64 elements after db - 2.
        int kb0[4], vb0[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) kb0[c] = ql * D + swz_k(ql, 2 * c + hh) * 8;
#pragma unroll
        for (int d1 = 0; d1 < 2; ++d1) {
            const int row = 4 * hh + (gi >> 2);
            const int d0 = 32 * d1 + 16 * gsel + 4 * (gi & 3);
            vb0[d1] = row * D + swz_v(row, d0 >> 3) * 8 + (d0 & 7);
        }
        auto kread1 = [&](bf16x8_t (&kf)[2][NC]) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    kf[kb][c] = as_bf16x8(*(const u32x4_t*)(kbuf + kb0[c & 3] + (c >> 2) * 64 + kb * 32 * D));
        };
        auto vread1 = [&](bf16x8_t (&va)[4][NDB]) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint16_t* p = vbuf + vb0[db & 1] + (db >> 1) * 64 + 16 * c * D;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p + 8 * D));
                    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                    const u32x4_t lh = {l2.x, l2.y, h2.x, h2.y};
                    va[c][db] = as_bf16x8(lh);
                }
        };

        int e0 = flat[0];
        int u_cur = tile_unit(e0);
        int kind_cur = rd(u_kind, u_cur), slot_cur = rd(u_slot, u_cur), g_cur = rd(u_g, u_cur);
        int valid_cur = rd(u_valid, u_cur);
        int tq_cur = query_token(kind_cur, g_cur);
        bf16x8_t qf[NC];
        load_q(tq_cur, g_cur, qf);
        if (MASK == MASK_BITS) wbits_cur = load_bits(e0);
        issue_tile(ktile(g_cur, tile_j(e0)), lo_k, kl);
        issue_tile(vtile(g_cur, tile_j(e0)), lo_v, vl);
        reset();
        using C0 = std::integral_constant<int, 0>;
        using C2 = std::integral_constant<int, 2>;
        for (int f = 0; f < F; ++f) {
            const int e1 = f + 1 < F ? flat[f + 1] : 0;
            wait_vmcnt<0>();   // this wave's loads of tile f (and Q, mask bits)
            stage_barrier();   // the other wave's
            f32x16_t s[2];
            {
                bf16x8_t kf[2][NC];
                kread1(kf);
                smma(kf, qf, s);
            }
            bf16x8_t va[4][NDB];
            vread1(va);
            wait_lgkm0();      // this wave's fragment reads are done,
            stage_barrier();   // and the other wave's: the buffers take tile f + 1
            if (f + 1 < F) {
                const int g1 = tile_g(e1), j1 = tile_j(e1);
                issue_tile(ktile(g1, j1), lo_k, kl);
                issue_tile(vtile(g1, j1), lo_v, vl);
                if (MASK == MASK_BITS) wbits_n1 = load_bits(e1);
            }
            const bool last = (e0 & kTileLast) != 0;
            int u_n = u_cur, kind_n = kind_cur, slot_n = slot_cur, g_n = g_cur, valid_n = valid_cur, tq_n = tq_cur;
            if (last) {
                const uint64_t rest = u_cur >= 63 ? 0ull : (live_units & ~((2ull << u_cur) - 1ull));
                if (rest != 0) {
                    u_n = __builtin_ctzll(rest);
                    kind_n = rd(u_kind, u_n);
                    slot_n = rd(u_slot, u_n);
                    g_n = rd(u_g, u_n);
                    valid_n = rd(u_valid, u_n);
                    tq_n = query_token(kind_n, g_n);
                    load_q(tq_n, g_n, qf);   // the score MFMAs above have taken Q
                }
            }
            softmax_prep(e0, kind_cur, tq_cur, valid_cur, s, (e0 & kTileFirst) != 0);
            u32x4_t pA[2], pB[2];
            softmax_exp(s, C0(), pA);
            pv(va, C0(), pA);
            softmax_exp(s, C2(), pB);
            pv(va, C2(), pB);
            if (last) {
                // ---- unit done: O = acc / l, LSE = (m + log2 l) ln 2 ----
                const float lt = pair_sum(l);
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
                store_unit(slot_cur, tq_cur, g_cur, rloc, o, inv, lse_v);
                reset();
                u_cur = u_n;
                kind_cur = kind_n;
                slot_cur = slot_n;
                tq_cur = tq_n;
                g_cur = g_n;
                valid_cur = valid_n;
            }
            if (MASK == MASK_BITS) wbits_cur = wbits_n1;
            e0 = e1;
        }
    } else {
        // ---- software pipeline over the flat tile list ----
        // Tile f's K sits in K buffer f & 1 and its V in V buffer f & 1.  Step f
        // computes the scores of tile f + 1 (MFMA) while it runs the softmax of
        // tile f (VALU), then accumulates tile f's PV product.  During step f the
        // direct loads of K(f + 2) and V(f + 1) are in flight, into the buffers
        // whose last readers (step f - 1) are behind the step's barrier.  A unit's
        // Q is loaded during the first step of the unit before it, so a unit
        // boundary costs no load latency.
        int e0 = flat[0];
        int e1 = F > 1 ? flat[1] : 0;
        int e2 = F > 2 ? flat[2] : 0;
        // group of a flat tile entry's unit
        auto tile_g = [&](int e) -> int { return rd(u_g, tile_unit(e)); };
        int u_cur = tile_unit(e0);
        int kind_cur = rd(u_kind, u_cur), slot_cur = rd(u_slot, u_cur), g_cur = rd(u_g, u_cur);
        int valid_cur = rd(u_valid, u_cur);
        int tq_cur = query_token(kind_cur, g_cur);
        int kind_n = 0, slot_n = -1, tq_n = -1, u_n = 0, g_n = 0, valid_n = a.L;
        bf16x8_t qf[NC], qf_n[NC];
        load_q(tq_cur, g_cur, qf);
    #pragma unroll
        for (int c = 0; c < NC; ++c) qf_n[c] = qf[c];
        if (MASK == MASK_BITS) {
            wbits_cur = load_bits(e0);
            if (F > 1) wbits_n1 = load_bits(e1);
        }

        wait_vmcnt<0>();
        issue_half<D>(ktile(g_cur, tile_j(e0)), 0, koffs, kl0);
        issue_half<D>(vtile(g_cur, tile_j(e0)), 0, voffs, vl0);
        if (F > 1) {
            issue_half<D>(ktile(tile_g(e1), tile_j(e1)), 0, koffs, kl0 + TILE * 2);
            wait_vmcnt<2 * Gm::LPT>();   // K(0) landed; V(0) and K(1) may still fly
        } else {
            wait_vmcnt<Gm::LPT>();
        }
        stage_barrier();
        f32x16_t s_cur[2], s_nxt[2];
        {
            bf16x8_t kf[2][NC];
            kread(kbuf, kf);
            smma(kf, qf, s_cur);
        }
        reset();


        // One step, written for a compile-time parity P = f & 1 so that the ring
        // buffers' addresses fold into instruction offsets; the loop runs steps in
        // pairs, swapping the roles of the two score register sets.  The running
        // max of tile f is taken before the step's wait: it needs only registers,
        // and it covers the latency of the previous step's output stores.
        auto step = [&](auto parity, int f, f32x16_t (&s_now)[2], f32x16_t (&s_next)[2]) {
            constexpr int P = decltype(parity)::value;
            softmax_prep(e0, kind_cur, tq_cur, valid_cur, s_now, (e0 & kTileFirst) != 0);
            wait_vmcnt<0>();
            stage_barrier();
            if (MASK == MASK_BITS && f + 2 < F) wbits_n2 = load_bits(e2);
            // Q of the next unit: loaded during the first step of the current unit
            // and, when the current unit ends here, moved in place for the scores
            // of tile f + 1 -- before this step's direct loads are issued, so that
            // any wait the compiler places for the Q loads cannot also wait for
            // the direct loads in flight.
            if (e0 & kTileFirst) {
                const uint64_t rest = u_cur >= 63 ? 0ull : (live_units & ~((2ull << u_cur) - 1ull));
                if (rest != 0) {
                    u_n = __builtin_ctzll(rest);
                    kind_n = rd(u_kind, u_n);
                    slot_n = rd(u_slot, u_n);
                    g_n = rd(u_g, u_n);
                    valid_n = rd(u_valid, u_n);
                    tq_n = query_token(kind_n, g_n);
                    load_q(tq_n, g_n, qf_n);
                }
            }
            if (e0 & kTileLast) {
    #pragma unroll
                for (int c = 0; c < NC; ++c) qf[c] = qf_n[c];
            }
    #pragma unroll
            for (int c = 0; c < NC; ++c) asm volatile("" ::"v"(qf[c]));   // materialise qf here
            const int e3 = f + 3 < F ? flat[f + 3] : 0;
            // Fragment reads first; the direct loads of K(f + 2) and V(f + 1) are
            // spread over the step (a burst of them right after the barrier makes
            // every wave queue at the texture unit with nothing else to issue).
            bf16x8_t kf[2][NC], va[4][NDB];
            kread(kbuf + (1 - P) * TILE, kf);
            vread(vbuf + P * TILE, va);
            if (f + 2 < F) issue_half<D>(ktile(tile_g(e2), tile_j(e2)), 0, koffs, kl0 + P * TILE * 2);
            // Scores of tile f + 1 (past the end they read a stale buffer and are
            // discarded), interleaved by the scheduler with the softmax of tile f.
            using C0 = std::integral_constant<int, 0>;
            using C2 = std::integral_constant<int, 2>;
            u32x4_t pA[2], pB[2];
            smma(kf, qf, s_next);
            softmax_exp(s_now, C0(), pA);
            __builtin_amdgcn_sched_group_barrier(0x100, 8 + 8 * NDB, 0);   // LDS reads first
    #pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // then one MFMA
            }
            if (f + 1 < F) issue_half<D>(vtile(tile_g(e1), tile_j(e1)), 0, voffs, vl0 + (1 - P) * TILE * 2);
            pv(va, C0(), pA);
            softmax_exp(s_now, C2(), pB);
    #pragma unroll
            for (int i = 0; i < 2 * NDB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // then eight VALU
            }
            pv(va, C2(), pB);
            if (e0 & kTileLast) {
                // ---- unit done: O = acc / l, LSE = (m + log2 l) ln 2 ----
                const float lt = pair_sum(l);
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
                store_unit(slot_cur, tq_cur, g_cur, rloc, o, inv, lse_v);
                reset();
                u_cur = u_n;
                kind_cur = kind_n;
                slot_cur = slot_n;
                tq_cur = tq_n;
                g_cur = g_n;
                valid_cur = valid_n;
            }
            e0 = e1;
            e1 = e2;
            e2 = e3;
            if (MASK == MASK_BITS) {
                wbits_cur = wbits_n1;
                wbits_n1 = wbits_n2;
            }
        };
        for (int f = 0; f < F; f += 2) {
            step(std::integral_constant<int, 0>(), f, s_cur, s_nxt);
            if (f + 1 < F) step(std::integral_constant<int, 1>(), f + 1, s_nxt, s_cur);
        }
    }
}

// ---------------------------------------------------------------------------
// D = 64: one workgroup of eight waves per CU, two waves per SIMD.  A wave owns
// a whole 64-row query tile, so each K and V fragment it reads from LDS feeds
// both 32-row halves, and it walks its own list of tiles with no barrier:
// every wave has its own single K and V buffer (16 KB).  Within a step the
// wave reads the tile's fragments first; the loads of its next tile then go
// into the same buffers while it runs the softmax and the PV products.
//
// A step works on the four 32 x 32 score blocks (key half, query half) in
// turn: the scores of the first block are issued alone, and each later
// scheduling region pairs the softmax of one block (VALU) with matrix
// products that do not depend on it -- the scores of later blocks, the PV
// product of earlier ones -- interleaved by group barriers.  The running max
// of a unit starts at its first block's max; the lazy raise (as in the
// two-wave kernel) works per block.
//
// The two waves that share a SIMD get lists of equal length, and they keep
// pace with each other: the SIMD's issue arbiter favours the older wave, so
// left alone the younger one would fall behind and finish long after it,
// running by itself with nothing to hide its latencies.  Each wave posts the
// tiles it has left in LDS and, while it has more left than its partner,
// raises its issue priority.
constexpr int kQThreads = 64 * kQWaves;

// Four direct loads of one wave, 1 KB apart: load r lands at m0v + 1024 r - 2048 + 16 lane.
__device__ __forceinline__ void lds_load16x4_1k(uint32_t voff, const void* sbase, uint32_t m0v) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:-2048\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:-1024\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(m0v), "s"(sbase)
        : "memory");
}

// A whole 64x64 bf16 tile (8 KB) by one wave: 8 loads of 1 KB, rows in order,
// in two groups of four (rows 0..31, 32..63).  voff is the lane's byte offset
// within a group (rows 0..7) plus 2 KB; one register serves both groups.
__device__ __forceinline__ void issue_tile1(const uint16_t* base, int j, uint32_t voff, uint32_t lds) {
    const uint16_t* t = base + (size_t)j * 64 * 64;
    lds_load16x4_1k(voff, t, lds + 2048);
    lds_load16x4_1k(voff, t + 32 * 64, lds + 4096 + 2048);
}

// As lds_load16x4_1k, for rows `rs` bytes apart: load r reads rows 8 r .. 8 r + 7
// from its own scalar base (sbase + r (8 rs - 1 KB), so that the instruction
// offset, which also places the LDS destination, cancels out).
__device__ __forceinline__ void lds_load16x4_rows(uint32_t voff, const char* sbase, uint32_t rs, uint32_t m0v) {
    const uint32_t step = 8u * rs - 1024u;
    const char* s1 = sbase + step;
    const char* s2 = s1 + step;
    const char* s3 = s2 + step;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:-2048\n\t"
        "global_load_lds_dwordx4 %1, %4 offset:-1024\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "global_load_lds_dwordx4 %1, %6 offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(m0v), "s"(sbase), "s"(s1), "s"(s2), "s"(s3)
        : "memory");
}

// The 64x64 tile starting at `t`, rows rs bytes apart (the layer's strided
// layout): voff is the lane's offset within rows 0..7 plus 2 KB.
__device__ __forceinline__ void issue_tile_rows(const uint16_t* t, uint32_t rs, uint32_t voff, uint32_t lds) {
    lds_load16x4_rows(voff, (const char*)t, rs, lds + 2048);
    lds_load16x4_rows(voff, (const char*)t + 32u * rs, rs, lds + 4096 + 2048);
}

// STRIDED: Q, K, V and O at the FwdArgs strides (the attention layer's layout)
template <int MASK, bool STRIDED = false>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_d64_kernel(const FwdArgs a) {
    constexpr int D = 64, NC = 4, NDB = 2, TILE = 64 * 64;
    __shared__ __attribute__((aligned(1024))) uint16_t kvbuf[kQWaves][2][TILE];
    __shared__ int flats[kQWaves][kMaxBinTiles];   // each wave's tile list
    __shared__ int simd_of[kQWaves];
    __shared__ int left[kQWaves];                  // tiles each wave has not finished
    __shared__ __attribute__((aligned(16))) int gtok_s[MASK == MASK_TOKEN ? kMaxTokGlobal : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
    const int ql = lane & 31;
    const int hh = lane >> 5;

    // Which waves share a SIMD (HW_ID bits 5:4).  With two waves on every
    // SIMD, the waves of SIMD s run lists 2s and 2s + 1 and pace each other;
    // otherwise wave w runs list w on its own.
    const int my_simd = (__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3;
    if (lane == 0) {
        simd_of[wv] = my_simd;
        left[wv] = 0;
    }
    if (MASK == MASK_TOKEN)
        for (int i = tid; i < a.n_gt * 64; i += kQThreads) gtok_s[i] = a.gtok[i];
    __syncthreads();
    int rank = 0, partner = -1;
    bool paired = true;
    for (int s2 = 0; s2 < 4; ++s2) {
        int n_on = 0;
        for (int w = 0; w < kQWaves; ++w) n_on += simd_of[w] == s2;
        paired = paired && n_on == 2;
    }
    for (int w = 0; w < kQWaves; ++w)
        if (w != wv && simd_of[w] == my_simd) {
            partner = w;
            rank += w < wv;
        }
    const int list = paired ? 2 * my_simd + rank : wv;
    if (!paired) partner = -1;
    int* const flat = flats[wv];

    const int x = blockIdx.x % kXcds;
    const int bin = blockIdx.x / kXcds + list * (a.n_bins / kQWaves);
    const int bi = x * a.n_bins + bin;
    const int up0 = a.unit_ptr[bi];
    const int tp0 = a.tile_ptr[bi];
    int nu = a.unit_ptr[bi + 1] - up0;   // <= kMaxBinUnits
    int nt = a.tile_ptr[bi + 1] - tp0;   // <= kMaxBinTiles
    dbg_lengths(a, nu, nt);
    if (nu <= 0) return;

    int u_kind = 0, u_slot = -1, u_g = 0, u_valid = a.L;
    if (lane < nu) {
        const int4 r = dbg_unit(a, a.units[up0 + lane]);
        const int ub = r.z / a.H;
        u_kind = r.x;
        u_g = r.z;
        if (r.x >= 0) u_slot = r.y < 0 ? -1 : ub * a.n_slots + r.y;
        else u_slot = a.r_slot_base + (r.z * a.n_rt + (-1 - r.x)) * a.r_chunks + r.y;
        if (MASK == MASK_PAD) u_valid = min(max(a.valid_len[ub], 0), a.L);
    }
    auto rd = [](int v, int k) -> int { return __builtin_amdgcn_readlane(v, k); };
    // row stride of Q, K and V (elements), and a group's first row
    const int64_t RS = STRIDED ? a.qkv_ts : D;
    auto gbase = [&](const void* t, int g) -> const uint16_t* {
        if (STRIDED) return (const uint16_t*)t + (int64_t)(g / a.H) * a.qkv_bs + (int64_t)(g % a.H) * a.qkv_hs;
        return (const uint16_t*)t + (size_t)g * a.L * D;
    };
    // K (V) tile j of group g: a block of the sequence, or (token layouts,
    // j >= nb) a gathered tile of the global tokens' keys
    auto ktile = [&](int g, int j) -> const uint16_t* {
        if (MASK == MASK_TOKEN && j >= a.nb) return a.kg + ((size_t)g * a.n_gt + (j - a.nb)) * TILE;
        return gbase(a.k, g) + (size_t)j * 64 * RS;
    };
    auto vtile = [&](int g, int j) -> const uint16_t* {
        if (MASK == MASK_TOKEN && j >= a.nb) return a.vg + ((size_t)g * a.n_gt + (j - a.nb)) * TILE;
        return gbase(a.v, g) + (size_t)j * 64 * RS;
    };
    // token of query row r (0..63) of a unit (-1: unused routed row)
    auto query_token = [&](int kind, int g, int r) -> int {
        if (kind >= 0) return kind * 64 + r;
        const int kk = (-1 - kind) * 64 + r;
        const int t = kk < a.n_routed ? a.routed_rows[(size_t)g * a.routed_stride + kk] : -1;
        return (t >= a.L) ? -1 : t;
    };
    // Q^T fragments of both halves: qf[qb][c] holds Q[row 32qb + ql][16c + 8hh .. +7].
    auto load_q = [&](int kind, int g, bf16x8_t (&qf)[2][NC], int (&tq)[2]) {
        const uint16_t* qp = gbase(a.q, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            tq[qb] = query_token(kind, g, 32 * qb + ql);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                u32x4_t u = {0u, 0u, 0u, 0u};
                if (tq[qb] >= 0) u = *(const u32x4_t*)(qp + (uint32_t)(tq[qb] * RS + 16 * c + 8 * hh));
                qf[qb][c] = as_bf16x8(u);
            }
        }
    };
    auto store_half = [&](int slot, int t, int g, int r, const f32x16_t (&ov)[NDB], float inv, float lse_v) {
        if (t < 0) return;
        const size_t bh = (size_t)g;
        // O^T register i of block db <-> d = 32db + 8(i/4) + 4hh + i%4
        // group / slot bases are uniform (scalar), the lane offsets 32-bit
        if (slot < 0) {
            uint16_t* orow = STRIDED ? o_row(a, bh, t, D) : (uint16_t*)a.out + bh * a.L * D + (uint32_t)(t * D);
            // Lanes l and l + 32 hold d = 8gq + 0..3 and 8gq + 4..7 of the same
            // row: swapping halves (v_permlane32_swap moves the upper half-wave's
            // first operand to the lower half-wave's second, and back) leaves
            // each lane 8 consecutive d, 16 bytes: even gq in the lower
            // half-wave, odd gq in the upper.
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int ge = 2 * pr, go = 2 * pr + 1;
                    const uint32_t e0 = pack_bf16x2(ov[db][4 * ge + 0] * inv, ov[db][4 * ge + 1] * inv);
                    const uint32_t e1 = pack_bf16x2(ov[db][4 * ge + 2] * inv, ov[db][4 * ge + 3] * inv);
                    const uint32_t o0 = pack_bf16x2(ov[db][4 * go + 0] * inv, ov[db][4 * go + 1] * inv);
                    const uint32_t o1 = pack_bf16x2(ov[db][4 * go + 2] * inv, ov[db][4 * go + 3] * inv);
                    const auto s0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
                    const u32x4_t w4 = {s0[0], s1[0], s0[1], s1[1]};
                    *(u32x4_t*)(orow + 32 * db + 16 * pr + 8 * hh) = w4;
                }
            if (hh == 0) (a.lse + bh * a.L)[(uint32_t)t] = lse_v;
        } else {
            uint32_t roff = (uint32_t)(r * D);
            asm volatile("" : "+v"(roff));   // keep the lane offset 32-bit and local (no 64-bit address held across the loop)
            float* orow = a.ws_o + (size_t)slot * 64 * D + roff;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *(float4*)(orow + 32 * db + 8 * gq + 4 * hh) =
                        make_float4(ov[db][4 * gq] * inv, ov[db][4 * gq + 1] * inv, ov[db][4 * gq + 2] * inv,
                                    ov[db][4 * gq + 3] * inv);
            if (hh == 0) (a.ws_lse + (size_t)slot * 64)[(uint32_t)r] = lse_v;
        }
    };
    // ---- tile list -> LDS (key padding: drop tiles past the valid length) ----
    int F = nt;
    uint64_t empty_units = 0;
    if (MASK != MASK_PAD) {
        for (int i = lane; i < nt; i += 64) flat[i] = dbg_tile(a, a.tiles[tp0 + i], nu, MASK == MASK_TOKEN);
    } else {
        int kept_total = 0;
        for (int base = 0; base < nt; base += 64) {
            const int i = base + lane;
            const int e = i < nt ? dbg_tile(a, a.tiles[tp0 + i], nu, MASK == MASK_TOKEN) : 0;
            const int en = i + 1 < nt ? dbg_tile(a, a.tiles[tp0 + i + 1], nu, MASK == MASK_TOKEN) : 0;
            const int valid = __shfl(u_valid, tile_unit(e));
            const bool keep = i < nt && tile_j(e) * 64 < valid;
            const bool keep_next = i + 1 < nt && !(e & kTileLast) && tile_j(en) * 64 < valid;
            const uint64_t km = __ballot(keep);
            const int pos = kept_total + __builtin_popcountll(km & ((1ull << lane) - 1ull));
            if (keep) flat[pos] = keep_next ? (e & ~kTileLast) : (e | kTileLast);
            const uint64_t em = __ballot(i < nt && (e & kTileFirst) && !keep);
            for (uint64_t mm = em; mm; mm &= mm - 1) empty_units |= 1ull << tile_unit(rd(e, __builtin_ctzll(mm)));
            kept_total += __builtin_popcountll(km);
        }
        F = kept_total;
        const f32x16_t zero[NDB] = {};
        for (uint64_t mm = empty_units; mm; mm &= mm - 1) {
            const int u = __builtin_ctzll(mm);
            const int g = rd(u_g, u), kind = rd(u_kind, u), slot = rd(u_slot, u);
            for (int qb = 0; qb < 2; ++qb)
                store_half(slot, query_token(kind, g, 32 * qb + ql), g, 32 * qb + ql, zero, 0.f, -INFINITY);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the list is in LDS
    if (F == 0) return;

    // Fragment read offsets (elements), as in the two-wave kernel.  The
    // swizzles depend on the row only through row & 7 (K) and row & 3 (V), so
    // rows 32 apart (K) and 8 apart (V) share a lane offset and differ by a
    // constant that goes into the read instruction.
    int koff[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) koff[c] = ql * D + swz_k(ql, 2 * c + hh) * 8;
    const int gi = lane & 15, gsel = (lane >> 4) & 1;
    int voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int row = 4 * hh + (gi >> 2);
        const int d0 = 32 * db + 16 * gsel + 4 * (gi & 3);
        voff[db] = row * D + swz_v(row, d0 >> 3) * 8 + (d0 & 7);
    }
    // Direct-load offsets: load r covers rows 8r .. 8r + 7, lane -> row 8r + lane/8,
    // piece lane%8; the swizzle depends on the row only through lane/8.
    uint32_t kdo, vdo;
    {
        const int row0 = lane >> 3, q = lane & 7;
        kdo = (uint32_t)(row0 * RS + swz_k(row0, q) * 8) * 2u + 2048u;
        vdo = (uint32_t)(row0 * RS + swz_v(row0, q) * 8) * 2u + 2048u;
    }
    const uint16_t* kbuf = kvbuf[wv][0];
    const uint16_t* vbuf = kvbuf[wv][1];
    const uint32_t kl = lds_addr(kbuf), vl = lds_addr(vbuf);

    auto kread = [&](const uint16_t* Ks, bf16x8_t (&kf)[2][NC]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c) kf[kb][c] = as_bf16x8(*(const u32x4_t*)(Ks + koff[c] + 32 * kb * D));
    };
    // V^T fragments (A operand of O^T = V^T P^T), transposed on read.
    auto vread = [&](const uint16_t* Vs, bf16x8_t (&va)[4][NDB]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(Vs + voff[db] + 16 * c * D));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(Vs + voff[db] + (16 * c + 8) * D));
                const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
                const u32x4_t lh = {l2.x, l2.y, h2.x, h2.y};
                va[c][db] = as_bf16x8(lh);
            }
    };

    const float c2 = a.scale_log2;
    f32x16_t o[NDB][2];
    float m[2], l[2];
    auto reset = [&]() {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.f;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            m[qb] = kNoMax;
            l[qb] = 0.f;
        }
    };
    // max (log2 units) of one 32 x 32 score block over the lane's 16 keys and
    // its partner lane's (the same query)
    auto blk_max = [&](const f32x16_t& s) -> float {
        float v = __builtin_fmaxf(s[0], s[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) v = __builtin_fmaxf(__builtin_fmaxf(v, s[i]), s[i + 1]);
        return pair_max(v) * c2;
    };
    // the same maximum taken in the opposite order, for the rare rescale: the
    // compiler then shares no partial maxima between the two and keeps none of
    // them on the common path
    auto blk_max_rev = [&](const f32x16_t& s) -> float {
        float v = __builtin_fmaxf(s[15], s[14]);
#pragma unroll
        for (int i = 13; i > 0; i -= 2) v = __builtin_fmaxf(__builtin_fmaxf(v, s[i]), s[i - 1]);
        return pair_max(v) * c2;
    };
    // masks of score block (kb, qb): keys 32kb .. 32kb + 31 of the tile for
    // query half qb, whose row this lane holds is tqq
    auto mask_blk = [&](int e, int kind, int tqq, int valid, f32x16_t& s, int kb, int qb) {
        const int j = tile_j(e);
        if (MASK == MASK_SUB) {
            // 32-token blocks: drop the key halves query half qb may not see
            if (!((tile_sub(e) >> (2 * qb + kb)) & 1))
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = -INFINITY;
        }
        if (MASK == MASK_PAD) {
            if (j * 64 + 64 > valid) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4) >= valid) s[i] = -INFINITY;
            }
        }
        if (MASK == MASK_BAND || MASK == MASK_TOKEN) {
            // a tile whose farthest (query, key) pair is inside the band needs no mask
            if (kind >= 0 && j < a.nb && 64 * abs(kind - j) + 63 > a.band) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (abs(tqq - (j * 64 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4))) > a.band) s[i] = -INFINITY;
            }
        }
        if (MASK == MASK_TOKEN && kind >= 0 && j >= a.nb) {
            // gathered global keys: padding (-1) and keys the band already covers drop out
            const int* gt = gtok_s + (j - a.nb) * 64;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int4 gv = *(const int4*)(gt + 32 * kb + 8 * g4 + 4 * hh);
                const int gs[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    if (gs[e2] < 0 || abs(tqq - gs[e2]) <= a.band) s[4 * g4 + e2] = -INFINITY;
            }
        }
    };
    // S^T block (kb, qb) = K[32kb ..] Q[32qb ..]^T: register i <-> key 32kb + 8(i/4) + 4hh + i%4.
    auto sblk = [&](const bf16x8_t (&kfb)[NC], const bf16x8_t (&qfb)[NC], f32x16_t& s) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfb[c], qfb[c], s, 0, 0, 0);
    };
    // Probabilities of one score block of half qb (key chunks 2kb, 2kb + 1).
    // On a unit's first tile the running max starts at the block's max, or at
    // the finite stand-in kNoMax when the lane's query sees no key of the block.
    // It is raised only when a lane's 16 probabilities would sum past kSumCap:
    // then O and l are rescaled to the block's max and the block is redone.  A
    // finite score met while the max is still kNoMax gives an infinite
    // probability, so it takes the same path, and l and O, still zero, are
    // scaled by exp2(kNoMax - max) = 0.  `issue` places NM matrix products
    // (scores of later blocks, PV products of earlier ones) in the same
    // scheduling region, and the group barriers alternate them with the
    // exp/pack work, so the wave keeps its matrix core busy during its own
    // softmax.
    auto softmax_blk = [&](const f32x16_t& s, int qb, bool first, u32x4_t (&u)[2], auto&& issue, auto nm) {
        constexpr int NM = decltype(nm)::value;
        if (first) m[qb] = __builtin_fmaxf(blk_max(s), kNoMax);
        float lsum;
        auto chunks = [&]() {
            const float muse = m[qb];
            float acc[8];
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * k + 2 * e], c2, -muse));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * k + 2 * e + 1], c2, -muse));
                    u[k][e] = pack_bf16x2(p0, p1);
                    acc[4 * k + e] = p0 + p1;
                }
            lsum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
        };
        issue();
        chunks();
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 56 / NM, 0);   // then a share of the VALU work
        }
        const bool bad = lsum > kSumCap;
        if (__ballot(bad) != 0) {          // wave-uniform, rare
            const float mx = blk_max_rev(s);
            const bool raise = mx > m[qb];
            const float alpha = raise ? __builtin_amdgcn_exp2f(m[qb] - mx) : 1.f;
            l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
            m[qb] = raise ? mx : m[qb];
            chunks();
        }
        l[qb] += lsum;
    };
    auto pv = [&](const bf16x8_t (&va)[4][NDB], int qb, auto c0, const u32x4_t (&u)[2]) {
        constexpr int C0 = decltype(c0)::value;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[C0 + k][db], as_bf16x8(u[k]), o[db][qb], 0, 0, 0);
    };

    // ---- walk the tile list ----
    int e0 = __builtin_amdgcn_readfirstlane(flat[0]);
    auto tile_g = [&](int e) -> int { return rd(u_g, tile_unit(e)); };
    int u_cur = tile_unit(e0);
    int kind_cur = rd(u_kind, u_cur), slot_cur = rd(u_slot, u_cur), g_cur = rd(u_g, u_cur);
    int valid_cur = rd(u_valid, u_cur);
    int tq_cur[2], tq_next[2] = {-1, -1};
    bf16x8_t qf[2][NC];
    load_q(kind_cur, g_cur, qf, tq_cur);
    if (STRIDED) {
        issue_tile_rows(ktile(g_cur, tile_j(e0)), (uint32_t)(RS * 2), kdo, kl);
        issue_tile_rows(vtile(g_cur, tile_j(e0)), (uint32_t)(RS * 2), vdo, vl);
    } else {
        issue_tile1(ktile(g_cur, tile_j(e0)), 0, kdo, kl);
        issue_tile1(vtile(g_cur, tile_j(e0)), 0, vdo, vl);
    }
    reset();

    // A unit's epilogue (normalise, store O and LSE, reset) runs in the next
    // step, after that step's first loads are issued: the stores then have a
    // whole step to drain before the wave next waits on its memory counter.
    bool pend = false;
    int p_slot = -1, p_g = 0, p_tq[2] = {-1, -1};
    auto finish = [&]() {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float lt = pair_sum(l[qb]);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const float lse_v = lt > 0.f ? (m[qb] + log2f(lt)) * kLn2 : -INFINITY;
            const f32x16_t oq[NDB] = {o[0][qb], o[1][qb]};
            store_half(p_slot, p_tq[qb], p_g, 32 * qb + ql, oq, inv, lse_v);
        }
        reset();
    };

    using C0 = std::integral_constant<int, 0>;
    using C2 = std::integral_constant<int, 2>;
    // The next list entry and the partner's count are read from LDS one step
    // ahead (pf_e, pf_left), so the step never waits on them.
    int e1 = F > 1 ? __builtin_amdgcn_readfirstlane(flat[1]) : 0;
    int pf_e = 0, pf_left = F;
    for (int f = 0; f < F; ++f) {
        if (lane == 0) left[wv] = F - f;
        const int partner_left = __builtin_amdgcn_readfirstlane(pf_left);
        if ((e0 & kTileFirst) && f > 0) {   // a new unit (its Q was loaded during the last step)
            u_cur = tile_unit(e0);
            kind_cur = rd(u_kind, u_cur);
            slot_cur = rd(u_slot, u_cur);
            g_cur = rd(u_g, u_cur);
            valid_cur = rd(u_valid, u_cur);
            tq_cur[0] = tq_next[0];
            tq_cur[1] = tq_next[1];
        }
        wait_vmcnt<0>();                   // K(f), V(f) and Q in place
        asm volatile("" ::: "memory");
        bf16x8_t kf[2][NC];
        kread(kbuf, kf);
        bf16x8_t va[4][NDB];
        vread(vbuf, va);
        // Step order: the scores of block (0, 0) first; each later region pairs
        // the softmax of one block with the products that do not depend on it:
        //   S01 S10 | P00;  S11 PV(P00) | P01;  PV(P01) | P10;  PV(P10) | P11;  PV(P11).
        f32x16_t s00, s01, s10, s11;
        sblk(kf[0], qf[0], s00);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every fragment read returned
        asm volatile("" ::: "memory");
        pf_e = f + 2 < F ? flat[f + 2] : 0;
        pf_left = partner >= 0 ? left[partner] : F - f;
        // behind the partner wave: issue first until caught up
        if (F - f > partner_left) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        // The buffers are free: the loads of tile f + 1 go out in four groups
        // spread over the softmax, so that no long burst stalls the wave.
        const bool more = f + 1 < F;
        const uint16_t* kn = ktile(tile_g(e1), tile_j(e1));
        const uint16_t* vn = vtile(tile_g(e1), tile_j(e1));
        if (more) {
            if (STRIDED) lds_load16x4_rows(kdo, (const char*)kn, (uint32_t)(RS * 2), kl + 2048);
            else lds_load16x4_1k(kdo, kn, kl + 2048);
        }
        if (pend) {                         // the previous unit's epilogue
            finish();
            pend = false;
        }
        const bool first = (e0 & kTileFirst) != 0;
        using I4 = std::integral_constant<int, 4>;
        using I8 = std::integral_constant<int, 8>;
        u32x4_t p0[2], p1[2], p2[2], p3[2];
        mask_blk(e0, kind_cur, tq_cur[0], valid_cur, s00, 0, 0);
        softmax_blk(s00, 0, first, p0, [&]() { sblk(kf[0], qf[1], s01); sblk(kf[1], qf[0], s10); }, I8());
        if (more) {
            if (STRIDED) lds_load16x4_rows(kdo, (const char*)(kn + 32 * RS), (uint32_t)(RS * 2), kl + 4096 + 2048);
            else lds_load16x4_1k(kdo, kn + 32 * 64, kl + 4096 + 2048);
        }
        mask_blk(e0, kind_cur, tq_cur[1], valid_cur, s01, 0, 1);
        softmax_blk(s01, 1, first, p1, [&]() { sblk(kf[1], qf[1], s11); pv(va, 0, C0(), p0); }, I8());
        // On a unit's last tile Q is free once every score product is issued:
        // load the next unit's, so that its latency hides behind this step.
        if ((e0 & kTileLast) && f + 1 < F) {
            const int un = tile_unit(e1);
            load_q(rd(u_kind, un), rd(u_g, un), qf, tq_next);
        }
        if (more) {
            if (STRIDED) lds_load16x4_rows(vdo, (const char*)vn, (uint32_t)(RS * 2), vl + 2048);
            else lds_load16x4_1k(vdo, vn, vl + 2048);
        }
        mask_blk(e0, kind_cur, tq_cur[0], valid_cur, s10, 1, 0);
        softmax_blk(s10, 0, false, p2, [&]() { pv(va, 1, C0(), p1); }, I4());
        if (more) {
            if (STRIDED) lds_load16x4_rows(vdo, (const char*)(vn + 32 * RS), (uint32_t)(RS * 2), vl + 4096 + 2048);
            else lds_load16x4_1k(vdo, vn + 32 * 64, vl + 4096 + 2048);
        }
        mask_blk(e0, kind_cur, tq_cur[1], valid_cur, s11, 1, 1);
        softmax_blk(s11, 1, false, p3, [&]() { pv(va, 0, C2(), p2); }, I4());
        pv(va, 1, C2(), p3);
        if (e0 & kTileLast) {               // finished once the next tile's loads are out
            pend = true;
            p_slot = slot_cur;
            p_g = g_cur;
            p_tq[0] = tq_cur[0];
            p_tq[1] = tq_cur[1];
        }
        e0 = e1;
        e1 = __builtin_amdgcn_readfirstlane(pf_e);
    }
    if (pend) finish();
    if (lane == 0) left[wv] = 0;
    wait_vmcnt<0>();

    // A workgroup whose eight lists were the chunks of 8 / n split rows of n
    // chunks each merges those rows here, once every chunk's partial is
    // stored: for each row, wave w takes rows 8w .. 8w + 7 of its 64, eight
    // lanes per row and eight columns per lane, and combines the chunks by
    // log-sum-exp as merge_bf16_kernel does.
    if (a.wg_merge) {
        const int* wm = a.wg_merge + (x * (a.n_bins / kQWaves) + blockIdx.x / kXcds) * kQWaves;
        if (wm[0] >= 0) {
            __syncthreads();
            // every lane-derived value of this tail is computed here, from a copy
            // the compiler cannot see through: nothing is hoisted above the
            // main loop to stay live (and spill) across it
            int tl = (int)threadIdx.x;
            asm volatile("" : "+v"(tl));
            const int tw = tl >> 6, tlane = tl & 63;
            const int r = 8 * tw + (tlane >> 3), part = tlane & 7;
            for (int k = 0; k < kQWaves; ++k) {
                const int mu = wm[k];
                if (mu < 0) break;
                const int b = mu / a.n_merges;
                const MergeItem mi = a.merges[mu % a.n_merges];
                const int nch = mi.n_chunks;
                const size_t bh = (size_t)b * a.H + mi.row / a.nb;
                const int t = (mi.row % a.nb) * 64 + r;
                const size_t first = (size_t)b * a.n_slots + mi.first_slot;
                float lsev[kQWaves];
                float4 p0[kQWaves], p1[kQWaves];
#pragma unroll
                for (int c = 0; c < kQWaves; ++c) {
                    lsev[c] = -INFINITY;
                    p0[c] = p1[c] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (c < nch) {
                        lsev[c] = a.ws_lse[(first + c) * 64 + r];
                        const float* src = a.ws_o + ((first + c) * 64 + r) * D + part * 8;
                        p0[c] = *(const float4*)src;
                        p1[c] = *(const float4*)(src + 4);
                    }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int c = 0; c < kQWaves; ++c) mx = __builtin_fmaxf(mx, lsev[c]);
                uint16_t* orow = (STRIDED ? o_row(a, bh, t, D) : (uint16_t*)a.out + (bh * a.L + t) * D) + part * 8;
                if (mx == -INFINITY) {
                    *(u32x4_t*)orow = u32x4_t{0u, 0u, 0u, 0u};
                    if (part == 0) a.lse[bh * a.L + t] = -INFINITY;
                } else {
                    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
#pragma unroll
                    for (int c = 0; c < kQWaves; ++c) {
                        const float w = expf(lsev[c] - mx);   // 0 past nch
                        wsum += w;
                        acc[0] += w * p0[c].x; acc[1] += w * p0[c].y; acc[2] += w * p0[c].z; acc[3] += w * p0[c].w;
                        acc[4] += w * p1[c].x; acc[5] += w * p1[c].y; acc[6] += w * p1[c].z; acc[7] += w * p1[c].w;
                    }
                    const float inv = 1.f / wsum;
                    u32x4_t o4;
                    o4.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
                    o4.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
                    o4.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
                    o4.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
                    *(u32x4_t*)orow = o4;
                    if (part == 0) a.lse[bh * a.L + t] = mx + logf(wsum);
                }
            }
        }
    }
}

// Merge of a split row (global rows, routed tiles): the chunks of the row
// wrote fp32 partials normalised over their own keys plus their LSE; the row's
// LSE is the log-sum-exp of the chunk LSEs and O the LSE-weighted mean of the
// partial outputs.  A chunk with no allowed key has LSE -inf and weight 0; a
// row with no allowed key at all gets O = 0, LSE = -inf.  Runs as its own
// launch after the attention kernel, so stream order makes the partials
// visible without any device-scope fence.  Four workgroups per split row, 16
// query rows each; 16 threads per row, each owning D/16 columns.  The chunk
// LSEs and the first 8 chunks' partials are loaded in one batch, before any
// of them is used.

template <int D>
__global__ __launch_bounds__(256) void merge_bf16_kernel(const FwdArgs a) {
    constexpr int DP = D / 16;   // columns per thread: 4 or 8
    const int u = blockIdx.x >> 2;
    const int tid = threadIdx.x;
    const int row = (blockIdx.x & 3) * 16 + (tid >> 4), part = tid & 15;
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
        t = kk < a.n_routed ? a.routed_rows[bh * a.routed_stride + kk] : -1;
        if (t >= a.L) t = -1;   // out-of-range rows are skipped, never dereferenced
    }
    if (t < 0) return;
    const float* lse_p = a.ws_lse + (size_t)first * 64 + row;
    const float* src = a.ws_o + ((size_t)first * 64 + row) * D + part * DP;
    // the chunk LSEs and the first 8 chunks' partials are loaded together:
    // one memory round trip for the common case of at most 8 chunks
    float lsev[kMaxChunks];
    float4 v4[8][DP / 4];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) lsev[c] = c < nch ? lse_p[(size_t)c * 64] : -INFINITY;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int d = 0; d < DP / 4; ++d)
            v4[c][d] = c < nch ? *(const float4*)(src + (size_t)c * 64 * D + 4 * d) : make_float4(0.f, 0.f, 0.f, 0.f);
    float mxl = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) mxl = __builtin_fmaxf(mxl, lsev[c]);
    uint16_t* orow = o_row(a, bh, t, D) + part * DP;
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
#pragma unroll
    for (int c0 = 0; c0 < kMaxChunks; c0 += 8) {
        if (c0 >= nch) break;
        if (c0 > 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int d = 0; d < DP / 4; ++d)
                    v4[c][d] = c0 + c < nch ? *(const float4*)(src + (size_t)(c0 + c) * 64 * D + 4 * d)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float w = expf(lsev[c0 + c] - mxl);   // 0 past nch (lse -inf)
            wsum += w;
#pragma unroll
            for (int d = 0; d < DP / 4; ++d) {
                acc[4 * d] += w * v4[c][d].x;
                acc[4 * d + 1] += w * v4[c][d].y;
                acc[4 * d + 2] += w * v4[c][d].z;
                acc[4 * d + 3] += w * v4[c][d].w;
            }
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

// Token layouts: every non-global row gets its random tokens here.  A row
// that fit one unit was written by the attention kernel like any other row
// (bf16 O normalised over its band and global keys, fp32 LSE): it is read
// back from the output and updated in place.  A split row's chunk partials
// (fp32 O and LSE per chunk) are combined by log-sum-exp as in
// merge_bf16_kernel.  Each random token s then joins the same running max and
// sum with score scale * q.k_s and value v_s.  Eight lanes per row,
// D/8 columns each (16- or 32-byte loads); 32 rows per workgroup.  The loads
// that depend on nothing -- chunk LSEs and partials, the q slice, the first
// eight link ids -- go out together, so a row costs two memory round trips:
// those, then the links' K and V slices.  The random tokens fall anywhere in
// their head, so workgroups are mapped to XCDs by (batch, head) group: XCD x
// (workgroup i runs on XCD i % 8) walks the rows of groups x, x + 8, ... one
// group after the other, and the group's K and V (2 x L x D bf16) stay in that
// XCD's L2.  Global rows are computed like the others but not written: their
// routed merge writes them.
template <int D>
__global__ __launch_bounds__(256) void links_merge_kernel(const FwdArgs a) {
    constexpr int DP = D / 8;    // columns per lane: 8 or 16
    constexpr int NC = 2;        // chunks whose partials are loaded up front
    constexpr int LG = 4;        // links whose K and V slices are loaded together
    const int tid = threadIdx.x;
    const int part = tid & 7;
    const int wg_per_group = a.L / 32;
    const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int g = x + kXcds * (j / wg_per_group);
    if (g >= a.B * a.H) return;
    const int t = (j % wg_per_group) * 32 + (tid >> 3);
    const int b = g / a.H, h = g % a.H;
    const int m = a.row_merge[h * a.nb + t / 64];   // the same for the wave's 8 rows
    const int r = t % 64;
    const size_t bh = (size_t)g;
    // read with the other first loads, tested only at the store: branching on
    // it here would put a memory round trip in front of everything else
    const bool global_row = a.tok_global[t] != 0;
    int first = 0, nch = 1;
    if (m >= 0) {
        const MergeItem mi = a.merges[m];
        first = b * a.n_slots + mi.first_slot;
        nch = mi.n_chunks;
    }
    const float* lse_p = a.ws_lse + (size_t)first * 64 + r;
    const float* src = a.ws_o + ((size_t)first * 64 + r) * D + part * DP;
    uint16_t* orow = (uint16_t*)a.out + (bh * a.L + t) * D + part * DP;
    const int32_t* lk = a.links + ((size_t)(bh % a.H) * a.L + t) * a.n_links;
    const uint16_t* kb = (const uint16_t*)a.k + bh * a.L * D + part * DP;
    const uint16_t* vb = (const uint16_t*)a.v + bh * a.L * D + part * DP;

    // ---- independent loads ----
    float lsev[NC];
    float4 pv4[NC][DP / 4];
    if (m >= 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            lsev[c] = c < nch ? lse_p[(size_t)c * 64] : -INFINITY;
#pragma unroll
            for (int d = 0; d < DP / 4; ++d)
                pv4[c][d] = c < nch ? *(const float4*)(src + (size_t)c * 64 * D + 4 * d) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        // a whole row: its output as the one "chunk"
        lsev[0] = a.lse[bh * a.L + t];
#pragma unroll
        for (int d = 0; d < DP / 8; ++d) {
            const u32x4_t w = *(const u32x4_t*)(orow + 8 * d);
            pv4[0][2 * d] = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
            pv4[0][2 * d + 1] = make_float4(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w));
        }
#pragma unroll
        for (int c = 1; c < NC; ++c) {
            lsev[c] = -INFINITY;
#pragma unroll
            for (int d = 0; d < DP / 4; ++d) pv4[c][d] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    u32x4_t qw[DP / 8];
#pragma unroll
    for (int d = 0; d < DP / 8; ++d) qw[d] = *(const u32x4_t*)((const uint16_t*)a.q + (bh * a.L + t) * D + part * DP + 8 * d);
    // the row's link ids, eight at a time: lane `part` loads id j0 + part and
    // the row's eight lanes share them by shuffle (one load instruction, not eight)
    const int lane_base = (threadIdx.x & 63) & ~7;
    int my_id = part < a.n_links ? lk[part] : -1;

    // ---- the band-and-global partials ----
    float mxl = -INFINITY;
    for (int c = 0; c < nch; ++c) mxl = __builtin_fmaxf(mxl, c < NC ? lsev[c] : lse_p[(size_t)c * 64]);
    float acc[DP], wsum = 0.f;
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = 0.f;
    if (mxl != -INFINITY) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float w = expf(lsev[c] - mxl);   // 0 past nch
            wsum += w;
#pragma unroll
            for (int d = 0; d < DP / 4; ++d) {
                acc[4 * d] += w * pv4[c][d].x;
                acc[4 * d + 1] += w * pv4[c][d].y;
                acc[4 * d + 2] += w * pv4[c][d].z;
                acc[4 * d + 3] += w * pv4[c][d].w;
            }
        }
        for (int c = NC; c < nch; ++c) {
            const float w = expf(lse_p[(size_t)c * 64] - mxl);
            wsum += w;
#pragma unroll
            for (int d = 0; d < DP / 4; ++d) {
                const float4 x = *(const float4*)(src + (size_t)c * 64 * D + 4 * d);
                acc[4 * d] += w * x.x;
                acc[4 * d + 1] += w * x.y;
                acc[4 * d + 2] += w * x.z;
                acc[4 * d + 3] += w * x.w;
            }
        }
    }
    float qv[DP];
#pragma unroll
    for (int d = 0; d < DP / 8; ++d) {
        const uint32_t w4[4] = {qw[d].x, qw[d].y, qw[d].z, qw[d].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[8 * d + 2 * e] = bf16_lo(w4[e]);
            qv[8 * d + 2 * e + 1] = bf16_hi(w4[e]);
        }
    }

    // ---- random tokens: ids eight at a time, K and V slices LG at a time ----
    for (int j0 = 0; j0 < a.n_links; j0 += 8) {
        if (j0 > 0) my_id = j0 + part < a.n_links ? lk[j0 + part] : -1;
        for (int q4 = 0; q4 < 8; q4 += LG) {
            int sid[LG];
#pragma unroll
            for (int jj = 0; jj < LG; ++jj) sid[jj] = __shfl(my_id, lane_base + q4 + jj, 64);
            u32x4_t kw[LG][DP / 8], vw[LG][DP / 8];
#pragma unroll
            for (int jj = 0; jj < LG; ++jj) {
                const size_t off = (size_t)(sid[jj] < 0 ? t : sid[jj]) * D;   // a valid row either way
#pragma unroll
                for (int d = 0; d < DP / 8; ++d) {
                    kw[jj][d] = *(const u32x4_t*)(kb + off + 8 * d);
                    vw[jj][d] = *(const u32x4_t*)(vb + off + 8 * d);
                }
            }
            float x[LG];
            float mnew = mxl;
#pragma unroll
            for (int jj = 0; jj < LG; ++jj) {
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < DP / 8; ++d) {
                    const uint32_t w4[4] = {kw[jj][d].x, kw[jj][d].y, kw[jj][d].z, kw[jj][d].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dot = fmaf(qv[8 * d + 2 * e], bf16_lo(w4[e]), dot);
                        dot = fmaf(qv[8 * d + 2 * e + 1], bf16_hi(w4[e]), dot);
                    }
                }
                dot += __shfl_xor(dot, 4, 8);
                dot += __shfl_xor(dot, 2, 8);
                dot += __shfl_xor(dot, 1, 8);
                x[jj] = sid[jj] < 0 ? -INFINITY : dot * a.scale;
                mnew = __builtin_fmaxf(mnew, x[jj]);
            }
            if (mnew > mxl) {
                const float c = mxl == -INFINITY ? 0.f : expf(mxl - mnew);
#pragma unroll
                for (int d = 0; d < DP; ++d) acc[d] *= c;
                wsum *= c;
                mxl = mnew;
            }
#pragma unroll
            for (int jj = 0; jj < LG; ++jj) {
                const float w = x[jj] == -INFINITY ? 0.f : expf(x[jj] - mxl);
                wsum += w;
#pragma unroll
                for (int d = 0; d < DP / 8; ++d) {
                    const uint32_t w4[4] = {vw[jj][d].x, vw[jj][d].y, vw[jj][d].z, vw[jj][d].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[8 * d + 2 * e] = fmaf(w, bf16_lo(w4[e]), acc[8 * d + 2 * e]);
                        acc[8 * d + 2 * e + 1] = fmaf(w, bf16_hi(w4[e]), acc[8 * d + 2 * e + 1]);
                    }
                }
            }
        }
    }

    if (global_row) return;
    const bool empty = mxl == -INFINITY;
    const float inv = empty ? 0.f : 1.f / wsum;
#pragma unroll
    for (int d = 0; d < DP / 8; ++d) {
        u32x4_t w4;
        w4.x = pack_bf16x2(acc[8 * d + 0] * inv, acc[8 * d + 1] * inv);
        w4.y = pack_bf16x2(acc[8 * d + 2] * inv, acc[8 * d + 3] * inv);
        w4.z = pack_bf16x2(acc[8 * d + 4] * inv, acc[8 * d + 5] * inv);
        w4.w = pack_bf16x2(acc[8 * d + 6] * inv, acc[8 * d + 7] * inv);
        *(u32x4_t*)(orow + 8 * d) = w4;
    }
    if (part == 0) a.lse[bh * a.L + t] = empty ? -INFINITY : mxl + logf(wsum);
}

// Token layouts: copy the K and V rows of the global tokens into contiguous
// 64-row tiles, kg/vg [B*H][n_gt*64][D], zero past the last global token (a
// masked key still meets V in the PV product, so it must hold a finite value).
// One thread per 16 bytes.
template <int D>
__global__ __launch_bounds__(256) void gather_global_kernel(const FwdArgs a, uint16_t* kg, uint16_t* vg) {
    const int rows_per_g = a.n_gt * 64;
    const size_t n8 = (size_t)a.B * a.H * rows_per_g * (D / 8);
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const size_t row = i / (D / 8);
    const int col = (int)(i % (D / 8)) * 8;
    const size_t g = row / rows_per_g;
    const int tok = a.gtok[row % rows_per_g];
    u32x4_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (tok >= 0) {
        const size_t src = (g * a.L + tok) * D + col;
        kv = *(const u32x4_t*)((const uint16_t*)a.k + src);
        vv = *(const u32x4_t*)((const uint16_t*)a.v + src);
    }
    *(u32x4_t*)(kg + row * D + col) = kv;
    *(u32x4_t*)(vg + row * D + col) = vv;
}

// The attention kernels are launched with hipExtLaunchKernelGGL: given events,
// the dispatch itself records the kernel's start and stop (no separate marker
// packets between kernels, which would add to the time they measure).
template <int D, int MASK, bool STRIDED = false>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s, hipEvent_t before, hipEvent_t after) {
    const int64_t grid = (int64_t)kXcds * a.n_bins;
    if (grid == 0) return hipSuccess;
    hipExtLaunchKernelGGL((fwd_bf16_kernel<D, MASK, STRIDED>), dim3((unsigned)grid), dim3(kThreads), 0, s, before,
                          after, 0, a);
    return hipGetLastError();
}

template <int MASK, bool STRIDED = false>
hipError_t launch_d64(const FwdArgs& a, hipStream_t s, hipEvent_t before, hipEvent_t after) {
    // kQWaves lists (bins) per workgroup
    if (a.n_bins % kQWaves != 0) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)kXcds * (a.n_bins / kQWaves);
    if (grid == 0) return hipSuccess;
    hipExtLaunchKernelGGL((fwd_bf16_d64_kernel<MASK, STRIDED>), dim3((unsigned)grid), dim3(kQThreads), 0, s, before,
                          after, 0, a);
    return hipGetLastError();
}

}  // namespace

int fwd_bf16_ctas_per_cu(int head_dim, bool two_wave) {
    // D = 64: one workgroup holds the whole CU.
    if (head_dim == 64 && !two_wave) return 1;
    int n = 0;
    hipError_t e = head_dim == 64
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_bf16_kernel<64, MASK_BITS>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_bf16_kernel<128, MASK_NONE>, kThreads, 0);
    if (e != hipSuccess || n < 1) n = 1;
    // Measured on MI355X: with 32 KiB of LDS per workgroup only 4 workgroups
    // are resident per CU (the occupancy query reports 5).  Both widths hold
    // about 34 KiB: four per CU, two waves per SIMD.
    return n < 4 ? n : 4;
}

#ifdef BSATTN_DEBUG
// Debug builds: the word the kernels report schedule errors into (one per
// device, cleared before and read back after every forward launch).
__device__ uint32_t g_dbg_word;
#endif

static hipError_t launch_fwd_bf16_impl(const FwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before,
                                hipEvent_t after) {
    hipError_t e;
    if (a.strided) {
        // the attention layer's layout: block (any block size) and band layouts
        if (mask == MASK_TOKEN || mask == MASK_BITS) return hipErrorInvalidValue;
        if (head_dim == 64)
            e = mask == MASK_PAD    ? launch_d64<MASK_PAD, true>(a, s, before, after)
              : mask == MASK_BAND   ? launch_d64<MASK_BAND, true>(a, s, before, after)
              : mask == MASK_SUB    ? launch_d64<MASK_SUB, true>(a, s, before, after)
                                    : launch_d64<MASK_NONE, true>(a, s, before, after);
        else
            e = mask == MASK_PAD    ? launch_fwd_t<128, MASK_PAD, true>(a, s, before, after)
              : mask == MASK_BAND   ? launch_fwd_t<128, MASK_BAND, true>(a, s, before, after)
              : mask == MASK_SUB    ? launch_fwd_t<128, MASK_SUB, true>(a, s, before, after)
                                    : launch_fwd_t<128, MASK_NONE, true>(a, s, before, after);
    } else if (mask == MASK_BITS) {
        // the two-wave kernel at either width (the D = 64 kernel has no bit mask)
        e = head_dim == 64 ? launch_fwd_t<64, MASK_BITS>(a, s, before, after)
                           : launch_fwd_t<128, MASK_BITS>(a, s, before, after);
    } else if (head_dim == 64) {
        e = mask == MASK_PAD   ? launch_d64<MASK_PAD>(a, s, before, after)
          : mask == MASK_BAND  ? launch_d64<MASK_BAND>(a, s, before, after)
          : mask == MASK_SUB   ? launch_d64<MASK_SUB>(a, s, before, after)
          : mask == MASK_TOKEN ? launch_d64<MASK_TOKEN>(a, s, before, after)
                               : launch_d64<MASK_NONE>(a, s, before, after);
    } else {
        e = mask == MASK_PAD   ? launch_fwd_t<128, MASK_PAD>(a, s, before, after)
          : mask == MASK_BAND  ? launch_fwd_t<128, MASK_BAND>(a, s, before, after)
          : mask == MASK_SUB   ? launch_fwd_t<128, MASK_SUB>(a, s, before, after)
          : mask == MASK_TOKEN ? launch_fwd_t<128, MASK_TOKEN>(a, s, before, after)
                               : launch_fwd_t<128, MASK_NONE>(a, s, before, after);
    }
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.B * a.n_merges + (a.n_routed > 0 ? (int64_t)a.B * a.H * a.n_rt : 0);
    if (units == 0 && mask != MASK_TOKEN) return hipSuccess;
    if (head_dim == 64 && a.wg_merge && a.n_routed == 0) return hipSuccess;   // merged inside the kernel
    if (mask == MASK_TOKEN) {
        // the global rows (routed units) by the plain merge, every other row with its random tokens
        FwdArgs g = a;
        g.n_merges = 0;
        const int64_t gu = a.n_routed > 0 ? (int64_t)a.B * a.H * a.n_rt : 0;
        if (gu > 0) {
            if (head_dim == 64) hipLaunchKernelGGL(merge_bf16_kernel<64>, dim3((unsigned)(4 * gu)), dim3(256), 0, s, g);
            else hipLaunchKernelGGL(merge_bf16_kernel<128>, dim3((unsigned)(4 * gu)), dim3(256), 0, s, g);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const int64_t groups = (int64_t)a.B * a.H;
        if (groups == 0) return hipSuccess;
        const dim3 grid((unsigned)(kXcds * ((groups + kXcds - 1) / kXcds) * (a.L / 32)));
        if (head_dim == 64) hipLaunchKernelGGL(links_merge_kernel<64>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(links_merge_kernel<128>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    // Split band rows first, routed tiles after them: a routed token can lie
    // in a split band row's block, and both merges write its O and LSE, so the
    // routed result must come second (stream order) to be the one that stays.
    auto merge = [&](const FwdArgs& m, int64_t n) {
        if (n == 0) return;
        if (head_dim == 64) hipLaunchKernelGGL(merge_bf16_kernel<64>, dim3((unsigned)(4 * n)), dim3(256), 0, s, m);
        else hipLaunchKernelGGL(merge_bf16_kernel<128>, dim3((unsigned)(4 * n)), dim3(256), 0, s, m);
    };
    const int64_t band_units = (int64_t)a.B * a.n_merges;
    if (a.n_routed > 0 && band_units > 0) {
        FwdArgs band = a;
        band.n_routed = 0;
        merge(band, band_units);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        FwdArgs routed = a;
        routed.n_merges = 0;
        merge(routed, units - band_units);
    } else {
        merge(a, units);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before,
                           hipEvent_t after) {
#ifdef BSATTN_DEBUG
    // Debug builds synchronise the stream: the kernels' schedule checks are
    // read back and a failed one is reported as a device-side assert.
    uint32_t* dw = nullptr;
    hipError_t e = hipGetSymbolAddress((void**)&dw, HIP_SYMBOL(g_dbg_word));
    if (e != hipSuccess) return e;
    static const uint32_t zero = 0;
    if ((e = hipMemcpyAsync(dw, &zero, sizeof(zero), hipMemcpyHostToDevice, s)) != hipSuccess) return e;
    FwdArgs ad = a;
    ad.dbg = dw;
    if ((e = launch_fwd_bf16_impl(ad, head_dim, mask, s, before, after)) != hipSuccess) return e;
    uint32_t flag = 0;
    if ((e = hipMemcpyAsync(&flag, dw, sizeof(flag), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    return flag ? hipErrorAssert : hipSuccess;
#else
    return launch_fwd_bf16_impl(a, head_dim, mask, s, before, after);
#endif
}

hipError_t launch_gather_global(const FwdArgs& a, int head_dim, hipStream_t s) {
    const size_t n8 = (size_t)a.B * a.H * a.n_gt * 64 * (head_dim / 8);
    if (n8 == 0) return hipSuccess;
    const dim3 grid((unsigned)((n8 + 255) / 256));
    uint16_t* kg = const_cast<uint16_t*>(a.kg);
    uint16_t* vg = const_cast<uint16_t*>(a.vg);
    if (head_dim == 64) hipLaunchKernelGGL(gather_global_kernel<64>, grid, dim3(256), 0, s, a, kg, vg);
    else hipLaunchKernelGGL(gather_global_kernel<128>, grid, dim3(256), 0, s, a, kg, vg);
    return hipGetLastError();
}

}  // namespace bsattn
