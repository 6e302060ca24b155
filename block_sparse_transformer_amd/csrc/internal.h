// internal.h -- layout object, work schedule and kernel argument blocks of libbsattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <memory>
#include <mutex>
#include <vector>

#include "bsattn.h"
#include "layout_rule.h"

namespace bsattn {

constexpr int kBlock = 64;        // tokens per block and rows per query tile
constexpr int kChunkTiles = 16;   // a row longer than this is split across workgroups
constexpr int kMaxChunks = 32;    // upper bound on the split of one row

// MASK_SUB: layouts of 32-token blocks; each 64-token tile carries which of
// its 2 x 2 sub-blocks are allowed (bit 2a + b: query half a, key half b).
// MASK_TOKEN: token-granular layouts -- the token band on a row's own tiles,
// and gathered tiles of the global tokens' keys (key blocks nb, nb + 1, ...).
// MASK_BITS: per-query kept keys given as one 64-bit word per (query, key
// block) (per-query top-keep layouts).
// Backward only: MASK_ROUTED_Q -- dQ of gathered routed query tiles over every
// key block; MASK_BAND_ROUTED -- dK/dV of band columns whose lists also hold
// the routed tiles (entries nb + r), whose pairs inside the band are skipped
// (the band entries hold them).
enum MaskMode : int {
    MASK_NONE = 0, MASK_PAD = 1, MASK_BAND = 2, MASK_SUB = 3, MASK_TOKEN = 4, MASK_BITS = 5,
    MASK_ROUTED_Q = 6, MASK_BAND_ROUTED = 7
};
constexpr int kMaxTokGlobal = 2048;   // global tokens of a token layout (their list lives in LDS)
constexpr int kMaxLinks = 64;         // random tokens per row of a token layout
constexpr int kMaxAdaptiveBlocks = 1024;   // key blocks per side of a content-adaptive layout
constexpr int kMaxTopLen = 8192;           // sequence length of a per-query top-keep layout

// One workgroup's share: query block `row` (= h*nb + i) over key blocks
// col_idx[col_begin, col_end).  slot < 0: the whole row, written straight to
// O/LSE; slot >= 0: one chunk of a split row, written as a partial (O
// normalised over the chunk, chunk LSE) to workspace slot b*n_slots + slot.
// The chunks of split row `merge` occupy slots [first_slot, first_slot +
// n_chunks); the merge kernel combines them.  row < 0: no work (padding of a
// head's item list).
struct WorkItem {
    int32_t row, col_begin, col_end, slot;
    int32_t merge, first_slot, n_chunks, pad;
};

// A split row: its chunks occupy slots [first_slot, first_slot + n_chunks).
struct MergeItem {
    int32_t row, first_slot, n_chunks, pad;
};

constexpr int kXcds = 8;             // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kMaxBinUnits = 64;     // units of one workgroup (one per lane)
constexpr int kMaxBinTiles = 512;    // tiles of one workgroup (its list lives in LDS)
// D = 64 kernel: one workgroup of kQWaves waves per CU, one unit/tile list per wave
constexpr int kQWaves = 8;
// Flat tile entry of a workgroup's list: key block (18 bits) | sub-block
// mask << 18 (4 bits) | unit << 22 | first | last.
constexpr int kTileJ = (1 << 18) - 1;
constexpr int kTileSubShift = 18;
constexpr int kTileUnitShift = 22;
constexpr int kTileFirst = 1 << 29;
constexpr int kTileLast = 1 << 30;

// Chunking of a row of `len` tiles: number of chunks and tiles per chunk
// (at most 64 tiles per chunk: a chunk's key-block list fits one wave's lanes).
inline void split_row(int32_t len, int32_t* n_chunks, int32_t* per_chunk, int32_t limit = kChunkTiles) {
    int32_t per = limit;
    if ((len + per - 1) / per > kMaxChunks) per = (len + kMaxChunks - 1) / kMaxChunks;
    if (per > 64) per = 64;
    const int32_t n = (len + per - 1) / per;
    *n_chunks = n;
    *per_chunk = (len + n - 1) / n;
}

// Everything a forward launch needs, passed by value to the kernels.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    float* ws_o;              // [total_slots][64][D] fp32
    float* ws_lse;            // [total_slots][64]
    const WorkItem* items;    // [H][n_item_per_head] explicit items, longest first per head
    const MergeItem* merges;
    const int32_t* col_idx;
    const int32_t* valid_len; // [B] or null
    const int32_t* routed_rows;
    int32_t n_items, n_merges;
    int32_t items_per_head;   // explicit items per head (NOP-padded to equal length)
    // persistent schedule: n_bins lists per XCD (one per workgroup, or one
    // per wave for D = 64, kQWaves per workgroup).  List (x, bin) runs units
    // units[unit_ptr[x*n_bins+bin] ..) -- {kind, slot, group, first tile}: kind >= 0 the query block of a layout row (slot: partial
    // slot within a batch entry, -1 for a whole row), kind < 0 routed tile
    // -1-kind (slot: chunk); group = b * H + h; first tile: offset of the
    // unit's tiles in the bin's list -- over the flat tile list
    // tiles[tile_ptr[x*n_bins+bin] ..), entries key block | sub-block mask
    // << 18 | unit << 22 | kTileFirst | kTileLast (unit: index within the
    // bin; mask bit 2a + b: query half a may see key half b, 0xF unless the
    // layout has 32-token blocks).
    int32_t n_bins;
    const int4* units;
    const int32_t* unit_ptr;
    const int32_t* tiles;
    const int32_t* tile_ptr;
    int32_t B, H, L, nb, n_slots;
    // routed tiles (gathered query rows over all key blocks), placed first in the grid
    int32_t n_routed;         // k rows per (b, h); 0 = no routed tiles
    int32_t n_rt;             // ceil(k / 64) routed tiles per (b, h)
    int32_t r_chunks;         // chunks per routed tile
    int32_t r_chunk_tiles;    // key blocks per chunk
    int32_t r_slot_base;      // first workspace slot of routed partials
    // D = 64 kernel: per workgroup, kQWaves entries: the split rows it merges
    // after its lists (b * n_merges + m, or -1); nullptr when the merge kernel
    // merges every row
    const int32_t* wg_merge;
    int32_t band;             // token band of non-routed rows (MASK_BAND, MASK_TOKEN)
    int32_t routed_stride;    // routed_rows entries between (b, h) groups (0: one list shared by all)
    // token layouts (MASK_TOKEN): key block j >= nb is gathered tile j - nb of
    // the global tokens' keys, kg/vg [B*H][n_gt*64][D]; gtok the global tokens
    // padded with -1 to n_gt*64; the merge adds each row's random tokens
    // links[h][t][0..n_links) (-1: none) and skips global rows (tok_global).
    const uint16_t* kg;
    const uint16_t* vg;
    const int32_t* gtok;
    int32_t n_gt;
    int32_t n_links;
    const int32_t* links;
    const uint8_t* tok_global;
    const int32_t* row_merge;   // token layouts: [H * nb] merge item of a split row, -1 for a whole row
    // per-query top-keep layouts (MASK_BITS): [B*H][L][nb] words, bit b of
    // word (g, t, j) set iff query t of group g keeps key 64 j + b
    const uint64_t* keep_bits;
    // strided tensors (the attention layer; the kernels' STRIDED instances):
    // row t of head h of batch entry b of Q, K, V sits at b*qkv_bs + h*qkv_hs
    // + t*qkv_ts elements from its base, of O at b*o_bs + h*o_hs + t*o_ts.
    // Otherwise Q, K, V and O are contiguous [B, H, L, D].
    bool strided;
    int64_t qkv_bs, qkv_hs, qkv_ts, o_bs, o_hs, o_ts;
    float scale;              // score scale
    float scale_log2;         // scale * log2(e)
    // debug builds (BSATTN_DEBUG): a device word the forward kernels OR a bit
    // into for every schedule entry out of bounds (1 unit record, 2 tile
    // entry, 4 list length); null otherwise
    uint32_t* dbg;
};

// ---- backward ----
// One workgroup's share of a backward kernel: block `head_blk` (= h*nb + blk)
// -- the query block for dQ, the key block for dK/dV -- against the blocks
// idx[begin, end) of the other side (the layout's key blocks of the row for
// dQ; the query blocks whose rows hold the key block for dK/dV).  slot < 0:
// the whole row/column, written straight to the bf16 output; slot >= 0: one
// chunk, written as an fp32 partial to workspace slot b*n_slots + slot.
struct BwdItem {
    int32_t head_blk, begin, end, slot;
};
// A split row/column: its chunks' partials occupy slots [first_slot, first_slot + n_chunks).
struct BwdSum {
    int32_t head_blk, first_slot, n_chunks, pad;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;             // [B*H*L] rowsum(dO * O)
    float* ws_dq;             // [B*n_qslots][64][D] fp32 partials
    float* ws_dk;             // [B*n_kslots][64][D]
    float* ws_dv;             // [B*n_kslots][64][D]
    const BwdItem* items;     // this launch's items (dQ or dK/dV), [H][items_per_head]
    const int32_t* idx;       // this launch's block lists
    const uint8_t* idx_sub;   // sub-block masks parallel to idx (32-token layouts), or null
    const BwdSum* sums;
    int32_t n_items, n_sums;
    int32_t items_per_head;   // per-head item lists padded to this length (head_blk < 0: none)
    const int32_t* valid_len; // [B] or null
    int32_t B, H, L, nb, n_slots;
    int32_t band;             // band layouts: |t - s| <= band (MASK_BAND)
    // routed variant: routed tile r holds rows routed_rows[grp * routed_stride
    // + r*64 ..] (routed_stride = n_routed: one list per (b, h); 0: one list
    // shared by all, the global rows of a token layout)
    const int32_t* routed_rows;
    int32_t n_routed;
    int32_t routed_stride;
    float scale;              // score scale
    float scale_log2;         // scale * log2(e)
    // token layouts: the global tokens gtok[0 .. n_g) and their flags [L]; the
    // random tokens links[h][t][0 .. n_links) (-1: none); per key, the rows whose
    // random tokens hold it: trows[tptr[h (L + 1) + s] .. tptr[h (L + 1) + s + 1]);
    // ws_g: fp32 partials of the global keys' dK, dV [B*H][n_g][g_chunks][2][D]
    const int32_t* gtok;
    int32_t n_g;
    const uint8_t* tok_global;
    const int32_t* links;
    int32_t n_links;
    const int32_t* tptr;
    const int32_t* trows;
    float* ws_g;
    int32_t g_chunks;
    // debug builds (BSATTN_DEBUG): a device word the dQ and dK/dV kernels OR a
    // bit into for an item (8) or a list entry (16) out of bounds; null otherwise
    uint32_t* dbg;
};

// ---- the allocation-free forward (kernels/noalloc.hip) ----
// Size of the file-scope device array that serves as its workspace.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// That array's device address on the current device (resolved once per device).
hipError_t noalloc_scratch(void** ptr);
// bsattn_forward that fails instead of building a schedule (api.cpp).
bsattn_status forward_prepared_only(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B, int32_t H,
                                    int32_t L, int32_t D, const void* q, const void* k, const void* v,
                                    void* out, float* lse, const int32_t* key_valid_len, float scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);
bsattn_status set_failure(bsattn_status st, const char* msg);

// ---- launchers (defined in kernels/*.hip) ----
hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int mask, hipStream_t s,
                           hipEvent_t before, hipEvent_t after);
// workgroups of the bf16 kernel resident per CU; two_wave: the two-wave
// kernel also at D = 64 (per-query top-keep layouts)
int fwd_bf16_ctas_per_cu(int head_dim, bool two_wave = false);
// per-query top-keep selection: bits [G][L][L/64] (see FwdArgs::keep_bits);
// given events, its dispatch records its start and stop
hipError_t launch_topr_select(const void* q, const void* k, uint64_t* bits, int G, int L, int D, int keep,
                              hipStream_t s, hipEvent_t before = nullptr, hipEvent_t after = nullptr);
// content-adaptive layouts (kernels/adaptive.hip): block sums of q and k, then the
// kept key blocks cols [G][nb][keep]; and the schedule's tile entries filled from cols
hipError_t launch_adaptive_select(const void* q, const void* k, double* qs, double* ks, int32_t* cols, int G,
                                  int L, int D, int keep, hipStream_t s);
hipError_t launch_fill_tiles(const int32_t* skel, int32_t* live, const int4* units, const int32_t* unit_ptr,
                             const int32_t* tile_ptr, int n_lists, const int32_t* cols, int nb, int keep,
                             hipStream_t s);
// token layouts: K/V rows of the global tokens -> kg/vg (zero past the last global token)
hipError_t launch_gather_global(const FwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, const int32_t* row_ptr, int head_dim, int mask,
                          hipStream_t s, hipEvent_t before, hipEvent_t after);
// router workspace: the fp64 scores [B, H, L]
size_t route_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t k);
hipError_t launch_route_topk(const void* q, const float* w, int32_t B, int32_t H, int32_t L,
                             int32_t D, int32_t k, int32_t* out, void* workspace, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int mask, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int mask, hipStream_t s, hipEvent_t before = nullptr,
                           hipEvent_t after = nullptr);
// sum split partials into the bf16 output(s): which = 0 dQ, 1 dK and dV
hipError_t launch_bwd_sum(const BwdArgs& a, int head_dim, int which, hipStream_t s);
// sum the routed tiles' dQ partials into the dQ rows of their routed tokens
hipError_t launch_bwd_routed_sum(const BwdArgs& a, int head_dim, hipStream_t s);
// token layouts (kernels/bwd_token.hip): the pairs the band and the global rows
// do not cover, added to dQ, dK, dV in place -- every non-global row's global
// keys outside its band and its random tokens
hipError_t launch_tok_bwd_extra(const BwdArgs& a, int head_dim, hipStream_t s);
// candidate-list attention (kernels/candidates.hip): positions [B, L, k] of the
// candidate generator (x bf16 [B, L, C], w fp32 [3][C][k], bias fp32 [k]),
// then attention over the best `keep` distinct candidates of every query
// (kept: optional int32 [B, H, L, keep], ascending, -1 padded)
constexpr int kMaxCandidates = 64;
hipError_t launch_cand_positions(const void* x, const float* w, const float* bias, int B, int L, int C, int k,
                                 int32_t* pos, hipStream_t s);
hipError_t launch_cand_attention(const void* q, const void* k, const void* v, const int32_t* pos, int B, int H,
                                 int L, int D, int n_cand, int keep, float scale, void* out, float* lse,
                                 int32_t* kept, hipStream_t s, hipEvent_t before = nullptr,
                                 hipEvent_t after = nullptr);
// global keys whose dK/dV one workgroup of the token backward accumulates
constexpr int tok_global_keys_per_wg(int head_dim) { return head_dim == 64 ? 4 : 2; }
// attention layer (kernels/layer.hip)
hipError_t launch_split_heads(const float* qkv32, const void* b_qkv, void* q, void* k, void* v, int B, int L,
                              int H, int D, hipStream_t s);
hipError_t launch_merge_heads(const void* o, void* o2, int B, int L, int H, int D, hipStream_t s);
hipError_t launch_bias_out(const float* out32, const void* b_proj, void* out, size_t rows, int C, hipStream_t s);
// kind 0: rule (64-token blocks), 1: token band, 2: rule on 32-token blocks
// (subs receives the quarter bits), 3: rule on 128-token blocks
hipError_t launch_layout_build(const RowRule& rule, int kind, int32_t H, int32_t nb,
                               int32_t band, int32_t* row_ptr, int32_t* col_idx, uint8_t* subs, hipStream_t s);

}  // namespace bsattn

// The opaque layout handle of the C ABI.
struct bsattn_layout {
    int32_t H = 0, L = 0, nb = 0, block = 0;
    int32_t kind = 0;           // 0: window/global/random rule, 1: token band, 2: token pattern,
                                // 3: content-adaptive (key blocks chosen per call from q and k),
                                // 4: per-query top-keep (every key block; keys chosen per call)
    int32_t band_tokens = -1;
    bsattn::RowRule rule{};
    std::vector<int32_t> row_ptr, col_idx;
    // 32-token layouts: for each tile of col_idx, its allowed 2 x 2 sub-blocks
    // (bit 2a + b: query half a, key half b); empty for 64/128-token layouts
    std::vector<uint8_t> tile_sub;
    // token pattern (kind 2): global tokens, their flags [L], random tokens
    // [H][L][n_links] (-1 past a row's count); the CSR rows list the band's
    // tiles and then the gathered tiles nb .. nb + n_gt - 1 of the global keys
    std::vector<int32_t> tok_g, links;
    std::vector<uint8_t> tok_flag;
    std::vector<int32_t> row_merge;   // [H * nb]: merge item of a split row, -1 for a whole row
    int32_t n_links = 0, n_gt = 0;
    int32_t* d_gtok = nullptr;      // tok_g padded with -1 to n_gt * 64
    int32_t* d_links = nullptr;
    uint8_t* d_tok_flag = nullptr;
    int32_t* d_row_merge = nullptr;
    std::vector<bsattn::WorkItem> items;
    std::vector<bsattn::MergeItem> merges;
    int32_t n_slots = 0;        // partial slots per batch entry
    int32_t chunk_tiles = bsattn::kChunkTiles;   // rows longer than this are split (into even chunks)
    // device copy (after upload)
    int device = -1;
    int32_t items_per_head = 0;
    int32_t* d_row_ptr = nullptr;
    int32_t* d_col_idx = nullptr;
    uint8_t* d_col_sub = nullptr;   // device tile_sub (32-token layouts)
    bsattn::WorkItem* d_items = nullptr;
    bsattn::MergeItem* d_merges = nullptr;
    // persistent schedules built on first use, keyed by (batch, head width,
    // routed units per group, tiles per routed unit); device arrays
    struct Sched {
        int32_t batch, head_dim, n_bins, nru, rct;
        int4* d_units;
        int32_t* d_unit_ptr;
        int32_t* d_tiles;
        int32_t* d_tile_ptr;
        // D = 64 with every split row in n chunks, n dividing kQWaves: the
        // workgroup (XCD x, index c) holding the chunks of kQWaves / n rows
        // merges them itself; d_wg_merge[(x * (n_bins / kQWaves) + c) * kQWaves
        // + r] = b * n_merges + m of its r-th row, -1 past its rows (and for
        // workgroups that merge nothing).  nullptr: the merge kernel merges.
        int32_t* d_wg_merge;
    };
    mutable std::vector<Sched> scheds;
    mutable std::unique_ptr<std::mutex> sched_mu{new std::mutex};
    // backward work lists, built and uploaded on the first backward call
    struct Bwd {
        int32_t n_qslots = 0, n_kslots = 0;
        int32_t q_per_head = 0, k_per_head = 0;
        std::vector<bsattn::BwdItem> q_items, k_items;   // [H][per_head], longest first
        std::vector<bsattn::BwdSum> q_sums, k_sums;
        std::vector<int32_t> k_idx;                      // query blocks per key block (CSC)
        std::vector<uint8_t> k_sub;                      // their sub-block masks (32-token layouts)
        bsattn::BwdItem* d_q_items = nullptr;
        bsattn::BwdItem* d_k_items = nullptr;
        bsattn::BwdSum* d_q_sums = nullptr;
        bsattn::BwdSum* d_k_sums = nullptr;
        int32_t* d_k_idx = nullptr;
        uint8_t* d_k_sub = nullptr;
        bool built = false, uploaded = false;
    };
    mutable Bwd bwd;
    // backward work lists of routed calls on a band layout, one per routed
    // tile count, built and uploaded on first use
    struct RoutedBwd {
        int32_t n_rt = 0, r_chunks = 1, per = 1;
        int32_t n_qslots = 0;                         // band dQ slots, then the routed tiles' chunks
        int32_t rq_per_head = 0, k_per_head = 0, n_kslots = 0;
        std::vector<bsattn::BwdItem> rq_items, k_items;
        std::vector<bsattn::BwdSum> rq_sums, k_sums;
        std::vector<int32_t> k_idx;                   // per column: band query blocks, then nb + r
        bsattn::BwdItem* d_rq_items = nullptr;
        bsattn::BwdItem* d_k_items = nullptr;
        bsattn::BwdSum* d_rq_sums = nullptr;
        bsattn::BwdSum* d_k_sums = nullptr;
        int32_t* d_k_idx = nullptr;
    };
    mutable std::vector<RoutedBwd> rbwd;
    // token layouts, backward: for each (head, key s) the non-global rows whose
    // random tokens hold s, ascending: tlink_rows[tlink_ptr[h (L + 1) + s] ..)
    std::vector<int32_t> tlink_ptr, tlink_rows;
    mutable int32_t* d_tlink_ptr = nullptr;
    mutable int32_t* d_tlink_rows = nullptr;
};

namespace bsattn {

// Host half of a forward schedule (no HIP call).  List i = x * n_bins + b
// (XCD x, bin b) holds units [unit_ptr[i], unit_ptr[i + 1]) and flat tile
// entries [tile_ptr[i], tile_ptr[i + 1]); wg_merge is empty unless the D = 64
// kernel merges split rows itself.  capacity: workgroups resident at once;
// cus: compute units.
struct PackedSchedule {
    int32_t n_bins = 0;
    std::vector<int4> units;
    std::vector<int32_t> unit_ptr, tiles, tile_ptr, wg_merge;
};
bsattn_status pack_schedule(const bsattn_layout* lay, int32_t B, int32_t D, int32_t nru, int32_t rct,
                            int32_t r_chunks, int capacity, int cus, PackedSchedule* out);

}  // namespace bsattn
