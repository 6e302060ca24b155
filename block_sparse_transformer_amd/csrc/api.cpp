// api.cpp -- C ABI of libbsattn: validation, host layout build, scheduling, dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <map>
#include <queue>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>
#include <tuple>

#include <hipblaslt/hipblaslt.h>
#include <rocblas/rocblas.h>

#include "internal.h"

using namespace bsattn;

namespace {

thread_local std::string g_error;
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;
// Set while a call must not allocate (bsattn_forward_noalloc): a schedule that
// was not built by bsattn_prepare is then an error instead of being built.
thread_local bool g_no_build = false;
// Strides of Q/K/V and O for the forward that the attention layer runs on its
// own buffers (null: contiguous [B, H, L, D]).
struct LayerStrides {
    int64_t qkv_bs, qkv_hs, qkv_ts, o_bs, o_hs, o_ts;
};
thread_local const LayerStrides* g_strides = nullptr;

bsattn_status fail(bsattn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

bsattn_status ok() {
    g_error.clear();
    return BSATTN_OK;
}

bsattn_status hip_fail(hipError_t e, const char* what) {
    return fail(BSATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work schedule: rows of <= kChunkTiles blocks become one item; longer rows are
// split into balanced chunks whose partials the merge kernel combines.  Each head's items are ordered longest first (so long chunks start
// before short rows) and padded with no-op items to a common length; the
// kernel deals whole (batch, head) groups to one XCD so their K/V stay in
// that XCD's L2.
void build_schedule(bsattn_layout* lay) {
    lay->items.clear();
    lay->merges.clear();
    int32_t slot = 0;
    std::vector<std::vector<WorkItem>> per_head((size_t)lay->H);
    for (int32_t h = 0; h < lay->H; ++h) {
        auto& hi = per_head[(size_t)h];
        for (int32_t i = 0; i < lay->nb; ++i) {
            const int32_t r = h * lay->nb + i;
            const int32_t b0 = lay->row_ptr[r], b1 = lay->row_ptr[r + 1];
            const int32_t len = b1 - b0;
            if (len <= lay->chunk_tiles) {
                hi.push_back({r, b0, b1, -1, -1, 0, 0, 0});
                continue;
            }
            int32_t nch, per;
            split_row(len, &nch, &per, lay->chunk_tiles);
            const int32_t m = (int32_t)lay->merges.size();
            lay->merges.push_back({r, slot, nch, 0});
            const int32_t first = slot;
            for (int32_t c = 0; c < nch; ++c) {
                const int32_t s0 = b0 + c * per;
                const int32_t e0 = std::min(b1, s0 + per);
                hi.push_back({r, s0, e0, slot++, m, first, nch, 0});
            }
        }
        std::stable_sort(hi.begin(), hi.end(), [](const WorkItem& x, const WorkItem& y) {
            return (x.col_end - x.col_begin) > (y.col_end - y.col_begin);
        });
    }
    // token layouts: which rows are split (their merge item), for the merge that adds random tokens
    if (lay->kind == 2) {
        lay->row_merge.assign((size_t)lay->H * lay->nb, -1);
        for (size_t m = 0; m < lay->merges.size(); ++m) lay->row_merge[(size_t)lay->merges[m].row] = (int32_t)m;
    }
    size_t per = 0;
    for (auto& hi : per_head) per = std::max(per, hi.size());
    for (auto& hi : per_head) {
        lay->items.insert(lay->items.end(), hi.begin(), hi.end());
        for (size_t a = hi.size(); a < per; ++a) lay->items.push_back({-1, 0, 0, -1, -1, 0, 0, 0});
    }
    lay->items_per_head = (int32_t)per;
    lay->n_slots = slot;
}

// End of the tiles of CSR row r that the backward's block passes walk: a
// token layout's rows end with its n_gt gathered tiles of global keys, whose
// pairs the token kernels take instead; the band tiles come first.
int32_t bwd_row_end(const bsattn_layout* lay, int32_t r) {
    return lay->row_ptr[(size_t)r + 1] - (lay->kind == 2 ? lay->n_gt : 0);
}

// Backward work lists.  dQ: every query block against the key blocks of its
// row; dK/dV: every key block against the query blocks whose rows hold it
// (the layout transposed, per head).  Lists longer than kChunkTiles are
// split into chunks whose fp32 partials a summing launch adds up.  Items go
// longest first so that long chunks start before short lists.
void build_bwd(bsattn_layout* lay) {
    auto& bw = lay->bwd;
    bw = bsattn_layout::Bwd{};
    const int32_t H = lay->H, nb = lay->nb;
    // transpose: for each (h, key block j) the query blocks i whose row holds j, ascending
    std::vector<int32_t> cptr((size_t)H * nb + 1, 0);
    for (int32_t h = 0; h < H; ++h)
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t r = h * nb + i;
            for (int32_t a = lay->row_ptr[r]; a < bwd_row_end(lay, r); ++a) ++cptr[(size_t)h * nb + lay->col_idx[a] + 1];
        }
    for (size_t c = 0; c + 1 < cptr.size(); ++c) cptr[c + 1] += cptr[c];
    bw.k_idx.assign((size_t)cptr.back(), 0);
    const bool subs = !lay->tile_sub.empty();
    if (subs) bw.k_sub.assign((size_t)cptr.back(), 0);
    std::vector<int32_t> fill(cptr.begin(), cptr.end() - 1);
    for (int32_t h = 0; h < H; ++h)
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t r = h * nb + i;
            for (int32_t a = lay->row_ptr[r]; a < bwd_row_end(lay, r); ++a) {
                const int32_t pos = fill[(size_t)h * nb + lay->col_idx[a]]++;
                bw.k_idx[(size_t)pos] = i;
                if (subs) bw.k_sub[(size_t)pos] = lay->tile_sub[(size_t)a];   // same bits: query half, key half
            }
        }
    // per head, longest first, padded with empty items (head_blk -1) to a common length
    // list hb is [begin(hb), end(hb)) of its index array
    auto make = [&](auto begin, auto end, std::vector<BwdItem>& items, std::vector<BwdSum>& sums,
                    int32_t& n_slots, int32_t& per_head) {
        n_slots = 0;
        std::vector<std::vector<BwdItem>> heads((size_t)H);
        for (int32_t hb = 0; hb < H * nb; ++hb) {
            auto& hi = heads[(size_t)(hb / nb)];
            const int32_t b0 = begin(hb), b1 = end(hb);
            const int32_t len = b1 - b0;
            if (len <= kChunkTiles) {
                hi.push_back({hb, b0, b1, -1});
                continue;
            }
            int32_t nch, per;
            split_row(len, &nch, &per);
            sums.push_back({hb, n_slots, nch, 0});
            for (int32_t c = 0; c < nch; ++c) {
                const int32_t s0 = b0 + c * per;
                hi.push_back({hb, s0, std::min(b1, s0 + per), n_slots++});
            }
        }
        per_head = 0;
        for (auto& hi : heads) {
            std::stable_sort(hi.begin(), hi.end(),
                             [](const BwdItem& x, const BwdItem& y) { return (x.end - x.begin) > (y.end - y.begin); });
            per_head = std::max<int32_t>(per_head, (int32_t)hi.size());
        }
        for (auto& hi : heads) {
            items.insert(items.end(), hi.begin(), hi.end());
            for (size_t a = hi.size(); a < (size_t)per_head; ++a) items.push_back({-1, 0, 0, -1});
        }
    };
    make([&](int32_t hb) { return lay->row_ptr[(size_t)hb]; }, [&](int32_t hb) { return bwd_row_end(lay, hb); },
         bw.q_items, bw.q_sums, bw.n_qslots, bw.q_per_head);
    make([&](int32_t hb) { return cptr[(size_t)hb]; }, [&](int32_t hb) { return cptr[(size_t)hb + 1]; }, bw.k_items,
         bw.k_sums, bw.n_kslots, bw.k_per_head);
    bw.built = true;
}

void free_bwd_device(bsattn_layout* lay) {
    auto& bw = lay->bwd;
    (void)hipFree(bw.d_q_items);
    (void)hipFree(bw.d_k_items);
    (void)hipFree(bw.d_q_sums);
    (void)hipFree(bw.d_k_sums);
    (void)hipFree(bw.d_k_idx);
    (void)hipFree(bw.d_k_sub);
    bw.d_q_items = bw.d_k_items = nullptr;
    bw.d_q_sums = bw.d_k_sums = nullptr;
    bw.d_k_idx = nullptr;
    bw.d_k_sub = nullptr;
    bw.uploaded = false;
    // the routed lists' host copies stay (a token layout's are built with it)
    for (auto& rb : lay->rbwd) {
        (void)hipFree(rb.d_rq_items);
        (void)hipFree(rb.d_k_items);
        (void)hipFree(rb.d_rq_sums);
        (void)hipFree(rb.d_k_sums);
        (void)hipFree(rb.d_k_idx);
        rb.d_rq_items = rb.d_k_items = nullptr;
        rb.d_rq_sums = rb.d_k_sums = nullptr;
        rb.d_k_idx = nullptr;
    }
    (void)hipFree(lay->d_tlink_ptr);
    (void)hipFree(lay->d_tlink_rows);
    lay->d_tlink_ptr = lay->d_tlink_rows = nullptr;
}

void free_device(bsattn_layout* lay) {
    if (lay->device >= 0) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != lay->device) (void)hipSetDevice(lay->device);
        (void)hipFree(lay->d_row_ptr);
        (void)hipFree(lay->d_col_idx);
        (void)hipFree(lay->d_col_sub);
        (void)hipFree(lay->d_gtok);
        (void)hipFree(lay->d_links);
        (void)hipFree(lay->d_tok_flag);
        (void)hipFree(lay->d_row_merge);
        (void)hipFree(lay->d_items);
        (void)hipFree(lay->d_merges);
        for (auto& sc : lay->scheds) {
            (void)hipFree(sc.d_units);
            (void)hipFree(sc.d_unit_ptr);
            (void)hipFree(sc.d_tiles);
            (void)hipFree(sc.d_tile_ptr);
            (void)hipFree(sc.d_wg_merge);
        }
        free_bwd_device(lay);
        if (cur >= 0 && cur != lay->device) (void)hipSetDevice(cur);
    }
    lay->scheds.clear();
    lay->d_row_ptr = lay->d_col_idx = nullptr;
    lay->d_col_sub = nullptr;
    lay->d_gtok = lay->d_links = nullptr;
    lay->d_tok_flag = nullptr;
    lay->d_row_merge = nullptr;
    lay->d_items = nullptr;
    lay->d_merges = nullptr;
    lay->device = -1;
}

bsattn_status check_layout_dims(int32_t H, int32_t L, int32_t block, bool any_block = false) {
    if (H < 1) return fail(BSATTN_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", H);
    if (block != kBlock && !(any_block && (block == kBlock / 2 || block == 2 * kBlock)))
        return fail(BSATTN_ERR_UNSUPPORTED, "block must be 64%s (got %d)", any_block ? ", 32 or 128" : "", block);
    if (L < kBlock || L % kBlock != 0 || L % block != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "seq_len must be a positive multiple of 64 and of block (got %d)", L);
    if ((int64_t)H * (L / kBlock) > (1 << 20) || L / kBlock > kTileJ + 1)
        return fail(BSATTN_ERR_UNSUPPORTED, "num_heads * seq_len/64 exceeds 2^20 or seq_len/64 exceeds 2^18");
    return BSATTN_OK;
}

void build_token_bwd(bsattn_layout* lay);

bsattn_status finish_layout(bsattn_layout* lay) {
    try {
        build_schedule(lay);
        if (lay->kind <= 2) build_bwd(lay);   // adaptive and top-keep layouts have no backward
        if (lay->kind == 2) build_token_bwd(lay);
    } catch (const std::bad_alloc&) {
        return fail(BSATTN_ERR_NO_MEMORY, "work list allocation failed");
    }
    return ok();
}

// Device copies of the backward lists (first backward call on the device).
bsattn_status upload_bwd(const bsattn_layout* lay, hipStream_t stream) {
    auto& bw = lay->bwd;
    if (bw.uploaded) return BSATTN_OK;
    void* p[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    const void* src[6] = {bw.q_items.data(), bw.k_items.data(), bw.q_sums.data(), bw.k_sums.data(),
                          bw.k_idx.data(), bw.k_sub.data()};
    const size_t sz[6] = {bw.q_items.size() * sizeof(BwdItem), bw.k_items.size() * sizeof(BwdItem),
                          bw.q_sums.size() * sizeof(BwdSum), bw.k_sums.size() * sizeof(BwdSum),
                          bw.k_idx.size() * sizeof(int32_t), bw.k_sub.size()};
    hipError_t e = hipSuccess;
    for (int a = 0; a < 6 && e == hipSuccess; ++a) {
        if (a == 5 && sz[a] == 0) break;   // no sub-block masks
        e = hipMalloc(&p[a], std::max<size_t>(sz[a], 16));
        if (e == hipSuccess && sz[a] > 0) e = hipMemcpyAsync(p[a], src[a], sz[a], hipMemcpyHostToDevice, stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        for (int a = 0; a < 6; ++a) (void)hipFree(p[a]);
        return fail(BSATTN_ERR_NO_MEMORY, "backward list upload: %s", hipGetErrorString(e));
    }
    if (lay->kind == 2) {   // token layouts: the transposed random-token lists
        void* tp = nullptr;
        void* tr = nullptr;
        const size_t np = lay->tlink_ptr.size() * sizeof(int32_t), nr = lay->tlink_rows.size() * sizeof(int32_t);
        e = hipMalloc(&tp, np);
        if (e == hipSuccess) e = hipMalloc(&tr, nr);
        if (e == hipSuccess) e = hipMemcpyAsync(tp, lay->tlink_ptr.data(), np, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(tr, lay->tlink_rows.data(), nr, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) {
            (void)hipFree(tp);
            (void)hipFree(tr);
            for (int a = 0; a < 6; ++a) (void)hipFree(p[a]);
            return fail(BSATTN_ERR_NO_MEMORY, "token backward list upload: %s", hipGetErrorString(e));
        }
        lay->d_tlink_ptr = (int32_t*)tp;
        lay->d_tlink_rows = (int32_t*)tr;
    }
    bw.d_q_items = (BwdItem*)p[0];
    bw.d_k_items = (BwdItem*)p[1];
    bw.d_q_sums = (BwdSum*)p[2];
    bw.d_k_sums = (BwdSum*)p[3];
    bw.d_k_idx = (int32_t*)p[4];
    bw.d_k_sub = (uint8_t*)p[5];
    bw.uploaded = true;
    return BSATTN_OK;
}

// Backward lists of a routed call with n_rt routed tiles per (b, h) on a band
// layout (or on a token layout's band, its global rows as the routed tiles).
// dQ: the band rows' items are the layout's own (lay->bwd); each routed tile
// r of head h adds r_chunks items over key blocks [c per, (c + 1)
// per), all written as partials after the band rows' slots, and one gathered
// sum.  dK/dV: every column lists the band's query blocks, then the routed
// tiles as entries nb + r; columns longer than kChunkTiles are split.  Per
// head, longest first, padded with empty items to a common length.
bsattn_layout::RoutedBwd build_routed_bwd(const bsattn_layout* lay, int32_t n_rt) {
    bsattn_layout::RoutedBwd rb;
    const int32_t H = lay->H, nb = lay->nb;
    rb.n_rt = n_rt;
    split_row(nb, &rb.r_chunks, &rb.per);
    rb.r_chunks = (nb + rb.per - 1) / rb.per;
    const int32_t base = lay->bwd.n_qslots;
    rb.n_qslots = base + H * n_rt * rb.r_chunks;
    rb.rq_per_head = n_rt * rb.r_chunks;
    for (int32_t h = 0; h < H; ++h)
        for (int32_t r = 0; r < n_rt; ++r) {
            const int32_t first = base + (h * n_rt + r) * rb.r_chunks;
            rb.rq_sums.push_back({h * nb + r, first, rb.r_chunks, 0});
            for (int32_t c = 0; c < rb.r_chunks; ++c)
                rb.rq_items.push_back({h * nb + r, c * rb.per, std::min(nb, (c + 1) * rb.per), first + c});
        }
    // columns: the band's CSC plus the routed tiles
    std::vector<int32_t> cptr((size_t)H * nb + 1, 0);
    for (int32_t h = 0; h < H; ++h)
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t r = h * nb + i;
            for (int32_t a = lay->row_ptr[r]; a < bwd_row_end(lay, r); ++a) ++cptr[(size_t)h * nb + lay->col_idx[a] + 1];
        }
    for (size_t c = 1; c < cptr.size(); ++c) cptr[c] += n_rt;
    for (size_t c = 0; c + 1 < cptr.size(); ++c) cptr[c + 1] += cptr[c];
    rb.k_idx.assign((size_t)cptr.back(), 0);
    std::vector<int32_t> fill(cptr.begin(), cptr.end() - 1);
    for (int32_t h = 0; h < H; ++h)
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t r = h * nb + i;
            for (int32_t a = lay->row_ptr[r]; a < bwd_row_end(lay, r); ++a)
                rb.k_idx[(size_t)fill[(size_t)h * nb + lay->col_idx[a]]++] = i;
        }
    for (size_t c = 0; c + 1 < cptr.size(); ++c)
        for (int32_t r = 0; r < n_rt; ++r) rb.k_idx[(size_t)fill[c]++] = nb + r;
    std::vector<std::vector<BwdItem>> heads((size_t)H);
    rb.n_kslots = 0;
    for (int32_t hb = 0; hb < H * nb; ++hb) {
        auto& hi = heads[(size_t)(hb / nb)];
        const int32_t b0 = cptr[(size_t)hb], b1 = cptr[(size_t)hb + 1], len = b1 - b0;
        if (len <= kChunkTiles) {
            hi.push_back({hb, b0, b1, -1});
            continue;
        }
        int32_t nch, per;
        split_row(len, &nch, &per);
        rb.k_sums.push_back({hb, rb.n_kslots, nch, 0});
        for (int32_t c = 0; c < nch; ++c) {
            const int32_t s0 = b0 + c * per;
            hi.push_back({hb, s0, std::min(b1, s0 + per), rb.n_kslots++});
        }
    }
    rb.k_per_head = 0;
    for (auto& hi : heads) {
        std::stable_sort(hi.begin(), hi.end(),
                         [](const BwdItem& x, const BwdItem& y) { return (x.end - x.begin) > (y.end - y.begin); });
        rb.k_per_head = std::max<int32_t>(rb.k_per_head, (int32_t)hi.size());
    }
    for (auto& hi : heads) {
        rb.k_items.insert(rb.k_items.end(), hi.begin(), hi.end());
        for (size_t a = hi.size(); a < (size_t)rb.k_per_head; ++a) rb.k_items.push_back({-1, 0, 0, -1});
    }
    return rb;
}

// Token layouts, backward: the global rows' routed lists (built with the
// layout, so that the workspace size is known before any device work), and
// for each (head, key s) the non-global rows whose random tokens hold s.
void build_token_bwd(bsattn_layout* lay) {
    const int32_t H = lay->H, L = lay->L, nl = lay->n_links;
    if (!lay->tok_g.empty()) lay->rbwd.push_back(build_routed_bwd(lay, lay->n_gt));
    lay->tlink_ptr.assign((size_t)H * (L + 1), 0);
    for (int32_t h = 0; h < H; ++h) {
        int32_t* ptr = lay->tlink_ptr.data() + (size_t)h * (L + 1);
        for (int32_t t = 0; t < L; ++t) {
            if (lay->tok_flag[(size_t)t]) continue;
            const int32_t* lk = lay->links.data() + ((size_t)h * L + t) * nl;
            for (int32_t j = 0; j < nl; ++j)
                if (lk[j] >= 0) ++ptr[lk[j] + 1];
        }
        for (int32_t s2 = 0; s2 < L; ++s2) ptr[s2 + 1] += ptr[s2];
    }
    // rows of head h are placed after those of heads < h
    size_t total = 0;
    for (int32_t h = 0; h < H; ++h) {
        int32_t* ptr = lay->tlink_ptr.data() + (size_t)h * (L + 1);
        const int32_t n = ptr[L];
        for (int32_t s2 = 0; s2 <= L; ++s2) ptr[s2] += (int32_t)total;
        total += (size_t)n;
    }
    lay->tlink_rows.assign(std::max<size_t>(total, 1), 0);
    std::vector<int32_t> fill(lay->tlink_ptr.size());
    std::copy(lay->tlink_ptr.begin(), lay->tlink_ptr.end(), fill.begin());
    for (int32_t h = 0; h < H; ++h)
        for (int32_t t = 0; t < L; ++t) {   // ascending t: each key's rows come out ascending
            if (lay->tok_flag[(size_t)t]) continue;
            const int32_t* lk = lay->links.data() + ((size_t)h * L + t) * nl;
            for (int32_t j = 0; j < nl; ++j)
                if (lk[j] >= 0) lay->tlink_rows[(size_t)fill[(size_t)h * (L + 1) + lk[j]]++] = t;
        }
}

// The routed lists for n_rt tiles, built and uploaded on first use (caller holds sched_mu).
bsattn_status get_routed_bwd(const bsattn_layout* lay, int32_t n_rt, hipStream_t stream,
                             const bsattn_layout::RoutedBwd** out) {
    bsattn_layout::RoutedBwd* found = nullptr;
    for (auto& rb : lay->rbwd)
        if (rb.n_rt == n_rt) found = &rb;
    if (found && found->d_rq_items) {
        *out = found;
        return BSATTN_OK;
    }
    if (g_no_build) return fail(BSATTN_ERR_STATE, "routed backward lists were not prepared with bsattn_prepare");
    bsattn_layout::RoutedBwd built;
    if (!found) {
        try {
            built = build_routed_bwd(lay, n_rt);
        } catch (const std::bad_alloc&) {
            return fail(BSATTN_ERR_NO_MEMORY, "routed backward list allocation failed");
        }
    }
    bsattn_layout::RoutedBwd& rb = found ? *found : built;   // host lists (a token layout builds them up front)
    void* p[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    const void* src[5] = {rb.rq_items.data(), rb.k_items.data(), rb.rq_sums.data(), rb.k_sums.data(),
                          rb.k_idx.data()};
    const size_t sz[5] = {rb.rq_items.size() * sizeof(BwdItem), rb.k_items.size() * sizeof(BwdItem),
                          rb.rq_sums.size() * sizeof(BwdSum), rb.k_sums.size() * sizeof(BwdSum),
                          rb.k_idx.size() * sizeof(int32_t)};
    hipError_t e = hipSuccess;
    for (int a = 0; a < 5 && e == hipSuccess; ++a) {
        e = hipMalloc(&p[a], std::max<size_t>(sz[a], 16));
        if (e == hipSuccess && sz[a] > 0) e = hipMemcpyAsync(p[a], src[a], sz[a], hipMemcpyHostToDevice, stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        for (int a = 0; a < 5; ++a) (void)hipFree(p[a]);
        return fail(BSATTN_ERR_NO_MEMORY, "routed backward list upload: %s", hipGetErrorString(e));
    }
    rb.d_rq_items = (BwdItem*)p[0];
    rb.d_k_items = (BwdItem*)p[1];
    rb.d_rq_sums = (BwdSum*)p[2];
    rb.d_k_sums = (BwdSum*)p[3];
    rb.d_k_idx = (int32_t*)p[4];
    if (found) {
        *out = found;
        return BSATTN_OK;
    }
    lay->rbwd.push_back(std::move(rb));
    *out = &lay->rbwd.back();
    return BSATTN_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of bsattn_backward_routed: delta, then the dQ (band and routed),
// dK and dV partial slots.
void routed_bwd_workspace_parts(const bsattn_layout* lay, int32_t B, int32_t D, int32_t n_qslots, int32_t n_kslots,
                                size_t* off_dq, size_t* off_dk, size_t* off_dv, size_t* total) {
    const size_t delta = align256((size_t)B * lay->H * lay->L * sizeof(float));
    const size_t qs = align256((size_t)B * n_qslots * kBlock * D * sizeof(float));
    const size_t ks = align256((size_t)B * n_kslots * kBlock * D * sizeof(float));
    *off_dq = delta;
    *off_dk = delta + qs;
    *off_dv = delta + qs + ks;
    *total = delta + qs + 2 * ks;
}

// Workspace of bsattn_backward: delta, then the dQ, dK and dV partial slots.
void bwd_workspace_parts(const bsattn_layout* lay, int32_t B, int32_t D, size_t* off_dq, size_t* off_dk,
                         size_t* off_dv, size_t* total) {
    const size_t delta = align256((size_t)B * lay->H * lay->L * sizeof(float));
    const size_t qs = align256((size_t)B * lay->bwd.n_qslots * kBlock * D * sizeof(float));
    const size_t ks = align256((size_t)B * lay->bwd.n_kslots * kBlock * D * sizeof(float));
    *off_dq = delta;
    *off_dk = delta + qs;
    *off_dv = delta + qs + ks;
    *total = delta + qs + 2 * ks;
}

// Workspace of the token-layout backward: the routed call's parts (delta, dQ,
// dK and dV slots; the global rows are the routed tiles), then the global
// keys' dK/dV chunk partials.  Row chunks per global key: enough workgroups
// (each takes tok_global_keys_per_wg keys) to fill the chip, at least 256
// rows each.
struct TokenBwdWs {
    size_t off_dq = 0, off_dk = 0, off_dv = 0, off_g = 0, total = 0;
    int32_t g_chunks = 0;
    int32_t n_qslots = 0, n_kslots = 0;
};
TokenBwdWs token_bwd_workspace(const bsattn_layout* lay, int32_t B, int32_t D) {
    TokenBwdWs w;
    const int32_t ng = (int32_t)lay->tok_g.size();
    w.n_qslots = lay->bwd.n_qslots;
    w.n_kslots = lay->bwd.n_kslots;
    for (const auto& rb : lay->rbwd)
        if (ng > 0 && rb.n_rt == lay->n_gt) {
            w.n_qslots = rb.n_qslots;
            w.n_kslots = rb.n_kslots;
        }
    routed_bwd_workspace_parts(lay, B, D, w.n_qslots, w.n_kslots, &w.off_dq, &w.off_dk, &w.off_dv, &w.total);
    if (ng > 0) {
        const int64_t keys = (int64_t)B * lay->H * ng;
        const int gk = tok_global_keys_per_wg(D);
        const int64_t wgs = (int64_t)B * lay->H * ((ng + gk - 1) / gk);
        w.g_chunks = (int32_t)std::max<int64_t>(1, std::min<int64_t>(lay->L / 256, (2048 + wgs - 1) / wgs));
        w.off_g = w.total;
        w.total += align256((size_t)keys * w.g_chunks * 2 * D * sizeof(float));
    }
    return w;
}

// Shape/pointer checks shared by both forward entry points.
bsattn_status check_forward_common(const bsattn_layout* lay, int32_t B, int32_t H, int32_t L,
                                   int32_t D, const void* q, const void* k, const void* v,
                                   void* out, float* lse, float scale) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (B < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", B);
    if (H != lay->H || L != lay->L)
        return fail(BSATTN_ERR_INVALID_ARG, "H=%d L=%d do not match the layout (H=%d L=%d)", H, L,
                    lay->H, lay->L);
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    if (!q || !k || !v || !out || !lse) return fail(BSATTN_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
        return fail(BSATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (out == q || out == k || out == v) return fail(BSATTN_ERR_INVALID_ARG, "out aliases an input");
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(BSATTN_ERR_INVALID_ARG, "scale must be positive and finite");
    if ((int64_t)B * H * L * D >= (int64_t)1 << 40)
        return fail(BSATTN_ERR_UNSUPPORTED, "tensor too large");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (lay->device < 0 || lay->device != dev)
        return fail(BSATTN_ERR_STATE, "layout is not uploaded to the current device (%d)", dev);
    return BSATTN_OK;
}

size_t slot_bytes(int32_t D) { return (size_t)kBlock * (size_t)(D + 1) * sizeof(float); }

void routed_split(int32_t nb, int32_t k, int32_t* n_rt, int32_t* r_chunks, int32_t* per) {
    *n_rt = (k + kBlock - 1) / kBlock;
    split_row(nb, r_chunks, per);
    *r_chunks = (nb + *per - 1) / *per;
}

// Workspace of a forward over a token layout: the partial slots of every row
// and of the global rows' routed chunks (fp32 O, then LSE), then the
// gathered K and V tiles of the global tokens.
struct TokenWs {
    size_t slots, kg, vg, total;
    int32_t n_rt, r_chunks, per;
};
TokenWs token_workspace(const bsattn_layout* lay, int32_t B, int32_t D) {
    TokenWs w{};
    const int32_t ng = (int32_t)lay->tok_g.size();
    w.n_rt = 0;
    w.r_chunks = 1;
    w.per = 1;
    if (ng > 0) routed_split(lay->nb, ng, &w.n_rt, &w.r_chunks, &w.per);
    w.slots = (size_t)B * lay->n_slots + (size_t)B * lay->H * w.n_rt * w.r_chunks;
    const size_t gbytes = (size_t)B * lay->H * lay->n_gt * kBlock * D * 2;
    w.kg = align256(w.slots * slot_bytes(D));
    w.vg = w.kg + align256(gbytes);
    w.total = w.vg + align256(gbytes);
    return w;
}

// Workspace of a forward over a content-adaptive layout: the partial slots of
// split rows (fp32 O, then LSE), the block sums of q and k (fp64), the kept key
// blocks [B*H][nb][keep], and the filled schedule tile entries (one per tile).
struct AdaptiveWs {
    size_t qs, ks, cols, live, total;
};
AdaptiveWs adaptive_workspace(const bsattn_layout* lay, int32_t B, int32_t D) {
    AdaptiveWs w{};
    const size_t G = (size_t)B * lay->H;
    const int32_t keep = lay->rule.r;
    w.qs = align256((size_t)B * lay->n_slots * slot_bytes(D));
    w.ks = w.qs + align256(G * lay->nb * D * sizeof(double));
    w.cols = w.ks + align256(G * lay->nb * D * sizeof(double));
    w.live = w.cols + align256(G * lay->nb * keep * sizeof(int32_t));
    w.total = w.live + align256(G * lay->nb * keep * sizeof(int32_t));
    return w;
}

// Workgroups of the bf16 kernel that one device holds at once (CUs x
// resident workgroups per CU), cached per device and head width.
int device_capacity(int dev, int32_t D, int* cus_out = nullptr, bool two_wave = false) {
    static std::mutex mu;
    static std::vector<int> cache, cus_cache;   // index 3 * dev + (D == 128 ? 1 : two_wave ? 2 : 0)
    std::lock_guard<std::mutex> g(mu);
    const size_t idx = 3 * (size_t)dev + (D == 128 ? 1 : two_wave ? 2 : 0);
    if (cache.size() <= idx) {
        cache.resize(idx + 1, 0);
        cus_cache.resize(idx + 1, 0);
    }
    if (cache[idx] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 1;
        cus_cache[idx] = cus;
        cache[idx] = cus * fwd_bf16_ctas_per_cu(D, two_wave);
    }
    if (cus_out) *cus_out = cus_cache[idx];
    return cache[idx];
}

// Persistent schedule for one call shape.  Workgroup i runs on XCD i % 8
// (workgroups are dealt round-robin), and XCD x serves the (batch, head)
// groups g = x, x + 8, ...  The units of those groups -- each head's items
// (rows of at most kChunkTiles blocks, chunks of split rows) plus the routed
// chunks -- are packed into the XCD's n_bins bins longest-processing-time
// first: each unit, by decreasing cost, goes to the least loaded bin, cost =
// tile count + a fixed overhead for loading Q and writing O.  n_bins is the
// number of lists per XCD that the device runs at once: one per workgroup
// (D = 128), or one per wave of the CU-wide workgroups (D = 64).  Within a bin
// the units are then ordered by group, so that all bins of an XCD walk its
// groups in the same order and the XCD's K/V working set stays near one
// group (which fits in its L2).  For every bin the device gets the unit
// records and the flat list of the units' key blocks in order, at most
// max_bin_units units and max_bin_tiles tiles per bin.
}  // namespace

// The host half of a schedule: pure computation on the layout, no HIP call.
bsattn_status bsattn::pack_schedule(const bsattn_layout* lay, int32_t B, int32_t D, int32_t nru, int32_t rct,
                            int32_t r_chunks, int capacity, int cus, PackedSchedule* ps) {
    const int32_t ipH = lay->items_per_head;
    const int64_t G = (int64_t)B * lay->H;
    auto routed_len = [&](int32_t v) {
        const int32_t c = v % r_chunks;
        return std::min(lay->nb, c * rct + rct) - c * rct;
    };
    struct Unit {
        int32_t g, id, tiles, order;   // id >= 0: item position in the head; < 0: routed -1-v
    };
    // units of each XCD, in group order
    std::vector<std::vector<Unit>> xu((size_t)kXcds);
    for (int64_t g = 0; g < G; ++g) {
        auto& v = xu[(size_t)(g % kXcds)];
        const int32_t h = (int32_t)(g % lay->H);
        for (int32_t k = 0; k < ipH; ++k) {
            const WorkItem& wi = lay->items[(size_t)h * ipH + k];
            if (wi.row >= 0) v.push_back({(int32_t)g, k, wi.col_end - wi.col_begin, (int32_t)v.size()});
        }
        for (int32_t r = 0; r < nru; ++r) v.push_back({(int32_t)g, -1 - r, routed_len(r), (int32_t)v.size()});
    }
    // D = 64 runs one workgroup of kQWaves waves per CU, one list (bin) per
    // wave; D = 128 one list per workgroup.
    const bool per_wave = D == 64 && lay->kind != 4;   // top-keep layouts run the two-wave kernel
    const int32_t max_bin_units = kMaxBinUnits;
    const int32_t max_bin_tiles = kMaxBinTiles;
    int64_t need = 1;
    for (const auto& v : xu) {
        int64_t t = 0;
        for (const auto& u : v) t += u.tiles;
        need = std::max<int64_t>(need, ((int64_t)v.size() + max_bin_units - 1) / max_bin_units);
        need = std::max<int64_t>(need, (t + max_bin_tiles / 2 - 1) / (max_bin_tiles / 2));
    }
    size_t max_units = 1;
    for (const auto& v : xu) max_units = std::max(max_units, v.size());
    const int32_t cus_per_xcd = std::max(1, cus / kXcds);
    const int32_t lists_per_wg = per_wave ? kQWaves : 1;
    int64_t nb64 = std::max<int64_t>((int64_t)capacity * lists_per_wg / kXcds, need);
    nb64 = std::min<int64_t>(nb64, (int64_t)max_units);
    nb64 = (nb64 + lists_per_wg - 1) / lists_per_wg * lists_per_wg;   // whole workgroups
    if (nb64 * kXcds >= ((int64_t)1 << 31)) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    int32_t n_bins = (int32_t)std::max<int64_t>(nb64, 1);

    std::vector<int4> units;
    std::vector<int32_t> unit_ptr, tiles, tile_ptr, wg_merge;
    // Fused merges (D = 64): every split row has the same number n of chunks, n
    // divides kQWaves, and there are no routed units; each workgroup then
    // takes the chunks of kQWaves / n split rows (one chunk per wave list) and
    // merges those rows at its end.
    const int32_t fuse_n = lay->merges.empty() ? 0 : lay->merges.front().n_chunks;
    bool fuse = per_wave && nru == 0 && fuse_n >= 2 && kQWaves % fuse_n == 0 && lay->kind != 2;
    for (const auto& mi : lay->merges) fuse = fuse && mi.n_chunks == fuse_n;
    const int32_t rows_per_wg = fuse ? kQWaves / fuse_n : 1;
    // pack every XCD's units into nbins bins; false if some bin overflows its lists
    auto pack = [&](int32_t nbins) -> bool {
        units.clear();
        tiles.clear();
        unit_ptr.assign(1, 0);
        tile_ptr.assign(1, 0);
        const bool fuse_here = fuse && nbins == kQWaves * cus_per_xcd;
        wg_merge.assign(fuse_here ? (size_t)kXcds * cus_per_xcd * kQWaves : 0, -1);
        for (int32_t x = 0; x < kXcds; ++x) {
            const auto& v = xu[(size_t)x];
            std::vector<std::vector<int32_t>> bins((size_t)nbins);
            std::vector<int64_t> tiles_in((size_t)nbins, 0);
            std::vector<int32_t> order(v.size());
            for (size_t u = 0; u < v.size(); ++u) order[u] = (int32_t)u;
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t a2, int32_t b2) { return v[(size_t)a2].tiles > v[(size_t)b2].tiles; });
            using Load = std::pair<int64_t, int32_t>;   // (load, index), least loaded first, then lowest
            // Least-loaded-first packing of `items` (indices into v, by decreasing cost) into n slots.
            auto lpt = [&](const std::vector<int32_t>& items, int32_t n) {
                std::vector<std::vector<int32_t>> out((size_t)n);
                std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
                for (int32_t i = 0; i < n; ++i) heap.push({0, i});
                for (int32_t u : items) {
                    Load t = heap.top();
                    heap.pop();
                    out[(size_t)t.second].push_back(u);
                    heap.push({t.first + v[(size_t)u].tiles + 2, t.second});
                }
                return out;
            };
            if (nbins % cus_per_xcd == 0 && nbins > cus_per_xcd) {
                // Bins b, b + cus_per_xcd, b + 2 cus_per_xcd, ... of an XCD run on one
                // CU (workgroups of one CU, measured dispatch order; or the waves of
                // one workgroup), and they share its SIMDs: balance the work per CU
                // first, then split each CU's share -- in pairs of equal load when
                // the waves of a SIMD pair up (lists 2s and 2s + 1).  With fused
                // merges the first CUs each take the kQWaves chunks of one split row.
                std::vector<std::vector<int32_t>> per_cu;
                if (fuse_here) {
                    std::map<std::pair<int32_t, int32_t>, std::vector<int32_t>> rows;   // (g, merge) -> chunks
                    std::vector<int32_t> rest;
                    for (int32_t u : order) {
                        const Unit& un = v[(size_t)u];
                        const WorkItem& wi = lay->items[(size_t)(un.g % lay->H) * ipH + un.id];
                        if (wi.merge >= 0) rows[{un.g, wi.merge}].push_back(u);
                        else rest.push_back(u);
                    }
                    // every wave of a merging workgroup must hold a chunk: whole workgroups only
                    const int32_t wgs = (int32_t)rows.size() / rows_per_wg;
                    if ((int32_t)rows.size() % rows_per_wg != 0 || wgs >= cus_per_xcd) return false;
                    auto it = rows.begin();
                    for (int32_t w = 0; w < wgs; ++w) {
                        std::vector<int32_t> chunks;
                        for (int32_t r = 0; r < rows_per_wg; ++r, ++it) {
                            wg_merge[((size_t)x * cus_per_xcd + per_cu.size()) * kQWaves + r] =
                                (it->first.first / lay->H) * (int32_t)lay->merges.size() + it->first.second;
                            chunks.insert(chunks.end(), it->second.begin(), it->second.end());
                        }
                        per_cu.push_back(chunks);
                    }
                    const auto others = lpt(rest, cus_per_xcd - (int32_t)per_cu.size());
                    per_cu.insert(per_cu.end(), others.begin(), others.end());
                } else {
                    per_cu = lpt(order, cus_per_xcd);
                }
                const int32_t per = nbins / cus_per_xcd;
                const bool pairs = per_wave && per % 2 == 0;
                for (int32_t c = 0; c < cus_per_xcd; ++c) {
                    std::vector<std::vector<int32_t>> split;
                    if (pairs) {
                        for (const auto& pr : lpt(per_cu[(size_t)c], per / 2))
                            for (auto& one : lpt(pr, 2)) split.push_back(std::move(one));
                    } else {
                        split = lpt(per_cu[(size_t)c], per);
                    }
                    for (int32_t m = 0; m < per; ++m) bins[(size_t)(c + m * cus_per_xcd)] = split[(size_t)m];
                }
            } else {
                bins = lpt(order, nbins);
            }
            for (int32_t i = 0; i < nbins; ++i)
                for (int32_t u : bins[(size_t)i]) tiles_in[(size_t)i] += v[(size_t)u].tiles;
            for (int32_t i = 0; i < nbins; ++i)
                if (bins[(size_t)i].size() > (size_t)max_bin_units || tiles_in[(size_t)i] > max_bin_tiles) return false;
            for (auto& bn : bins) {
                std::sort(bn.begin(), bn.end(),
                          [&](int32_t a2, int32_t b2) { return v[(size_t)a2].order < v[(size_t)b2].order; });
                int32_t k = 0;
                const size_t bin_tile0 = tiles.size();
                for (int32_t u : bn) {
                    const Unit& un = v[(size_t)u];
                    const int32_t h = un.g % lay->H;
                    int32_t first = 0;
                    const bool routed = un.id < 0;
                    if (!routed) {
                        const WorkItem& wi = lay->items[(size_t)h * ipH + un.id];
                        units.push_back(make_int4(wi.row % lay->nb, wi.slot, un.g, (int32_t)(tiles.size() - bin_tile0)));
                        first = wi.col_begin;
                    } else {
                        const int32_t r = -1 - un.id;
                        units.push_back(make_int4(-1 - r / r_chunks, r % r_chunks, un.g, (int32_t)(tiles.size() - bin_tile0)));
                        first = (r % r_chunks) * rct;
                    }
                    for (int32_t t = 0; t < un.tiles; ++t) {
                        const int32_t j = routed ? first + t : lay->col_idx[(size_t)first + t];
                        const int32_t sub = (routed || lay->tile_sub.empty()) ? 15 : lay->tile_sub[(size_t)first + t];
                        tiles.push_back(j | (sub << kTileSubShift) | (k << kTileUnitShift) | (t == 0 ? kTileFirst : 0) |
                                        (t == un.tiles - 1 ? kTileLast : 0));
                    }
                    ++k;
                }
                unit_ptr.push_back((int32_t)units.size());
                tile_ptr.push_back((int32_t)tiles.size());
            }
        }
        return true;
    };
    if (fuse && !pack(n_bins)) fuse = false;   // fusion did not fit: the merge kernel merges
    while (!pack(n_bins)) {
        if ((size_t)n_bins >= max_units) return fail(BSATTN_ERR_UNSUPPORTED, "a unit exceeds the per-workgroup tile list");
        const int64_t nn = std::min<int64_t>((int64_t)max_units, (int64_t)n_bins * 2);
        n_bins = (int32_t)((nn + lists_per_wg - 1) / lists_per_wg * lists_per_wg);
    }
    if (wg_merge.empty()) fuse = false;
    if (units.empty()) units.push_back(make_int4(0, -1, 0, 0));
    if (tiles.empty()) tiles.push_back(0);
    if (!fuse) wg_merge.clear();
    ps->n_bins = n_bins;
    ps->units = std::move(units);
    ps->unit_ptr = std::move(unit_ptr);
    ps->tiles = std::move(tiles);
    ps->tile_ptr = std::move(tile_ptr);
    ps->wg_merge = std::move(wg_merge);
    return BSATTN_OK;
}

namespace {

bsattn_status get_schedule(const bsattn_layout* lay, int32_t B, int32_t D, int32_t nru, int32_t rct,
                           int32_t r_chunks, hipStream_t stream, bsattn_layout::Sched* out) {
    // a built schedule is looked up before anything else: this runs on every call
    std::lock_guard<std::mutex> guard(*lay->sched_mu);
    for (const auto& sc : lay->scheds)
        if (sc.batch == B && sc.head_dim == D && sc.nru == nru && sc.rct == rct) {
            *out = sc;
            return BSATTN_OK;
        }
    if (g_no_build)
        return fail(BSATTN_ERR_STATE, "call shape (batch %d, head_dim %d) was not prepared with bsattn_prepare", B, D);
    int cus = 1;
    const int capacity = device_capacity(lay->device, D, &cus, lay->kind == 4);
    PackedSchedule ps;
    bsattn_status st = pack_schedule(lay, B, D, nru, rct, r_chunks, capacity, cus, &ps);
    if (st != BSATTN_OK) return st;
    bsattn_layout::Sched sc{B, D, ps.n_bins, nru, rct, nullptr, nullptr, nullptr, nullptr, nullptr};
    void* p[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    const void* src[5] = {ps.units.data(), ps.unit_ptr.data(), ps.tiles.data(), ps.tile_ptr.data(),
                          ps.wg_merge.data()};
    const size_t sz[5] = {ps.units.size() * sizeof(int4), ps.unit_ptr.size() * sizeof(int32_t),
                          ps.tiles.size() * sizeof(int32_t), ps.tile_ptr.size() * sizeof(int32_t),
                          ps.wg_merge.size() * sizeof(int32_t)};
    hipError_t e = hipSuccess;
    for (int a = 0; a < 5 && e == hipSuccess; ++a) {
        if (sz[a] == 0) continue;
        e = hipMalloc(&p[a], sz[a]);
        if (e == hipSuccess) e = hipMemcpyAsync(p[a], src[a], sz[a], hipMemcpyHostToDevice, stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        for (int a = 0; a < 5; ++a) (void)hipFree(p[a]);
        return fail(BSATTN_ERR_NO_MEMORY, "schedule upload: %s", hipGetErrorString(e));
    }
    sc.d_units = (int4*)p[0];
    sc.d_unit_ptr = (int32_t*)p[1];
    sc.d_tiles = (int32_t*)p[2];
    sc.d_tile_ptr = (int32_t*)p[3];
    sc.d_wg_merge = (int32_t*)p[4];
    lay->scheds.push_back(sc);
    *out = sc;
    return BSATTN_OK;
}

// ---- attention layer ----

// rocBLAS handles, one per (thread, device); created on first use.
rocblas_handle blas_handle(int dev) {
    thread_local std::vector<rocblas_handle> handles;
    if (handles.size() <= (size_t)dev) handles.resize((size_t)dev + 1, nullptr);
    if (!handles[(size_t)dev] && rocblas_create_handle(&handles[(size_t)dev]) != rocblas_status_success)
        handles[(size_t)dev] = nullptr;
    return handles[(size_t)dev];
}

// Row-major C[M, N] (fp32) = A[M, K] (bf16) * W[N, K]^T (bf16): in rocBLAS's
// column-major terms C^T = W * A^T, i.e. op(W) = transpose, op(A) = none.
rocblas_status gemm_xwt(rocblas_handle h, const void* A, const void* W, float* C, int M, int N, int K) {
    const float one = 1.f, zero = 0.f;
    return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &one, W,
                           rocblas_datatype_bf16_r, K, A, rocblas_datatype_bf16_r, K, &zero, C,
                           rocblas_datatype_f32_r, N, C, rocblas_datatype_f32_r, N, rocblas_datatype_f32_r,
                           rocblas_gemm_algo_standard, 0, 0);
}

// Workspace of bsattn_layer_forward: [qkv32 | out32] [q | o2] [k] [v] [o] [lse] [attention workspace].
struct LayerWs {
    size_t qkv32, q, k, v, o, lse, attn, lt, total;
};
constexpr size_t kLtWorkspace = (size_t)32 << 20;   // hipBLASLt's workspace within the layer's
LayerWs layer_workspace(const bsattn_layout* lay, int32_t B, int32_t D, size_t attn_bytes) {
    const size_t rows = (size_t)B * lay->L;
    const size_t C = (size_t)lay->H * D;
    LayerWs w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    w.qkv32 = take(rows * 3 * C * sizeof(float));
    w.q = take(rows * C * 2);
    w.k = take(rows * C * 2);
    w.v = take(rows * C * 2);
    w.o = take(rows * C * 2);
    w.lse = take(rows * lay->H * sizeof(float));
    w.attn = take(attn_bytes);
    w.lt = take(kLtWorkspace);
    w.total = off;
    return w;
}

// hipBLASLt handles, one per (thread, device); created on first use.
hipblasLtHandle_t lt_handle(int dev) {
    thread_local std::vector<hipblasLtHandle_t> handles;
    if (handles.size() <= (size_t)dev) handles.resize((size_t)dev + 1, nullptr);
    if (!handles[(size_t)dev] && hipblasLtCreate(&handles[(size_t)dev]) != HIPBLAS_STATUS_SUCCESS)
        handles[(size_t)dev] = nullptr;
    return handles[(size_t)dev];
}

// One GEMM shape with a bias epilogue: row-major Y[M, N] (bf16) = X[M, K] (bf16)
// * W[N, K]^T (bf16) + bias[N] (bf16), fp32 accumulation, the bias added in
// fp32 and the sum rounded once.  In hipBLASLt's column-major terms
// Y^T = op(W) X^T with op = transpose, and the bias runs along Y^T's rows.
struct LtPlan {
    bool ok = false;
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ly = nullptr;
    hipblasLtMatmulAlgo_t algo{};
};

// The plan of (device, M, N, K), built on first use per thread; !ok when the
// library has no algorithm for it (the layer then takes its unfused path).
const LtPlan& lt_plan(int dev, int M, int N, int K) {
    thread_local std::map<std::tuple<int, int, int, int>, LtPlan> plans;
    auto key = std::make_tuple(dev, M, N, K);
    auto it = plans.find(key);
    if (it != plans.end()) return it->second;
    LtPlan p;
    hipblasLtHandle_t h = lt_handle(dev);
    bool good = h != nullptr;
    good = good && hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t tA = HIPBLAS_OP_T, tB = HIPBLAS_OP_N;
    const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
    const hipDataType bias_type = HIP_R_16BF;
    good = good && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &tA, sizeof(tA)) ==
                       HIPBLAS_STATUS_SUCCESS;
    good = good && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tB, sizeof(tB)) ==
                       HIPBLAS_STATUS_SUCCESS;
    good = good && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
                       HIPBLAS_STATUS_SUCCESS;
    good = good && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                                   sizeof(bias_type)) == HIPBLAS_STATUS_SUCCESS;
    // W as stored: column-major K x N (ld K); X^T: K x M (ld K); Y^T: N x M (ld N)
    good = good && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
    good = good && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
    good = good && hipblasLtMatrixLayoutCreate(&p.ly, HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS;
    if (good) {
        hipblasLtMatmulPreference_t pref = nullptr;
        const uint64_t ws = kLtWorkspace;
        good = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
               hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                     sizeof(ws)) == HIPBLAS_STATUS_SUCCESS;
        hipblasLtMatmulHeuristicResult_t res{};
        int found = 0;
        good = good && hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.ly, p.ly, pref, 1, &res, &found) ==
                           HIPBLAS_STATUS_SUCCESS && found > 0;
        if (good) p.algo = res.algo;
        if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
    }
    p.ok = good;
    return plans.emplace(key, p).first->second;
}

// Y = X W^T + bias through the plan; false when the plan is unusable.
bool lt_gemm_bias(int dev, const void* X, const void* W, const void* bias, void* Y, int M, int N, int K, void* ws,
                  hipStream_t stream) {
    const LtPlan& p = lt_plan(dev, M, N, K);
    if (!p.ok) return false;
    if (hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) !=
        HIPBLAS_STATUS_SUCCESS)
        return false;
    const float one = 1.f, zero = 0.f;
    return hipblasLtMatmul(lt_handle(dev), p.desc, &one, W, p.la, X, p.lb, &zero, Y, p.ly, Y, p.ly, &p.algo, ws,
                           kLtWorkspace, stream) == HIPBLAS_STATUS_SUCCESS;
}

// Forward over a token layout (bf16): the gathered global K/V tiles, then the
// attention kernel (band tiles and gathered tiles for every query block, the
// global rows as routed tiles over all keys), then the merge that adds each
// row's random tokens.  Every row goes through an fp32 partial and the merge.
bsattn_status token_forward(const bsattn_layout* lay, int32_t B, int32_t D, const void* q, const void* k,
                            const void* v, void* out, float* lse, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    const TokenWs w = token_workspace(lay, B, D);
    if (w.total > 0 && (!workspace || workspace_bytes < w.total))
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", w.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const int32_t ng = (int32_t)lay->tok_g.size();
    if ((int64_t)w.n_rt * w.r_chunks > (1 << 24)) return fail(BSATTN_ERR_UNSUPPORTED, "too many global tiles");
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.ws_o = (float*)workspace;
    a.ws_lse = a.ws_o + w.slots * kBlock * D;
    a.items = lay->d_items;
    a.merges = lay->d_merges;
    a.col_idx = lay->d_col_idx;
    a.valid_len = nullptr;
    a.routed_rows = lay->d_gtok;
    a.routed_stride = 0;   // one list of global rows for every (batch, head)
    a.n_items = (int32_t)lay->items.size();
    a.n_merges = (int32_t)lay->merges.size();
    a.items_per_head = lay->items_per_head;
    a.B = B; a.H = lay->H; a.L = lay->L; a.nb = lay->nb; a.n_slots = lay->n_slots;
    a.n_routed = ng; a.n_rt = w.n_rt; a.r_chunks = w.r_chunks; a.r_chunk_tiles = w.per;
    a.r_slot_base = B * lay->n_slots;
    a.band = lay->band_tokens;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.kg = (const uint16_t*)((char*)workspace + w.kg);
    a.vg = (const uint16_t*)((char*)workspace + w.vg);
    a.gtok = lay->d_gtok;
    a.n_gt = lay->n_gt;
    a.n_links = lay->n_links;
    a.links = lay->d_links;
    a.tok_global = lay->d_tok_flag;
    a.row_merge = lay->d_row_merge;

    bsattn_layout::Sched sc{};
    bsattn_status st = get_schedule(lay, B, D, w.n_rt * w.r_chunks, w.per, w.r_chunks, stream, &sc);
    if (st != BSATTN_OK) return st;
    a.n_bins = sc.n_bins;
    a.units = sc.d_units;
    a.unit_ptr = sc.d_unit_ptr;
    a.tiles = sc.d_tiles;
    a.tile_ptr = sc.d_tile_ptr;
    hipError_t e = launch_gather_global(a, D, stream);
    if (e != hipSuccess) return hip_fail(e, "global gather launch");
    e = launch_fwd_bf16(a, D, MASK_TOKEN, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "token forward launch");
    return ok();
}

// Forward over a content-adaptive layout (bf16): block sums of q and k and
// the kept key blocks of every query block (written to cols_out too when
// given), the schedule's tile entries filled with them, then the attention
// kernel and the merge of split rows.  With attend = false only the
// selection runs (cols_out required).
bsattn_status adaptive_run(const bsattn_layout* lay, int32_t B, int32_t D, const void* q, const void* k,
                           const void* v, void* out, float* lse, float scale, int32_t* cols_out, bool attend,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const AdaptiveWs w = adaptive_workspace(lay, B, D);
    if (!workspace || workspace_bytes < w.total)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", w.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    char* base = (char*)workspace;
    const int32_t keep = lay->rule.r;
    int32_t* cols = cols_out ? cols_out : (int32_t*)(base + w.cols);
    hipError_t e = launch_adaptive_select(q, k, (double*)(base + w.qs), (double*)(base + w.ks), cols, B * lay->H,
                                          lay->L, D, keep, stream);
    if (e != hipSuccess) return hip_fail(e, "adaptive selection launch");
    if (!attend) return ok();

    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.ws_o = (float*)workspace;
    a.ws_lse = a.ws_o + (size_t)B * lay->n_slots * kBlock * D;
    a.items = lay->d_items;
    a.merges = lay->d_merges;
    a.col_idx = lay->d_col_idx;
    a.n_items = (int32_t)lay->items.size();
    a.n_merges = (int32_t)lay->merges.size();
    a.items_per_head = lay->items_per_head;
    a.B = B; a.H = lay->H; a.L = lay->L; a.nb = lay->nb; a.n_slots = lay->n_slots;
    a.n_routed = 0; a.n_rt = 0; a.r_chunks = 1; a.r_chunk_tiles = 1; a.r_slot_base = 0;
    a.band = -1;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    bsattn_layout::Sched sc{};
    bsattn_status st = get_schedule(lay, B, D, 0, 1, 1, stream, &sc);
    if (st != BSATTN_OK) return st;
    int32_t* live = (int32_t*)(base + w.live);
    const int32_t n_lists = kXcds * sc.n_bins;
    e = launch_fill_tiles(sc.d_tiles, live, sc.d_units, sc.d_unit_ptr, sc.d_tile_ptr, n_lists, cols, lay->nb, keep,
                          stream);
    if (e != hipSuccess) return hip_fail(e, "tile fill launch");
    a.n_bins = sc.n_bins;
    a.units = sc.d_units;
    a.unit_ptr = sc.d_unit_ptr;
    a.tiles = live;
    a.tile_ptr = sc.d_tile_ptr;
    e = launch_fwd_bf16(a, D, MASK_NONE, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "adaptive forward launch");
    return ok();
}

bsattn_status adaptive_forward(const bsattn_layout* lay, int32_t B, int32_t D, const void* q, const void* k,
                               const void* v, void* out, float* lse, float scale, int32_t* cols_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return adaptive_run(lay, B, D, q, k, v, out, lse, scale, cols_out, true, workspace, workspace_bytes, stream);
}

// Workspace of a forward over a per-query top-keep layout: the partial slots
// of split rows (fp32 O, then LSE) and the kept-key words [B*H][L][nb].
struct ToprWs {
    size_t bits, total;
};
ToprWs topr_workspace(const bsattn_layout* lay, int32_t B, int32_t D) {
    ToprWs w{};
    w.bits = align256((size_t)B * lay->n_slots * slot_bytes(D));
    w.total = w.bits + align256((size_t)B * lay->H * lay->L * lay->nb * sizeof(uint64_t));
    return w;
}

// Forward over a per-query top-keep layout: the selection writes the kept-key
// words (to bits_out too when given), then the two-wave attention kernel runs
// every tile of the dense grid under that bit mask, then the merge of split
// rows.  With attend = false only the selection runs (bits_out required).
bsattn_status topr_run(const bsattn_layout* lay, int32_t B, int32_t D, const void* q, const void* k, const void* v,
                       void* out, float* lse, float scale, uint64_t* bits_out, bool attend, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    const ToprWs w = topr_workspace(lay, B, D);
    if (!workspace || workspace_bytes < w.total)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", w.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    char* base = (char*)workspace;
    uint64_t* bits = bits_out ? bits_out : (uint64_t*)(base + w.bits);
    // profile events time the selection, the kernel that dominates a top-keep forward
    hipError_t e = launch_topr_select(q, k, bits, B * lay->H, lay->L, D, lay->rule.r, stream, g_ev_before,
                                      g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "top-keep selection launch");
    if (!attend) return ok();
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.ws_o = (float*)workspace;
    a.ws_lse = a.ws_o + (size_t)B * lay->n_slots * kBlock * D;
    a.items = lay->d_items;
    a.merges = lay->d_merges;
    a.col_idx = lay->d_col_idx;
    a.n_items = (int32_t)lay->items.size();
    a.n_merges = (int32_t)lay->merges.size();
    a.items_per_head = lay->items_per_head;
    a.B = B; a.H = lay->H; a.L = lay->L; a.nb = lay->nb; a.n_slots = lay->n_slots;
    a.n_routed = 0; a.n_rt = 0; a.r_chunks = 1; a.r_chunk_tiles = 1; a.r_slot_base = 0;
    a.band = -1;
    a.keep_bits = bits;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    bsattn_layout::Sched sc{};
    bsattn_status st = get_schedule(lay, B, D, 0, 1, 1, stream, &sc);
    if (st != BSATTN_OK) return st;
    a.n_bins = sc.n_bins;
    a.units = sc.d_units;
    a.unit_ptr = sc.d_unit_ptr;
    a.tiles = sc.d_tiles;
    a.tile_ptr = sc.d_tile_ptr;
    a.wg_merge = nullptr;
    e = launch_fwd_bf16(a, D, MASK_BITS, stream, nullptr, nullptr);
    if (e != hipSuccess) return hip_fail(e, "top-keep forward launch");
    return ok();
}

// Backward over a token layout (bf16).  The band and the global rows run
// through the block passes as a routed call whose routed tiles are the global
// rows, one list shared by every (batch, head) group:
//   1. dQ of every row over its band tiles, and delta;
//   2. dQ of the global rows over every key block, summed into their rows;
//   3. dK and dV over the band's query blocks and the global rows' tiles
//      (outside the band);
//   4. the token kernels: each non-global row's global keys outside its band
//      and its random tokens, added to dQ, dK and dV.
bsattn_status token_backward(const bsattn_layout* lay, int32_t B, int32_t H, int32_t L, int32_t D, const void* q,
                             const void* k, const void* v, const void* out, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv, float scale, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    const TokenBwdWs w = token_bwd_workspace(lay, B, D);
    if (!workspace || workspace_bytes < w.total)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", w.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const int32_t ng = (int32_t)lay->tok_g.size();
    const auto& bw = lay->bwd;
    BwdItem *rq_items = nullptr, *k_items = bw.d_k_items;
    BwdSum *rq_sums = nullptr, *k_sums = bw.d_k_sums;
    int32_t* k_idx = bw.d_k_idx;
    int32_t n_rq_items = 0, n_rq_sums = 0, rq_per_head = 0;
    int32_t n_k_items = (int32_t)bw.k_items.size(), n_k_sums = (int32_t)bw.k_sums.size(), k_per_head = bw.k_per_head;
    {
        std::lock_guard<std::mutex> guard(*lay->sched_mu);
        bsattn_status st = upload_bwd(lay, stream);
        if (st != BSATTN_OK) return st;
        k_items = bw.d_k_items; k_sums = bw.d_k_sums; k_idx = bw.d_k_idx;
        if (ng > 0) {
            const bsattn_layout::RoutedBwd* rb = nullptr;
            st = get_routed_bwd(lay, lay->n_gt, stream, &rb);
            if (st != BSATTN_OK) return st;
            rq_items = rb->d_rq_items; rq_sums = rb->d_rq_sums;
            n_rq_items = (int32_t)rb->rq_items.size(); n_rq_sums = (int32_t)rb->rq_sums.size();
            rq_per_head = rb->rq_per_head;
            k_items = rb->d_k_items; k_sums = rb->d_k_sums; k_idx = rb->d_k_idx;
            n_k_items = (int32_t)rb->k_items.size(); n_k_sums = (int32_t)rb->k_sums.size();
            k_per_head = rb->k_per_head;
        }
    }
    if (((int64_t)B * H + kXcds) * std::max(std::max(bw.q_per_head, rq_per_head), std::max(k_per_head, L / 32)) >=
        ((int64_t)1 << 31))
        return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    char* ws = (char*)workspace;
    a.delta = (float*)ws;
    a.ws_dq = (float*)(ws + w.off_dq);
    a.ws_dk = (float*)(ws + w.off_dk);
    a.ws_dv = (float*)(ws + w.off_dv);
    a.valid_len = nullptr;
    a.B = B; a.H = H; a.L = L; a.nb = lay->nb;
    a.band = lay->band_tokens;
    a.routed_rows = lay->d_gtok;
    a.n_routed = ng;
    a.routed_stride = 0;   // one list of global rows for every (batch, head)
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.gtok = lay->d_gtok;
    a.n_g = ng;
    a.tok_global = lay->d_tok_flag;
    a.links = lay->d_links;
    a.n_links = lay->n_links;
    a.tptr = lay->d_tlink_ptr;
    a.trows = lay->d_tlink_rows;
    a.ws_g = ng > 0 ? (float*)(ws + w.off_g) : nullptr;
    a.g_chunks = w.g_chunks;
    hipError_t e;
    // 1. dQ of every row over its band (the global rows are redone below), and delta
    a.items = bw.d_q_items; a.n_items = (int32_t)bw.q_items.size(); a.items_per_head = bw.q_per_head;
    a.sums = bw.d_q_sums; a.n_sums = (int32_t)bw.q_sums.size();
    a.idx = lay->d_col_idx; a.idx_sub = nullptr; a.n_slots = w.n_qslots;
    if ((e = launch_bwd_dq(a, D, MASK_BAND, stream)) != hipSuccess) return hip_fail(e, "backward dQ launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 0, stream)) != hipSuccess)
        return hip_fail(e, "backward dQ sum launch");
    // 2. dQ of the global rows over every key block, as partials, summed into their rows
    if (ng > 0) {
        a.items = rq_items; a.n_items = n_rq_items; a.items_per_head = rq_per_head;
        a.sums = rq_sums; a.n_sums = n_rq_sums;
        a.idx = nullptr;
        if ((e = launch_bwd_dq(a, D, MASK_ROUTED_Q, stream)) != hipSuccess) return hip_fail(e, "global-row dQ launch");
        if ((e = launch_bwd_routed_sum(a, D, stream)) != hipSuccess) return hip_fail(e, "global-row dQ sum launch");
    }
    // 3. dK and dV over the band's query blocks (and the global rows' tiles)
    a.items = k_items; a.n_items = n_k_items; a.items_per_head = k_per_head;
    a.sums = k_sums; a.n_sums = n_k_sums;
    a.idx = k_idx; a.n_slots = w.n_kslots;
    if ((e = launch_bwd_dkdv(a, D, ng > 0 ? MASK_BAND_ROUTED : MASK_BAND, stream, g_ev_before, g_ev_after)) !=
        hipSuccess)
        return hip_fail(e, "token dK/dV launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 1, stream)) != hipSuccess)
        return hip_fail(e, "token dK/dV sum launch");
    // 4. the global keys outside each row's band and the random tokens
    if ((e = launch_tok_bwd_extra(a, D, stream)) != hipSuccess) return hip_fail(e, "token backward launch");
    return ok();
}

}  // namespace

namespace bsattn {

bsattn_status set_failure(bsattn_status st, const char* msg) { return fail(st, "%s", msg); }

bsattn_status forward_prepared_only(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B, int32_t H,
                                    int32_t L, int32_t D, const void* q, const void* k, const void* v,
                                    void* out, float* lse, const int32_t* key_valid_len, float scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    struct Guard {
        Guard() { g_no_build = true; }
        ~Guard() { g_no_build = false; }
    } guard;
    return bsattn_forward(lay, dtype, B, H, L, D, q, k, v, out, lse, key_valid_len, scale, workspace,
                          workspace_bytes, stream);
}

}  // namespace bsattn

extern "C" {

const char* bsattn_status_string(bsattn_status st) {
    switch (st) {
        case BSATTN_OK: return "ok";
        case BSATTN_ERR_INVALID_ARG: return "invalid argument";
        case BSATTN_ERR_UNSUPPORTED: return "unsupported";
        case BSATTN_ERR_HIP: return "HIP runtime error";
        case BSATTN_ERR_NO_MEMORY: return "out of memory";
        case BSATTN_ERR_STATE: return "layout not uploaded to this device";
    }
    return "unknown status";
}

const char* bsattn_last_error(void) { return g_error.c_str(); }

bsattn_status bsattn_make_layout(int32_t num_heads, int32_t seq_len, int32_t block,
                                 int32_t window_blocks, const int32_t* global_blocks,
                                 int32_t num_global, int32_t random_blocks, uint64_t seed,
                                 bsattn_layout** out) {
    if (!out) return fail(BSATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsattn_status st = check_layout_dims(num_heads, seq_len, block, true);
    if (st != BSATTN_OK) return st;
    const int32_t nb = seq_len / block;   // blocks of the rule (32, 64 or 128 tokens)
    if (window_blocks < 1 || window_blocks % 2 == 0)
        return fail(BSATTN_ERR_INVALID_ARG, "window_blocks must be odd and >= 1 (got %d)", window_blocks);
    if (window_blocks > kMaxWindowBlocks)
        return fail(BSATTN_ERR_UNSUPPORTED, "window_blocks > %d", kMaxWindowBlocks);
    if (num_global < 0 || num_global > kMaxGlobal)
        return fail(BSATTN_ERR_INVALID_ARG, "num_global must be in [0, %d] (got %d)", kMaxGlobal, num_global);
    if (num_global > 0 && !global_blocks) return fail(BSATTN_ERR_INVALID_ARG, "global_blocks is NULL");
    if (random_blocks < 0 || random_blocks > kMaxRandom)
        return fail(BSATTN_ERR_INVALID_ARG, "random_blocks must be in [0, %d] (got %d)", kMaxRandom,
                    random_blocks);
    RowRule rule{};
    rule.nb = nb;
    rule.wh = (window_blocks - 1) / 2;
    rule.r = random_blocks;
    rule.ng = num_global;
    rule.seed = seed;
    for (int32_t a = 0; a < num_global; ++a) {
        const int32_t g = global_blocks[a];
        if (g < 0 || g >= nb) return fail(BSATTN_ERR_INVALID_ARG, "global block %d out of [0, %d)", g, nb);
        rule.g[a] = g;
    }
    std::sort(rule.g, rule.g + num_global);
    for (int32_t a = 1; a < num_global; ++a)
        if (rule.g[a] == rule.g[a - 1]) return fail(BSATTN_ERR_INVALID_ARG, "duplicate global block %d", rule.g[a]);

    bsattn_layout* lay = new (std::nothrow) bsattn_layout();
    if (!lay) return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    try {
        // The rule runs on blocks of `block` tokens; the kernels walk 64-token
        // tiles, so a 128-token block (I, J) becomes the 2 x 2 tiles
        // (2I + a, 2J + b), rows and columns still ascending; a 32-token block
        // (I, J) is sub-block (I % 2, J % 2) of tile (I / 2, J / 2).
        const int32_t nt = seq_len / kBlock;
        if (block < kBlock) {
            lay->H = num_heads;
            lay->L = seq_len;
            lay->nb = nt;
            lay->block = block;
            lay->kind = 0;
            lay->rule = rule;
            lay->row_ptr.assign((size_t)num_heads * nt + 1, 0);
            std::vector<int32_t> r0, r1;
            std::vector<uint8_t> sub((size_t)nt);
            for (int32_t h = 0; h < num_heads; ++h)
                for (int32_t i = 0; i < nt; ++i) {
                    r0.assign((size_t)rule_row_count(rule, h, 2 * i), 0);
                    rule_row_fill(rule, h, 2 * i, r0.data());
                    r1.assign((size_t)rule_row_count(rule, h, 2 * i + 1), 0);
                    rule_row_fill(rule, h, 2 * i + 1, r1.data());
                    std::fill(sub.begin(), sub.end(), 0);
                    for (int32_t J : r0) sub[(size_t)(J / 2)] |= (uint8_t)(1u << (J % 2));
                    for (int32_t J : r1) sub[(size_t)(J / 2)] |= (uint8_t)(1u << (2 + J % 2));
                    int32_t n = 0;
                    for (int32_t j = 0; j < nt; ++j)
                        if (sub[(size_t)j]) {
                            lay->col_idx.push_back(j);
                            lay->tile_sub.push_back(sub[(size_t)j]);
                            ++n;
                        }
                    lay->row_ptr[(size_t)h * nt + i + 1] = lay->row_ptr[(size_t)h * nt + i] + n;
                }
            *out = lay;
            return finish_layout(lay);
        }
        const int32_t f = block / kBlock;
        lay->H = num_heads;
        lay->L = seq_len;
        lay->nb = nt;
        lay->block = block;
        lay->kind = 0;
        lay->rule = rule;
        std::vector<int32_t> cnt((size_t)num_heads * nb), buf;
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t i = 0; i < nb; ++i) cnt[(size_t)h * nb + i] = rule_row_count(rule, h, i);
        const int32_t rows = num_heads * nt;
        lay->row_ptr.assign((size_t)rows + 1, 0);
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t i = 0; i < nt; ++i) lay->row_ptr[(size_t)h * nt + i + 1] = f * cnt[(size_t)h * nb + i / f];
        for (int32_t r = 0; r < rows; ++r) lay->row_ptr[r + 1] += lay->row_ptr[r];
        lay->col_idx.assign((size_t)lay->row_ptr[rows], 0);
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t i = 0; i < nb; ++i) {
                buf.assign((size_t)cnt[(size_t)h * nb + i], 0);
                rule_row_fill(rule, h, i, buf.data());
                for (int32_t a = 0; a < f; ++a) {
                    int32_t* dst = lay->col_idx.data() + lay->row_ptr[(size_t)h * nt + f * i + a];
                    for (size_t c = 0; c < buf.size(); ++c)
                        for (int32_t b = 0; b < f; ++b) *dst++ = f * buf[c] + b;
                }
            }
    } catch (const std::bad_alloc&) {
        delete lay;
        return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    }
    *out = lay;
    return finish_layout(lay);
}

bsattn_status bsattn_make_band_layout(int32_t num_heads, int32_t seq_len, int32_t block,
                                      int32_t band_tokens, bsattn_layout** out) {
    if (!out) return fail(BSATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsattn_status st = check_layout_dims(num_heads, seq_len, block);
    if (st != BSATTN_OK) return st;
    if (band_tokens < 0 || band_tokens >= seq_len)
        return fail(BSATTN_ERR_INVALID_ARG, "band_tokens must be in [0, seq_len) (got %d)", band_tokens);
    const int32_t nb = seq_len / block;
    bsattn_layout* lay = new (std::nothrow) bsattn_layout();
    if (!lay) return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    try {
        lay->H = num_heads;
        lay->L = seq_len;
        lay->nb = nb;
        lay->block = block;
        lay->kind = 1;
        lay->band_tokens = band_tokens;
        lay->rule.nb = nb;
        const int32_t rows = num_heads * nb;
        lay->row_ptr.assign((size_t)rows + 1, 0);
        for (int32_t r = 0; r < rows; ++r)
            lay->row_ptr[r + 1] = lay->row_ptr[r] + band_row_fill(nb, block, band_tokens, r % nb, nullptr);
        lay->col_idx.assign((size_t)lay->row_ptr[rows], 0);
        for (int32_t r = 0; r < rows; ++r)
            band_row_fill(nb, block, band_tokens, r % nb, lay->col_idx.data() + lay->row_ptr[r]);
    } catch (const std::bad_alloc&) {
        delete lay;
        return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    }
    *out = lay;
    return finish_layout(lay);
}

bsattn_status bsattn_make_token_layout(int32_t num_heads, int32_t seq_len, int32_t band_tokens,
                                       int32_t num_global, int32_t random_tokens, uint64_t seed,
                                       bsattn_layout** out) {
    if (!out) return fail(BSATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsattn_status st = check_layout_dims(num_heads, seq_len, kBlock);
    if (st != BSATTN_OK) return st;
    if (band_tokens < 0 || band_tokens >= seq_len)
        return fail(BSATTN_ERR_INVALID_ARG, "band_tokens must be in [0, seq_len) (got %d)", band_tokens);
    if (num_global < 0 || num_global > seq_len)
        return fail(BSATTN_ERR_INVALID_ARG, "num_global must be in [0, seq_len] (got %d)", num_global);
    if (num_global > kMaxTokGlobal)
        return fail(BSATTN_ERR_UNSUPPORTED, "num_global exceeds %d", kMaxTokGlobal);
    if (random_tokens < 0 || random_tokens > kMaxLinks)
        return fail(BSATTN_ERR_INVALID_ARG, "random_tokens must be in [0, %d] (got %d)", kMaxLinks, random_tokens);
    if ((int64_t)num_heads * seq_len * random_tokens > ((int64_t)1 << 28))
        return fail(BSATTN_ERR_UNSUPPORTED, "num_heads * seq_len * random_tokens exceeds 2^28");
    const int32_t nb = seq_len / kBlock;
    if (nb + (num_global + kBlock - 1) / kBlock > kTileJ + 1)
        return fail(BSATTN_ERR_UNSUPPORTED, "seq_len too large for a token layout");
    bsattn_layout* lay = new (std::nothrow) bsattn_layout();
    if (!lay) return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    try {
        lay->H = num_heads;
        lay->L = seq_len;
        lay->nb = nb;
        lay->block = 1;
        lay->kind = 2;
        lay->band_tokens = band_tokens;
        lay->rule.nb = nb;
        lay->rule.seed = seed;
        lay->rule.r = random_tokens;
        // global tokens: floor(i (L - 1) / (n - 1)), distinct and ascending for n <= L
        for (int32_t i = 0; i < num_global; ++i)
            lay->tok_g.push_back(num_global == 1 ? 0
                                                 : (int32_t)(((int64_t)i * (seq_len - 1)) / (num_global - 1)));
        lay->tok_flag.assign((size_t)seq_len, 0);
        for (int32_t g : lay->tok_g) lay->tok_flag[(size_t)g] = 1;
        lay->n_gt = (num_global + kBlock - 1) / kBlock;
        // random tokens of every row
        lay->n_links = random_tokens;
        lay->links.assign((size_t)num_heads * seq_len * random_tokens, -1);
        TokenRule tr{seq_len, band_tokens, random_tokens, seed, lay->tok_g.data(), num_global};
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t t = 0; t < seq_len; ++t)
                token_links_fill(tr, h, t, lay->links.data() + ((size_t)h * seq_len + t) * random_tokens);
        // tiles: the band's blocks, then the gathered global tiles
        const int32_t rows = num_heads * nb;
        lay->row_ptr.assign((size_t)rows + 1, 0);
        for (int32_t r = 0; r < rows; ++r)
            lay->row_ptr[r + 1] =
                lay->row_ptr[r] + band_row_fill(nb, kBlock, band_tokens, r % nb, nullptr) + lay->n_gt;
        lay->col_idx.assign((size_t)lay->row_ptr[rows], 0);
        for (int32_t r = 0; r < rows; ++r) {
            int32_t* dst = lay->col_idx.data() + lay->row_ptr[r];
            const int32_t n = band_row_fill(nb, kBlock, band_tokens, r % nb, dst);
            for (int32_t c = 0; c < lay->n_gt; ++c) dst[n + c] = nb + c;
        }
    } catch (const std::bad_alloc&) {
        delete lay;
        return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    }
    *out = lay;
    return finish_layout(lay);
}

bsattn_status bsattn_make_adaptive_layout(int32_t num_heads, int32_t seq_len, int32_t keep_blocks,
                                          bsattn_layout** out) {
    if (!out) return fail(BSATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsattn_status st = check_layout_dims(num_heads, seq_len, kBlock);
    if (st != BSATTN_OK) return st;
    const int32_t nb = seq_len / kBlock;
    if (nb > kMaxAdaptiveBlocks)
        return fail(BSATTN_ERR_UNSUPPORTED, "seq_len/64 exceeds %d for an adaptive layout", kMaxAdaptiveBlocks);
    if (keep_blocks < 1 || keep_blocks > nb)
        return fail(BSATTN_ERR_INVALID_ARG, "keep_blocks must be in [1, seq_len/64] (got %d)", keep_blocks);
    bsattn_layout* lay = new (std::nothrow) bsattn_layout();
    if (!lay) return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    try {
        lay->H = num_heads;
        lay->L = seq_len;
        lay->nb = nb;
        lay->block = kBlock;
        lay->kind = 3;
        lay->rule.nb = nb;
        lay->rule.r = keep_blocks;
        // Every row has the same length, so the split decides the balance alone:
        // chunks of up to 24 tiles keep the merge traffic down (each chunk is an
        // fp32 partial) while leaving several units per wave list.
        lay->chunk_tiles = 24;
        // every row holds keep_blocks tiles; the stored columns are positions
        // 0 .. keep_blocks - 1, replaced on the device by the chosen key blocks
        const int32_t rows = num_heads * nb;
        lay->row_ptr.assign((size_t)rows + 1, 0);
        lay->col_idx.assign((size_t)rows * keep_blocks, 0);
        for (int32_t r = 0; r < rows; ++r) {
            lay->row_ptr[r + 1] = (r + 1) * keep_blocks;
            for (int32_t p = 0; p < keep_blocks; ++p) lay->col_idx[(size_t)r * keep_blocks + p] = p;
        }
    } catch (const std::bad_alloc&) {
        delete lay;
        return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    }
    *out = lay;
    return finish_layout(lay);
}

bsattn_status bsattn_adaptive_select(const bsattn_layout* lay, int32_t B, int32_t H, int32_t L, int32_t D,
                                     const void* q, const void* k, int32_t* selected_blocks, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind != 3) return fail(BSATTN_ERR_INVALID_ARG, "not an adaptive layout");
    if (!selected_blocks) return fail(BSATTN_ERR_INVALID_ARG, "selected_blocks is NULL");
    if (B < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", B);
    if (H != lay->H || L != lay->L) return fail(BSATTN_ERR_INVALID_ARG, "H, L do not match the layout");
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    if (!q || !k) return fail(BSATTN_ERR_INVALID_ARG, "NULL tensor pointer");
    return adaptive_run(lay, B, D, q, k, nullptr, nullptr, nullptr, 1.f, selected_blocks, false, workspace,
                        workspace_bytes, stream);
}

bsattn_status bsattn_make_topr_layout(int32_t num_heads, int32_t seq_len, int32_t keep_tokens, bsattn_layout** out) {
    if (!out) return fail(BSATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    bsattn_status st = check_layout_dims(num_heads, seq_len, kBlock);
    if (st != BSATTN_OK) return st;
    if (seq_len > kMaxTopLen)
        return fail(BSATTN_ERR_UNSUPPORTED, "seq_len exceeds %d for a top-keep layout", kMaxTopLen);
    if (keep_tokens < 1 || keep_tokens > seq_len)
        return fail(BSATTN_ERR_INVALID_ARG, "keep_tokens must be in [1, seq_len] (got %d)", keep_tokens);
    bsattn_layout* lay = new (std::nothrow) bsattn_layout();
    if (!lay) return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    try {
        const int32_t nb = seq_len / kBlock;
        lay->H = num_heads;
        lay->L = seq_len;
        lay->nb = nb;
        lay->block = kBlock;
        lay->kind = 4;
        lay->rule.nb = nb;
        lay->rule.r = keep_tokens;
        // every query block meets every key block; the kept keys are a bit mask per call
        const int32_t rows = num_heads * nb;
        lay->row_ptr.assign((size_t)rows + 1, 0);
        lay->col_idx.assign((size_t)rows * nb, 0);
        for (int32_t r = 0; r < rows; ++r) {
            lay->row_ptr[r + 1] = (r + 1) * nb;
            for (int32_t j = 0; j < nb; ++j) lay->col_idx[(size_t)r * nb + j] = j;
        }
    } catch (const std::bad_alloc&) {
        delete lay;
        return fail(BSATTN_ERR_NO_MEMORY, "layout allocation failed");
    }
    *out = lay;
    return finish_layout(lay);
}

bsattn_status bsattn_topr_select(const bsattn_layout* lay, int32_t B, int32_t H, int32_t L, int32_t D, const void* q,
                                 const void* k, uint64_t* keep_bits, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind != 4) return fail(BSATTN_ERR_INVALID_ARG, "not a top-keep layout");
    if (!keep_bits) return fail(BSATTN_ERR_INVALID_ARG, "keep_bits is NULL");
    if (B < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", B);
    if (H != lay->H || L != lay->L) return fail(BSATTN_ERR_INVALID_ARG, "H, L do not match the layout");
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    if (!q || !k) return fail(BSATTN_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(keep_bits))
        return fail(BSATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    return topr_run(lay, B, D, q, k, nullptr, nullptr, nullptr, 1.f, keep_bits, false, workspace, workspace_bytes,
                    stream);
}

bsattn_status bsattn_layout_token_links(const bsattn_layout* lay, const int32_t** global_tokens,
                                        int32_t* num_global, const int32_t** links, int32_t* links_per_row) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind != 2) return fail(BSATTN_ERR_INVALID_ARG, "not a token layout");
    if (global_tokens) *global_tokens = lay->tok_g.empty() ? nullptr : lay->tok_g.data();
    if (num_global) *num_global = (int32_t)lay->tok_g.size();
    if (links) *links = lay->links.empty() ? nullptr : lay->links.data();
    if (links_per_row) *links_per_row = lay->n_links;
    return ok();
}

bsattn_status bsattn_layout_csr(const bsattn_layout* lay, const int32_t** row_ptr,
                                const int32_t** col_idx, int32_t* num_rows, int64_t* nnz) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (row_ptr) *row_ptr = lay->row_ptr.data();
    if (col_idx) *col_idx = lay->col_idx.data();
    if (num_rows) *num_rows = lay->H * lay->nb;
    if (nnz) *nnz = (int64_t)lay->col_idx.size();
    return ok();
}

bsattn_status bsattn_layout_tile_masks(const bsattn_layout* lay, const uint8_t** masks, int64_t* n) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (masks) *masks = lay->tile_sub.empty() ? nullptr : lay->tile_sub.data();
    if (n) *n = (int64_t)lay->tile_sub.size();
    return ok();
}

bsattn_status bsattn_layout_upload(bsattn_layout* lay, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    free_device(lay);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    const size_t nrp = lay->row_ptr.size() * sizeof(int32_t);
    const size_t ncol = std::max<size_t>(1, lay->col_idx.size()) * sizeof(int32_t);
    const size_t nit = std::max<size_t>(1, lay->items.size()) * sizeof(WorkItem);
    const size_t nmg = std::max<size_t>(1, lay->merges.size()) * sizeof(MergeItem);
    void* p[4] = {nullptr, nullptr, nullptr, nullptr};
    const size_t sz[4] = {nrp, ncol, nit, nmg};
    for (int a = 0; a < 4; ++a) {
        e = hipMalloc(&p[a], sz[a]);
        if (e != hipSuccess) {
            for (int c = 0; c < a; ++c) (void)hipFree(p[c]);
            return fail(BSATTN_ERR_NO_MEMORY, "hipMalloc of %zu bytes failed: %s", sz[a], hipGetErrorString(e));
        }
    }
    lay->device = dev;
    lay->d_row_ptr = (int32_t*)p[0];
    lay->d_col_idx = (int32_t*)p[1];
    lay->d_items = (WorkItem*)p[2];
    lay->d_merges = (MergeItem*)p[3];
    const void* src[4] = {lay->row_ptr.data(), lay->col_idx.data(), lay->items.data(), lay->merges.data()};
    const size_t cp[4] = {nrp, lay->col_idx.size() * sizeof(int32_t), lay->items.size() * sizeof(WorkItem),
                          lay->merges.size() * sizeof(MergeItem)};
    for (int a = 0; a < 4; ++a) {
        if (cp[a] == 0) continue;
        e = hipMemcpyAsync(p[a], src[a], cp[a], hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) {
            free_device(lay);
            return hip_fail(e, "hipMemcpyAsync (layout upload)");
        }
    }
    if (lay->kind == 2) {
        std::vector<int32_t> gpad((size_t)std::max(1, lay->n_gt * kBlock), -1);
        std::copy(lay->tok_g.begin(), lay->tok_g.end(), gpad.begin());
        const size_t nl = std::max<size_t>(1, lay->links.size());
        e = hipMalloc(&lay->d_gtok, gpad.size() * sizeof(int32_t));
        if (e == hipSuccess) e = hipMalloc(&lay->d_links, nl * sizeof(int32_t));
        if (e == hipSuccess) e = hipMalloc(&lay->d_tok_flag, lay->tok_flag.size());
        if (e == hipSuccess) e = hipMalloc(&lay->d_row_merge, lay->row_merge.size() * sizeof(int32_t));
        if (e == hipSuccess)
            e = hipMemcpyAsync(lay->d_row_merge, lay->row_merge.data(), lay->row_merge.size() * sizeof(int32_t),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(lay->d_gtok, gpad.data(), gpad.size() * sizeof(int32_t), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess && !lay->links.empty())
            e = hipMemcpyAsync(lay->d_links, lay->links.data(), lay->links.size() * sizeof(int32_t),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(lay->d_tok_flag, lay->tok_flag.data(), lay->tok_flag.size(), hipMemcpyHostToDevice,
                               stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);   // gpad is a local
        if (e != hipSuccess) {
            free_device(lay);
            return fail(BSATTN_ERR_NO_MEMORY, "token layout upload: %s", hipGetErrorString(e));
        }
    }
    if (!lay->tile_sub.empty()) {
        e = hipMalloc(&lay->d_col_sub, lay->tile_sub.size());
        if (e == hipSuccess)
            e = hipMemcpyAsync(lay->d_col_sub, lay->tile_sub.data(), lay->tile_sub.size(), hipMemcpyHostToDevice,
                               stream);
        if (e != hipSuccess) {
            free_device(lay);
            return fail(BSATTN_ERR_NO_MEMORY, "sub-block mask upload: %s", hipGetErrorString(e));
        }
    }
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        free_device(lay);
        return hip_fail(e, "hipStreamSynchronize (layout upload)");
    }
    return ok();
}

bsattn_status bsattn_layout_build_device(const bsattn_layout* lay, int32_t* row_ptr_dev,
                                         int32_t* col_idx_dev, uint8_t* tile_masks_dev, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (!row_ptr_dev || (!col_idx_dev && !lay->col_idx.empty()))
        return fail(BSATTN_ERR_INVALID_ARG, "NULL device array");
    if (lay->kind != 0 && lay->kind != 1)
        return fail(BSATTN_ERR_UNSUPPORTED, "the device rule builds window/global/random and band layouts only");
    int kind = lay->kind;
    if (lay->kind == 0 && lay->block == 32) {
        if (!tile_masks_dev && !lay->col_idx.empty())
            return fail(BSATTN_ERR_INVALID_ARG, "a layout of 32-token blocks needs tile_masks_dev");
        kind = 2;
    } else if (lay->kind == 0 && lay->block == 128) {
        kind = 3;
    } else if (lay->block != kBlock) {
        return fail(BSATTN_ERR_UNSUPPORTED, "the device rule runs 32-, 64- and 128-token blocks");
    }
    hipError_t e = launch_layout_build(lay->rule, kind, lay->H, lay->nb, lay->band_tokens,
                                       row_ptr_dev, col_idx_dev, tile_masks_dev, stream);
    if (e != hipSuccess) return hip_fail(e, "layout build launch");
    return ok();
}

void bsattn_layout_destroy(bsattn_layout* lay) {
    if (!lay) return;
    free_device(lay);
    delete lay;
}

bsattn_status bsattn_workspace_size(const bsattn_layout* lay, int32_t batch, int32_t head_dim,
                                    int32_t num_routed, size_t* bytes) {
    if (!lay || !bytes) return fail(BSATTN_ERR_INVALID_ARG, "NULL argument");
    if (batch < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (num_routed < 0 || num_routed > lay->L)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed must be in [0, seq_len]");
    if (lay->kind == 2) {
        *bytes = token_workspace(lay, batch, head_dim).total;
        return ok();
    }
    if (lay->kind == 3) {
        *bytes = adaptive_workspace(lay, batch, head_dim).total;
        return ok();
    }
    if (lay->kind == 4) {
        *bytes = topr_workspace(lay, batch, head_dim).total;
        return ok();
    }
    size_t slots = (size_t)batch * lay->n_slots;
    int32_t n_rt = 0;
    if (num_routed > 0) {
        int32_t rch, per;
        routed_split(lay->nb, num_routed, &n_rt, &rch, &per);
        slots += (size_t)batch * lay->H * n_rt * rch;
    }
    *bytes = slots * slot_bytes(head_dim);
    return ok();
}

bsattn_status bsattn_prepare(const bsattn_layout* lay, int32_t batch, int32_t head_dim, int32_t num_routed,
                             int32_t backward, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (batch < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (head_dim != 64 && head_dim != 128)
        return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
    if (num_routed < 0 || num_routed > lay->L)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed must be in [0, seq_len] (got %d)", num_routed);
    if (num_routed > 0 && lay->kind != 1)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed > 0 needs a band layout");
    if (backward && lay->kind != 0 && lay->kind != 1 && lay->kind != 2)
        return fail(BSATTN_ERR_UNSUPPORTED, "the backward takes window/global/random, band and token layouts");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (lay->device < 0 || lay->device != dev)
        return fail(BSATTN_ERR_STATE, "layout is not uploaded to the current device (%d)", dev);
    // the same schedule parameters the calls derive
    int32_t nru = 0, rct = 1, rch = 1;
    if (lay->kind == 2) {
        const TokenWs w = token_workspace(lay, batch, head_dim);
        nru = w.n_rt * w.r_chunks;
        rct = w.per;
        rch = w.r_chunks;
    } else if (num_routed > 0) {
        int32_t n_rt = 0, per = 1;
        routed_split(lay->nb, num_routed, &n_rt, &rch, &per);
        nru = n_rt * rch;
        rct = per;
    }
    bsattn_layout::Sched sc{};
    bsattn_status st = get_schedule(lay, batch, head_dim, nru, rct, rch, stream, &sc);
    if (st != BSATTN_OK) return st;
    if (backward) {
        std::lock_guard<std::mutex> guard(*lay->sched_mu);
        st = upload_bwd(lay, stream);
        if (st != BSATTN_OK) return st;
        if (num_routed > 0 || (lay->kind == 2 && !lay->tok_g.empty())) {   // the routed (global-row) lists
            const bsattn_layout::RoutedBwd* rb = nullptr;
            const int32_t n_rt = lay->kind == 2 ? lay->n_gt : (num_routed + kBlock - 1) / kBlock;
            st = get_routed_bwd(lay, n_rt, stream, &rb);
            if (st != BSATTN_OK) return st;
        }
    }
    return ok();
}

bsattn_status bsattn_candidate_positions(const void* x, const float* w, const float* bias, int32_t batch,
                                         int32_t seq_len, int32_t channels, int32_t num_candidates,
                                         int32_t* positions, hipStream_t stream) {
    if (!x || !w || !bias || !positions) return fail(BSATTN_ERR_INVALID_ARG, "NULL pointer");
    if (batch < 1 || seq_len < 1 || channels < 1)
        return fail(BSATTN_ERR_INVALID_ARG, "batch, seq_len and channels must be >= 1");
    if (num_candidates < 1 || num_candidates > kMaxCandidates)
        return fail(BSATTN_ERR_INVALID_ARG, "num_candidates must be in [1, %d] (got %d)", kMaxCandidates,
                    num_candidates);
    if ((reinterpret_cast<uintptr_t>(x) & 1u) || (reinterpret_cast<uintptr_t>(w) & 3u) ||
        (reinterpret_cast<uintptr_t>(bias) & 3u) || (reinterpret_cast<uintptr_t>(positions) & 3u))
        return fail(BSATTN_ERR_INVALID_ARG, "pointers must be aligned to their element size");
    if ((int64_t)batch * seq_len * std::max(channels, num_candidates) >= ((int64_t)1 << 40) ||
        (int64_t)batch * seq_len >= ((int64_t)1 << 31) / 4)
        return fail(BSATTN_ERR_UNSUPPORTED, "input too large");
    const hipError_t e = launch_cand_positions(x, w, bias, batch, seq_len, channels, num_candidates, positions,
                                               stream);
    if (e != hipSuccess) return hip_fail(e, "candidate positions launch");
    return ok();
}

bsattn_status bsattn_candidate_forward(bsattn_dtype dtype, int32_t B, int32_t H, int32_t L, int32_t D, const void* q,
                                       const void* k, const void* v, const int32_t* positions,
                                       int32_t num_candidates, int32_t keep, float scale, void* out, float* lse,
                                       int32_t* kept, hipStream_t stream) {
    if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "candidate attention is bf16 only");
    if (!q || !k || !v || !positions || !out || !lse) return fail(BSATTN_ERR_INVALID_ARG, "NULL pointer");
    if (B < 1 || H < 1 || L < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch, heads and seq_len must be >= 1");
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    if (num_candidates < 1 || num_candidates > kMaxCandidates)
        return fail(BSATTN_ERR_INVALID_ARG, "num_candidates must be in [1, %d] (got %d)", kMaxCandidates,
                    num_candidates);
    if (keep < 1 || keep > num_candidates)
        return fail(BSATTN_ERR_INVALID_ARG, "keep must be in [1, num_candidates] (got %d)", keep);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(BSATTN_ERR_INVALID_ARG, "scale must be > 0 and finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(positions) & 3u) ||
        (reinterpret_cast<uintptr_t>(kept) & 3u))
        return fail(BSATTN_ERR_INVALID_ARG, "q, k, v, out must be 16-byte aligned, the others 4-byte");
    const void* ins[4] = {q, k, v, positions};
    for (const void* in : ins)
        if (in == out || in == (const void*)lse || (kept && in == (const void*)kept))
            return fail(BSATTN_ERR_INVALID_ARG, "an output aliases an input");
    if (((int64_t)B * H * L + 3) / 4 >= ((int64_t)1 << 31)) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    const hipError_t e = launch_cand_attention(q, k, v, positions, B, H, L, D, num_candidates, keep, scale, out, lse,
                                               kept, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "candidate attention launch");
    return ok();
}

bsattn_status bsattn_set_profile_events(hipEvent_t before, hipEvent_t after) {
    if ((before == nullptr) != (after == nullptr))
        return fail(BSATTN_ERR_INVALID_ARG, "set both events or neither");
    g_ev_before = before;
    g_ev_after = after;
    return ok();
}

bsattn_status bsattn_forward(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B, int32_t H,
                             int32_t L, int32_t D, const void* q, const void* k, const void* v,
                             void* out, float* lse, const int32_t* key_valid_len, float scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    bsattn_status st = check_forward_common(lay, B, H, L, D, q, k, v, out, lse, scale);
    if (st != BSATTN_OK) return st;
    if (dtype != BSATTN_BF16 && dtype != BSATTN_F32) return fail(BSATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    const bool band = lay->kind == 1;   // token band |t - s| <= band_tokens (a token-granular window)
    if (band && dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "band layouts are bf16 only");
    if (band && key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "band layouts take no key padding");
    const bool sub = !lay->tile_sub.empty();   // 32-token blocks
    if (sub && dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "32-token layouts are bf16 only");
    if (sub && key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "32-token layouts take no key padding");
    if (lay->kind == 2) {
        if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "token layouts are bf16 only");
        if (key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "token layouts take no key padding");
        return token_forward(lay, B, D, q, k, v, out, lse, scale, workspace, workspace_bytes, stream);
    }
    if (lay->kind == 3) {
        if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "adaptive layouts are bf16 only");
        if (key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "adaptive layouts take no key padding");
        return adaptive_forward(lay, B, D, q, k, v, out, lse, scale, nullptr, workspace, workspace_bytes, stream);
    }
    if (lay->kind == 4) {
        if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "top-keep layouts are bf16 only");
        if (key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "top-keep layouts take no key padding");
        return topr_run(lay, B, D, q, k, v, out, lse, scale, nullptr, true, workspace, workspace_bytes, stream);
    }
    size_t need = 0;
    st = bsattn_workspace_size(lay, B, D, 0, &need);
    if (st != BSATTN_OK) return st;
    if (dtype == BSATTN_BF16 && need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }

    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    const size_t total_slots = (size_t)B * lay->n_slots;
    a.ws_o = workspace ? (float*)workspace : nullptr;
    a.ws_lse = workspace ? a.ws_o + total_slots * kBlock * D : nullptr;
    a.items = lay->d_items;
    a.merges = lay->d_merges;
    a.col_idx = lay->d_col_idx;
    a.valid_len = key_valid_len;
    a.routed_rows = nullptr;
    a.n_items = (int32_t)lay->items.size();
    a.n_merges = (int32_t)lay->merges.size();
    a.items_per_head = lay->items_per_head;
    a.B = B; a.H = H; a.L = L; a.nb = lay->nb; a.n_slots = lay->n_slots;
    a.n_routed = 0; a.n_rt = 0; a.r_chunks = 1; a.r_chunk_tiles = 1; a.r_slot_base = 0;
    a.routed_stride = 0;
    a.band = band ? lay->band_tokens : -1;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    const int mask = band ? MASK_BAND : (sub ? MASK_SUB : (key_valid_len ? MASK_PAD : MASK_NONE));
    a.strided = g_strides != nullptr && dtype == BSATTN_BF16;
    if (a.strided) {
        a.qkv_bs = g_strides->qkv_bs; a.qkv_hs = g_strides->qkv_hs; a.qkv_ts = g_strides->qkv_ts;
        a.o_bs = g_strides->o_bs; a.o_hs = g_strides->o_hs; a.o_ts = g_strides->o_ts;
    }

    hipError_t e;
    if (dtype == BSATTN_F32) {
        e = launch_fwd_f32(a, lay->d_row_ptr, D, mask, stream, g_ev_before, g_ev_after);
        if (e != hipSuccess) return hip_fail(e, "fp32 forward launch");
        return ok();
    }
    bsattn_layout::Sched sc{};
    st = get_schedule(lay, B, D, 0, 1, 1, stream, &sc);
    if (st != BSATTN_OK) return st;
    a.n_bins = sc.n_bins;
    a.units = sc.d_units;
    a.unit_ptr = sc.d_unit_ptr;
    a.tiles = sc.d_tiles;
    a.tile_ptr = sc.d_tile_ptr;
    // padding can empty a wave's list, and a workgroup that merges needs all its waves
    a.wg_merge = mask == MASK_PAD ? nullptr : sc.d_wg_merge;
    e = launch_fwd_bf16(a, D, mask, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "bf16 forward launch");
    return ok();
}

static bsattn_status check_route_shape(int32_t B, int32_t H, int32_t L, int32_t k) {
    if (B < 1 || H < 1 || L < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch, heads and seq_len must be >= 1");
    if (L > 8192) return fail(BSATTN_ERR_UNSUPPORTED, "seq_len > 8192 in the router");
    if (k < 1 || k > L) return fail(BSATTN_ERR_INVALID_ARG, "k must be in [1, seq_len] (got %d)", k);
    if ((int64_t)B * H * ((L + 63) / 64) > 0x7fffffff)
        return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    return BSATTN_OK;
}

bsattn_status bsattn_route_workspace_size(int32_t B, int32_t H, int32_t L, int32_t k, size_t* bytes) {
    if (!bytes) return fail(BSATTN_ERR_INVALID_ARG, "NULL argument");
    bsattn_status st = check_route_shape(B, H, L, k);
    if (st != BSATTN_OK) return st;
    *bytes = route_workspace_bytes(B, H, L, k);
    return ok();
}

bsattn_status bsattn_route_topk(const void* q, const float* w, int32_t B, int32_t H, int32_t L,
                                int32_t D, int32_t k, int32_t* routed_rows, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if (!q || !w || !routed_rows) return fail(BSATTN_ERR_INVALID_ARG, "NULL pointer");
    bsattn_status st = check_route_shape(B, H, L, k);
    if (st != BSATTN_OK) return st;
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    if (!aligned16(q)) return fail(BSATTN_ERR_INVALID_ARG, "q must be 16-byte aligned");
    const size_t need = route_workspace_bytes(B, H, L, k);
    if (!workspace || workspace_bytes < need)
        return fail(BSATTN_ERR_INVALID_ARG, "router workspace too small (need %zu bytes, got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    hipError_t e = launch_route_topk(q, w, B, H, L, D, k, routed_rows, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    return ok();
}

bsattn_status bsattn_forward_routed(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B,
                                    int32_t H, int32_t L, int32_t D, const void* q, const void* k,
                                    const void* v, const int32_t* routed_rows, int32_t num_routed,
                                    void* out, float* lse, float scale, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    bsattn_status st = check_forward_common(lay, B, H, L, D, q, k, v, out, lse, scale);
    if (st != BSATTN_OK) return st;
    if (lay->kind != 1) return fail(BSATTN_ERR_INVALID_ARG, "bsattn_forward_routed needs a band layout");
    if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the routed variant is bf16 only");
    if (num_routed < 1 || num_routed > L)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed must be in [1, seq_len] (got %d)", num_routed);
    if (!routed_rows) return fail(BSATTN_ERR_INVALID_ARG, "routed_rows is NULL");
    size_t need = 0;
    st = bsattn_workspace_size(lay, B, D, num_routed, &need);
    if (st != BSATTN_OK) return st;
    if (!workspace || workspace_bytes < need)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    int32_t n_rt, rch, per;
    routed_split(lay->nb, num_routed, &n_rt, &rch, &per);
    if ((int64_t)n_rt * rch > (1 << 24)) return fail(BSATTN_ERR_UNSUPPORTED, "too many routed tiles");

    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    const size_t total_slots = (size_t)B * lay->n_slots + (size_t)B * H * n_rt * rch;
    a.ws_o = (float*)workspace;
    a.ws_lse = a.ws_o + total_slots * kBlock * D;
    a.items = lay->d_items;
    a.merges = lay->d_merges;
    a.col_idx = lay->d_col_idx;
    a.valid_len = nullptr;
    a.routed_rows = routed_rows;
    a.n_items = (int32_t)lay->items.size();
    a.n_merges = (int32_t)lay->merges.size();
    a.items_per_head = lay->items_per_head;
    a.B = B; a.H = H; a.L = L; a.nb = lay->nb; a.n_slots = lay->n_slots;
    a.n_routed = num_routed; a.n_rt = n_rt; a.r_chunks = rch; a.r_chunk_tiles = per;
    a.routed_stride = num_routed;
    a.r_slot_base = B * lay->n_slots;
    a.band = lay->band_tokens;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;

    bsattn_layout::Sched sc{};
    st = get_schedule(lay, B, D, n_rt * rch, per, rch, stream, &sc);
    if (st != BSATTN_OK) return st;
    a.n_bins = sc.n_bins;
    a.units = sc.d_units;
    a.unit_ptr = sc.d_unit_ptr;
    a.tiles = sc.d_tiles;
    a.tile_ptr = sc.d_tile_ptr;
    hipError_t e = launch_fwd_bf16(a, D, MASK_BAND, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "routed forward launch");
    return ok();
}

bsattn_status bsattn_backward_workspace_size(const bsattn_layout* lay, int32_t batch, int32_t head_dim,
                                             size_t* bytes) {
    if (!lay || !bytes) return fail(BSATTN_ERR_INVALID_ARG, "NULL argument");
    if (batch < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (lay->kind == 2) {
        *bytes = token_bwd_workspace(lay, batch, head_dim).total;
        return ok();
    }
    size_t a, b, c;
    bwd_workspace_parts(lay, batch, head_dim, &a, &b, &c, bytes);
    return ok();
}


bsattn_status bsattn_backward(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B, int32_t H,
                              int32_t L, int32_t D, const void* q, const void* k, const void* v,
                              const void* out, const float* lse, const void* dout, void* dq, void* dk,
                              void* dv, const int32_t* key_valid_len, float scale, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind != 0 && lay->kind != 1 && lay->kind != 2)
        return fail(BSATTN_ERR_UNSUPPORTED, "the backward takes window/global/random, band and token layouts");
    if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the backward is bf16 only");
    const bool band = lay->kind == 1;
    if (band && key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "band layouts take no key padding");
    if (lay->kind == 2 && key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "token layouts take no key padding");
    if (!dout || !dq || !dk || !dv) return fail(BSATTN_ERR_INVALID_ARG, "NULL gradient pointer");
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(BSATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const void* ins[6] = {q, k, v, out, lse, dout};
    const void* outs[3] = {dq, dk, dv};
    for (const void* o : outs) {
        for (const void* in : ins)
            if (o == in) return fail(BSATTN_ERR_INVALID_ARG, "a gradient output aliases an input");
    }
    if (dq == dk || dq == dv || dk == dv) return fail(BSATTN_ERR_INVALID_ARG, "gradient outputs alias");
    const bool sub = !lay->tile_sub.empty();
    if (sub && key_valid_len) return fail(BSATTN_ERR_UNSUPPORTED, "32-token layouts take no key padding");
    // the forward's checks: shapes against the layout, q, k, v, out, lse, scale, the device
    bsattn_status st = check_forward_common(lay, B, H, L, D, q, k, v, const_cast<void*>(out),
                                            const_cast<float*>(lse), scale);
    if (st != BSATTN_OK) return st;
    if (lay->kind == 2)
        return token_backward(lay, B, H, L, D, q, k, v, out, lse, dout, dq, dk, dv, scale, workspace, workspace_bytes,
                              stream);
    size_t off_dq, off_dk, off_dv, need;
    bwd_workspace_parts(lay, B, D, &off_dq, &off_dk, &off_dv, &need);
    if (!workspace || workspace_bytes < need)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const auto& bw = lay->bwd;
    if (((int64_t)B * H + kXcds) * std::max(bw.q_per_head, bw.k_per_head) >= ((int64_t)1 << 31))
        return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    {
        std::lock_guard<std::mutex> guard(*lay->sched_mu);
        st = upload_bwd(lay, stream);
        if (st != BSATTN_OK) return st;
    }

    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    char* ws = (char*)workspace;
    a.delta = (float*)ws;
    a.ws_dq = (float*)(ws + off_dq);
    a.ws_dk = (float*)(ws + off_dk);
    a.ws_dv = (float*)(ws + off_dv);
    a.valid_len = key_valid_len;
    a.B = B; a.H = H; a.L = L; a.nb = lay->nb;
    a.band = band ? lay->band_tokens : 0;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    const int mask = band ? MASK_BAND : sub ? MASK_SUB : (key_valid_len ? MASK_PAD : MASK_NONE);

    // delta = rowsum(dO * O) is computed by the dQ pass (every query row has an
    // item there) and read by the dK/dV pass after it
    hipError_t e;
    a.items = bw.d_q_items; a.n_items = (int32_t)bw.q_items.size(); a.items_per_head = bw.q_per_head;
    a.sums = bw.d_q_sums; a.n_sums = (int32_t)bw.q_sums.size();
    a.idx = lay->d_col_idx; a.idx_sub = lay->d_col_sub; a.n_slots = bw.n_qslots;
    e = launch_bwd_dq(a, D, mask, stream);
    if (e != hipSuccess) return hip_fail(e, "backward dQ launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 0, stream)) != hipSuccess) return hip_fail(e, "backward dQ sum launch");

    a.items = bw.d_k_items; a.n_items = (int32_t)bw.k_items.size(); a.items_per_head = bw.k_per_head;
    a.sums = bw.d_k_sums; a.n_sums = (int32_t)bw.k_sums.size();
    a.idx = bw.d_k_idx; a.idx_sub = bw.d_k_sub; a.n_slots = bw.n_kslots;
    e = launch_bwd_dkdv(a, D, mask, stream, g_ev_before, g_ev_after);
    if (e != hipSuccess) return hip_fail(e, "backward dK/dV launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 1, stream)) != hipSuccess)
        return hip_fail(e, "backward dK/dV sum launch");
    return ok();
}

bsattn_status bsattn_backward_routed_workspace_size(const bsattn_layout* lay, int32_t batch, int32_t head_dim,
                                                    int32_t num_routed, size_t* bytes) {
    if (!lay || !bytes) return fail(BSATTN_ERR_INVALID_ARG, "NULL argument");
    if (lay->kind != 1) return fail(BSATTN_ERR_INVALID_ARG, "the routed backward needs a band layout");
    if (batch < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (num_routed < 1 || num_routed > lay->L)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed must be in [1, seq_len] (got %d)", num_routed);
    const int32_t n_rt = (num_routed + kBlock - 1) / kBlock;
    int32_t rch, per;
    split_row(lay->nb, &rch, &per);
    rch = (lay->nb + per - 1) / per;
    // column slots: count the split columns' chunks as the list builder does
    int32_t n_kslots = 0;
    std::vector<int32_t> len((size_t)lay->H * lay->nb, n_rt);
    for (int32_t r = 0; r < lay->H * lay->nb; ++r)
        for (int32_t a = lay->row_ptr[r]; a < lay->row_ptr[r + 1]; ++a)
            ++len[(size_t)(r / lay->nb) * lay->nb + lay->col_idx[a]];
    for (int32_t c : len)
        if (c > kChunkTiles) {
            int32_t nch, pc;
            split_row(c, &nch, &pc);
            n_kslots += nch;
        }
    const int32_t n_qslots = lay->bwd.n_qslots + lay->H * n_rt * rch;
    size_t a, b, c;
    routed_bwd_workspace_parts(lay, batch, head_dim, n_qslots, n_kslots, &a, &b, &c, bytes);
    return ok();
}

bsattn_status bsattn_backward_routed(const bsattn_layout* lay, bsattn_dtype dtype, int32_t B, int32_t H, int32_t L,
                                     int32_t D, const void* q, const void* k, const void* v, const void* out,
                                     const float* lse, const void* dout, const int32_t* routed_rows,
                                     int32_t num_routed, void* dq, void* dk, void* dv, float scale, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind != 1) return fail(BSATTN_ERR_INVALID_ARG, "bsattn_backward_routed needs a band layout");
    if (dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the backward is bf16 only");
    if (!routed_rows) return fail(BSATTN_ERR_INVALID_ARG, "routed_rows is NULL");
    if (num_routed < 1 || num_routed > L)
        return fail(BSATTN_ERR_INVALID_ARG, "num_routed must be in [1, seq_len] (got %d)", num_routed);
    if (!dout || !dq || !dk || !dv) return fail(BSATTN_ERR_INVALID_ARG, "NULL gradient pointer");
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(BSATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const void* ins[7] = {q, k, v, out, lse, dout, routed_rows};
    const void* outs[3] = {dq, dk, dv};
    for (const void* o : outs)
        for (const void* in : ins)
            if (o == in) return fail(BSATTN_ERR_INVALID_ARG, "a gradient output aliases an input");
    if (dq == dk || dq == dv || dk == dv) return fail(BSATTN_ERR_INVALID_ARG, "gradient outputs alias");
    bsattn_status st = check_forward_common(lay, B, H, L, D, q, k, v, const_cast<void*>(out),
                                            const_cast<float*>(lse), scale);
    if (st != BSATTN_OK) return st;
    size_t need = 0;
    st = bsattn_backward_routed_workspace_size(lay, B, D, num_routed, &need);
    if (st != BSATTN_OK) return st;
    if (!workspace || workspace_bytes < need)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const int32_t n_rt = (num_routed + kBlock - 1) / kBlock;
    const auto& bw = lay->bwd;
    // device lists copied out under the lock (later builds may move the cache)
    BwdItem *rq_items, *k_items;
    BwdSum *rq_sums, *k_sums;
    int32_t* k_idx;
    int32_t n_rq_items, n_rq_sums, rq_per_head, n_k_items, n_k_sums, k_per_head, n_qslots, n_kslots;
    {
        std::lock_guard<std::mutex> guard(*lay->sched_mu);
        st = upload_bwd(lay, stream);
        if (st != BSATTN_OK) return st;
        const bsattn_layout::RoutedBwd* rb = nullptr;
        st = get_routed_bwd(lay, n_rt, stream, &rb);
        if (st != BSATTN_OK) return st;
        rq_items = rb->d_rq_items; k_items = rb->d_k_items; rq_sums = rb->d_rq_sums; k_sums = rb->d_k_sums;
        k_idx = rb->d_k_idx;
        n_rq_items = (int32_t)rb->rq_items.size(); n_rq_sums = (int32_t)rb->rq_sums.size();
        rq_per_head = rb->rq_per_head;
        n_k_items = (int32_t)rb->k_items.size(); n_k_sums = (int32_t)rb->k_sums.size(); k_per_head = rb->k_per_head;
        n_qslots = rb->n_qslots; n_kslots = rb->n_kslots;
    }
    if (((int64_t)B * H + kXcds) * std::max(std::max(bw.q_per_head, rq_per_head), k_per_head) >= ((int64_t)1 << 31))
        return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
    size_t off_dq, off_dk, off_dv, total;
    routed_bwd_workspace_parts(lay, B, D, n_qslots, n_kslots, &off_dq, &off_dk, &off_dv, &total);

    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    char* ws = (char*)workspace;
    a.delta = (float*)ws;
    a.ws_dq = (float*)(ws + off_dq);
    a.ws_dk = (float*)(ws + off_dk);
    a.ws_dv = (float*)(ws + off_dv);
    a.valid_len = nullptr;
    a.B = B; a.H = H; a.L = L; a.nb = lay->nb;
    a.band = lay->band_tokens;
    a.routed_rows = routed_rows;
    a.n_routed = num_routed;
    a.routed_stride = num_routed;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    hipError_t e;
    // 1. dQ of every row over its band (routed rows are redone below), and delta
    a.items = bw.d_q_items; a.n_items = (int32_t)bw.q_items.size(); a.items_per_head = bw.q_per_head;
    a.sums = bw.d_q_sums; a.n_sums = (int32_t)bw.q_sums.size();
    a.idx = lay->d_col_idx; a.idx_sub = nullptr; a.n_slots = n_qslots;
    if ((e = launch_bwd_dq(a, D, MASK_BAND, stream)) != hipSuccess) return hip_fail(e, "backward dQ launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 0, stream)) != hipSuccess)
        return hip_fail(e, "backward dQ sum launch");
    // 2. dQ of the routed rows over every key block, as partials, summed into their rows
    a.items = rq_items; a.n_items = n_rq_items; a.items_per_head = rq_per_head;
    a.sums = rq_sums; a.n_sums = n_rq_sums;
    a.idx = nullptr;
    if ((e = launch_bwd_dq(a, D, MASK_ROUTED_Q, stream)) != hipSuccess) return hip_fail(e, "routed dQ launch");
    if ((e = launch_bwd_routed_sum(a, D, stream)) != hipSuccess) return hip_fail(e, "routed dQ sum launch");
    // 3. dK and dV over the band's query blocks and the routed tiles
    a.items = k_items; a.n_items = n_k_items; a.items_per_head = k_per_head;
    a.sums = k_sums; a.n_sums = n_k_sums;
    a.idx = k_idx; a.n_slots = n_kslots;
    if ((e = launch_bwd_dkdv(a, D, MASK_BAND_ROUTED, stream, g_ev_before, g_ev_after)) != hipSuccess)
        return hip_fail(e, "routed dK/dV launch");
    if (a.n_sums > 0 && (e = launch_bwd_sum(a, D, 1, stream)) != hipSuccess)
        return hip_fail(e, "routed dK/dV sum launch");
    return ok();
}

bsattn_status bsattn_layer_workspace_size(const bsattn_layout* lay, int32_t batch, int32_t head_dim,
                                          size_t* bytes) {
    if (!lay || !bytes) return fail(BSATTN_ERR_INVALID_ARG, "NULL argument");
    size_t attn = 0;
    bsattn_status st = bsattn_workspace_size(lay, batch, head_dim, 0, &attn);
    if (st != BSATTN_OK) return st;
    *bytes = layer_workspace(lay, batch, head_dim, attn).total;
    return ok();
}

bsattn_status bsattn_layer_forward(const bsattn_layout* lay, int32_t B, int32_t H, int32_t L, int32_t D,
                                   const void* x, const void* w_qkv, const void* b_qkv, const void* w_proj,
                                   const void* b_proj, void* out, const int32_t* key_valid_len, float scale,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!lay) return fail(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    if (lay->kind == 3 || lay->kind == 4)
        return fail(BSATTN_ERR_UNSUPPORTED,
                    "the layer takes block, band and token layouts (not adaptive or top-keep ones)");
    if (!x || !w_qkv || !b_qkv || !w_proj || !b_proj || !out) return fail(BSATTN_ERR_INVALID_ARG, "NULL pointer");
    const void* ps[6] = {x, w_qkv, b_qkv, w_proj, b_proj, out};
    for (const void* p : ps)
        if (!aligned16(p)) return fail(BSATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    if (out == x || out == w_qkv || out == b_qkv || out == w_proj || out == b_proj)
        return fail(BSATTN_ERR_INVALID_ARG, "out aliases an input");
    if (H != lay->H || L != lay->L) return fail(BSATTN_ERR_INVALID_ARG, "H=%d L=%d do not match the layout", H, L);
    if (B < 1) return fail(BSATTN_ERR_INVALID_ARG, "batch must be >= 1");
    if (D != 64 && D != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
    const int64_t rows = (int64_t)B * L, C = (int64_t)H * D;
    if (rows * 3 * C >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31))
        return fail(BSATTN_ERR_UNSUPPORTED, "layer too large for 32-bit GEMM sizes");
    size_t attn_bytes = 0;
    bsattn_status st = bsattn_workspace_size(lay, B, D, 0, &attn_bytes);
    if (st != BSATTN_OK) return st;
    const LayerWs w = layer_workspace(lay, B, D, attn_bytes);
    if (!workspace || workspace_bytes < w.total)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", w.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    rocblas_handle hb = blas_handle(dev);
    if (!hb) return fail(BSATTN_ERR_HIP, "rocblas_create_handle failed");
    if (rocblas_set_stream(hb, stream) != rocblas_status_success) return fail(BSATTN_ERR_HIP, "rocblas_set_stream failed");

    char* ws = (char*)workspace;
    float* qkv32 = (float*)(ws + w.qkv32);
    void *q = ws + w.q, *k = ws + w.k, *v = ws + w.v, *o = ws + w.o;
    float* lse = (float*)(ws + w.lse);
    if (lay->kind == 0 || lay->kind == 1) {
        // Fused path: the qkv GEMM adds b_qkv in its epilogue and writes bf16
        // token-major [B L, 3C] (into qkv32's space), the attention reads its
        // heads in place and writes O as the concatenated heads [B L, C] (into
        // q's space), and the output GEMM adds b_proj in its epilogue.
        uint16_t* qkv = (uint16_t*)qkv32;
        void* lt_ws = ws + w.lt;
        if (lt_gemm_bias(dev, x, w_qkv, b_qkv, qkv, (int)rows, (int)(3 * C), (int)C, lt_ws, stream)) {
            const LayerStrides ls{(int64_t)L * 3 * C, D, 3 * C, (int64_t)L * C, D, C};
            g_strides = &ls;
            st = bsattn_forward(lay, BSATTN_BF16, B, H, L, D, qkv, qkv + C, qkv + 2 * C, q, lse, key_valid_len,
                                scale, attn_bytes ? ws + w.attn : nullptr, attn_bytes, stream);
            g_strides = nullptr;
            if (st != BSATTN_OK) return st;
            if (!lt_gemm_bias(dev, q, w_proj, b_proj, out, (int)rows, (int)C, (int)C, lt_ws, stream))
                return fail(BSATTN_ERR_HIP, "output GEMM failed");
            return ok();
        }
    }
    // 1. qkv = x W_qkv^T (fp32), then + bias, rounded, split into heads
    if (gemm_xwt(hb, x, w_qkv, qkv32, (int)rows, (int)(3 * C), (int)C) != rocblas_status_success)
        return fail(BSATTN_ERR_HIP, "qkv GEMM failed");
    if ((e = launch_split_heads(qkv32, b_qkv, q, k, v, B, L, H, D, stream)) != hipSuccess)
        return hip_fail(e, "split heads launch");
    // 2. block-sparse attention
    st = bsattn_forward(lay, BSATTN_BF16, B, H, L, D, q, k, v, o, lse, key_valid_len, scale,
                        attn_bytes ? ws + w.attn : nullptr, attn_bytes, stream);
    if (st != BSATTN_OK) return st;
    // 3. heads concatenated (into q's space), out = o2 W_proj^T + bias (fp32 in qkv32's space)
    if ((e = launch_merge_heads(o, q, B, L, H, D, stream)) != hipSuccess) return hip_fail(e, "merge heads launch");
    if (gemm_xwt(hb, q, w_proj, qkv32, (int)rows, (int)C, (int)C) != rocblas_status_success)
        return fail(BSATTN_ERR_HIP, "output GEMM failed");
    if ((e = launch_bias_out(qkv32, b_proj, out, (size_t)rows, (int)C, stream)) != hipSuccess)
        return hip_fail(e, "output bias launch");
    return ok();
}

}  // extern "C"
