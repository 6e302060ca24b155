// schedule_check.cpp -- host test of the forward schedule packing and the
// host-only layout calls, built with AddressSanitizer and UndefinedBehavior-
// Sanitizer (tests/test_host_sanitize.py).  No GPU is touched: layouts are
// built on the host and pack_schedule is the pure host half of a schedule.
//
// For random layouts of every host-built kind (window/global/random rule at
// 32-, 64- and 128-token blocks, token bands with and without routed rows,
// token patterns), batch sizes, head widths and device sizes, it checks that
// the packed lists hold every unit of the call exactly once, on the XCD of
// its (batch, head) group, with its tiles in order and flagged first/last,
// within the per-list limits the kernels assume.
//
//   schedule_check [cases] [seed]     prints "OK <n> cases" and exits 0
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "internal.h"

using namespace bsattn;

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                     \
    do {                                                     \
        if (!(cond)) {                                       \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);               \
            std::fprintf(stderr, "\n");                      \
            ++g_fail;                                        \
            return false;                                    \
        }                                                    \
    } while (0)

struct Expected {
    int32_t g, kind, slot;
    std::vector<int32_t> tiles;   // key block | sub mask << 18
};

// Every unit a call (B, nru routed units of rct tiles in r_chunks chunks) must run.
std::vector<Expected> expected_units(const bsattn_layout* lay, int32_t B, int32_t nru, int32_t rct, int32_t r_chunks) {
    std::vector<Expected> out;
    const int32_t ipH = lay->items_per_head;
    for (int32_t g = 0; g < B * lay->H; ++g) {
        const int32_t h = g % lay->H;
        for (int32_t k = 0; k < ipH; ++k) {
            const WorkItem& wi = lay->items[(size_t)h * ipH + k];
            if (wi.row < 0) continue;
            Expected e{g, wi.row % lay->nb, wi.slot, {}};
            for (int32_t c = wi.col_begin; c < wi.col_end; ++c) {
                const int32_t sub = lay->tile_sub.empty() ? 15 : lay->tile_sub[(size_t)c];
                e.tiles.push_back(lay->col_idx[(size_t)c] | (sub << kTileSubShift));
            }
            out.push_back(e);
        }
        for (int32_t r = 0; r < nru; ++r) {
            const int32_t c = r % r_chunks;
            const int32_t len = std::min(lay->nb, c * rct + rct) - c * rct;
            Expected e{g, -1 - r / r_chunks, c, {}};
            for (int32_t t = 0; t < len; ++t) e.tiles.push_back((c * rct + t) | (15 << kTileSubShift));
            out.push_back(e);
        }
    }
    return out;
}

bool check_packed(const bsattn_layout* lay, int32_t B, int32_t D, int32_t nru, int32_t rct, int32_t r_chunks,
                  const PackedSchedule& ps, const char* tag) {
    const int32_t nl = kXcds * ps.n_bins;
    CHECK(ps.n_bins >= 1, "%s: n_bins %d", tag, ps.n_bins);
    CHECK(D != 64 || ps.n_bins % kQWaves == 0, "%s: D=64 bins %d not whole workgroups", tag, ps.n_bins);
    CHECK((int32_t)ps.unit_ptr.size() == nl + 1 && (int32_t)ps.tile_ptr.size() == nl + 1,
          "%s: pointer arrays %zu %zu for %d lists", tag, ps.unit_ptr.size(), ps.tile_ptr.size(), nl);
    CHECK(ps.unit_ptr[0] == 0 && ps.tile_ptr[0] == 0, "%s: pointers start at %d %d", tag, ps.unit_ptr[0],
          ps.tile_ptr[0]);
    std::map<std::tuple<int32_t, int32_t, int32_t>, std::vector<int32_t>> seen;
    for (int32_t i = 0; i < nl; ++i) {
        const int32_t x = i / ps.n_bins;
        const int32_t u0 = ps.unit_ptr[i], u1 = ps.unit_ptr[i + 1];
        const int32_t t0 = ps.tile_ptr[i], t1 = ps.tile_ptr[i + 1];
        CHECK(u0 <= u1 && t0 <= t1, "%s: list %d pointers not monotone", tag, i);
        CHECK(u1 <= (int32_t)ps.units.size() && t1 <= (int32_t)ps.tiles.size(), "%s: list %d past the arrays", tag, i);
        CHECK(u1 - u0 <= kMaxBinUnits, "%s: list %d holds %d units", tag, i, u1 - u0);
        CHECK(t1 - t0 <= kMaxBinTiles, "%s: list %d holds %d tiles", tag, i, t1 - t0);
        int32_t t = t0;
        for (int32_t u = u0; u < u1; ++u) {
            const int4 un = ps.units[(size_t)u];
            const int32_t k = u - u0;
            CHECK(un.z >= 0 && un.z < B * lay->H, "%s: list %d unit %d group %d", tag, i, k, un.z);
            CHECK(un.z % kXcds == x, "%s: group %d on XCD %d", tag, un.z, x);
            CHECK(un.w == t - t0, "%s: list %d unit %d starts at %d, tiles at %d", tag, i, k, un.w, t - t0);
            std::vector<int32_t> mine;
            while (t < t1 && ((ps.tiles[(size_t)t] >> kTileUnitShift) & (kMaxBinUnits - 1)) == k &&
                   (mine.empty() || !(ps.tiles[(size_t)t - 1] & kTileLast))) {
                const int32_t e = ps.tiles[(size_t)t];
                CHECK(((e & kTileFirst) != 0) == mine.empty(), "%s: first flag at tile %d", tag, t);
                mine.push_back(e & (kTileJ | (15 << kTileSubShift)));
                ++t;
            }
            CHECK(!mine.empty() && (ps.tiles[(size_t)t - 1] & kTileLast), "%s: unit without a last tile", tag);
            const auto key = std::make_tuple(un.z, un.x, un.y);
            CHECK(seen.find(key) == seen.end(), "%s: unit (g %d, kind %d, slot %d) twice", tag, un.z, un.x, un.y);
            seen[key] = mine;
        }
        CHECK(t == t1, "%s: list %d has %d tiles past its units", tag, i, t1 - t);
    }
    const auto want = expected_units(lay, B, nru, rct, r_chunks);
    CHECK(seen.size() == want.size(), "%s: %zu units packed, %zu expected", tag, seen.size(), want.size());
    for (const auto& e : want) {
        const auto it = seen.find(std::make_tuple(e.g, e.kind, e.slot));
        CHECK(it != seen.end(), "%s: unit (g %d, kind %d, slot %d) missing", tag, e.g, e.kind, e.slot);
        CHECK(it->second == e.tiles, "%s: unit (g %d, kind %d, slot %d) tiles differ", tag, e.g, e.kind, e.slot);
    }
    if (!ps.wg_merge.empty()) {
        CHECK(D == 64 && nru == 0, "%s: fused merges outside D = 64 block layouts", tag);
        std::set<int32_t> ids;
        for (int32_t v : ps.wg_merge) {
            if (v < 0) continue;
            CHECK(v < B * (int32_t)lay->merges.size(), "%s: merge id %d", tag, v);
            CHECK(ids.insert(v).second, "%s: merge id %d twice", tag, v);
        }
        CHECK((int32_t)ids.size() == B * (int32_t)lay->merges.size(), "%s: %zu of %zu split rows merged", tag,
              ids.size(), (size_t)B * lay->merges.size());
    }
    return true;
}

int pick(std::mt19937_64& rng, int lo, int hi) { return lo + (int)(rng() % (uint64_t)(hi - lo + 1)); }

}  // namespace

int main(int argc, char** argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 200;
    std::mt19937_64 rng(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345);
    const int dev_cus[] = {256, 304, 80, 8, 1};
    int done = 0;
    for (int c = 0; c < cases; ++c) {
        bsattn_layout* lay = nullptr;
        const int kind = c % 4;
        const int H = pick(rng, 1, 12);
        char tag[160];
        int32_t k_routed = 0;
        bsattn_status st = BSATTN_OK;
        if (kind == 0) {
            const int block = (int[]){32, 64, 128}[pick(rng, 0, 2)];
            const int nb = pick(rng, 1, block == 32 ? 160 : 96);
            const int w = 2 * pick(rng, 0, 3) + 1;
            std::vector<int32_t> gl;
            for (int j = 0; j < nb; ++j)
                if (rng() % 23 == 0) gl.push_back(j);
            const int r = pick(rng, 0, 3);
            st = bsattn_make_layout(H, nb * block, block, w, gl.data(), (int32_t)gl.size(), r, rng(), &lay);
            std::snprintf(tag, sizeof tag, "rule H%d L%d block%d w%d g%zu r%d", H, nb * block, block, w, gl.size(), r);
        } else if (kind == 1 || kind == 2) {
            const int nb = pick(rng, 1, 96);
            const int band = pick(rng, 0, kind == 1 ? 1200 : 128);
            st = bsattn_make_band_layout(H, nb * 64, 64, band, &lay);
            if (kind == 2) k_routed = pick(rng, 1, std::min(nb * 64, 200));
            std::snprintf(tag, sizeof tag, "band H%d L%d band%d routed%d", H, nb * 64, band, k_routed);
        } else {
            const int nb = pick(rng, 2, 64);
            const int band = pick(rng, 1, 256), ng = pick(rng, 0, 70), rt = pick(rng, 0, 8);
            st = bsattn_make_token_layout(H, nb * 64, band, ng, rt, rng(), &lay);
            std::snprintf(tag, sizeof tag, "token H%d L%d band%d g%d r%d", H, nb * 64, band, ng, rt);
        }
        if (st != BSATTN_OK) {
            // the rule can refuse a combination (e.g. more random blocks than free ones): skip it
            if (st != BSATTN_ERR_INVALID_ARG && st != BSATTN_ERR_UNSUPPORTED) {
                std::fprintf(stderr, "FAIL %s: make returned %d (%s)\n", tag, (int)st, bsattn_last_error());
                ++g_fail;
            }
            continue;
        }
        // the device rule's tile-row expansions (32- and 128-token blocks), run here on
        // the host, must give the host builder's CSR and quarter masks
        if (kind == 0 && (lay->block == 32 || lay->block == 128)) {
            std::vector<int32_t> cols((size_t)lay->nb * 2 + 8);
            std::vector<uint8_t> subs(cols.size());
            for (int32_t r = 0; r < lay->H * lay->nb && !g_fail; ++r) {
                const int32_t h = r / lay->nb, i = r % lay->nb;
                const int32_t n = lay->block == 32 ? sub_tile_row(lay->rule, h, i, cols.data(), subs.data())
                                                   : wide_tile_row_fill(lay->rule, h, i, cols.data());
                const int32_t cnt = lay->block == 32 ? sub_tile_row(lay->rule, h, i, nullptr, nullptr)
                                                     : wide_tile_row_fill(lay->rule, h, i, nullptr);
                bool same = n == cnt && n == lay->row_ptr[r + 1] - lay->row_ptr[r];
                for (int32_t a = 0; same && a < n; ++a) {
                    same = cols[(size_t)a] == lay->col_idx[(size_t)lay->row_ptr[r] + a];
                    if (lay->block == 32) same = same && subs[(size_t)a] == lay->tile_sub[(size_t)lay->row_ptr[r] + a];
                }
                if (!same) {
                    std::fprintf(stderr, "FAIL %s: device-rule tile row %d differs from the host layout\n", tag, r);
                    ++g_fail;
                }
            }
        }
        // host-only queries must hold together with the layout
        const int32_t* rp = nullptr;
        const int32_t* ci = nullptr;
        int32_t rows = 0;
        int64_t nnz = 0;
        if (bsattn_layout_csr(lay, &rp, &ci, &rows, &nnz) != BSATTN_OK || rows != lay->H * lay->nb ||
            rp[rows] != nnz) {
            std::fprintf(stderr, "FAIL %s: csr view\n", tag);
            ++g_fail;
        }
        const int B = pick(rng, 1, 5);
        const int D = rng() % 2 ? 64 : 128;
        int32_t nru = 0, rct = 1, rch = 1;
        if (lay->kind == 2) {
            const int32_t ng = (int32_t)lay->tok_g.size();
            if (ng > 0) {
                int32_t per = 0;
                split_row(lay->nb, &rch, &per);
                rch = (lay->nb + per - 1) / per;
                nru = ((ng + kBlock - 1) / kBlock) * rch;
                rct = per;
            }
        } else if (k_routed > 0) {
            int32_t per = 0;
            split_row(lay->nb, &rch, &per);
            rch = (lay->nb + per - 1) / per;
            nru = ((k_routed + kBlock - 1) / kBlock) * rch;
            rct = per;
        }
        size_t ws = 0;
        if (bsattn_workspace_size(lay, B, D, k_routed, &ws) != BSATTN_OK) {
            std::fprintf(stderr, "FAIL %s: workspace size (%s)\n", tag, bsattn_last_error());
            ++g_fail;
        }
        // the backward's host work lists (block and band layouts; others are refused)
        st = bsattn_backward_workspace_size(lay, B, D, &ws);
        if (st != BSATTN_OK && st != BSATTN_ERR_UNSUPPORTED) {
            std::fprintf(stderr, "FAIL %s: backward workspace size returned %d (%s)\n", tag, (int)st,
                         bsattn_last_error());
            ++g_fail;
        }
        const int cus = dev_cus[c % 5];
        const int capacity = cus * (D == 64 ? 1 : 2);
        PackedSchedule ps;
        char full[240];
        std::snprintf(full, sizeof full, "%s B%d D%d cus%d", tag, B, D, cus);
        st = pack_schedule(lay, B, D, nru, rct, rch, capacity, cus, &ps);
        if (st == BSATTN_OK) {
            if (check_packed(lay, B, D, nru, rct, rch, ps, full)) ++done;
        } else if (st != BSATTN_ERR_UNSUPPORTED) {
            std::fprintf(stderr, "FAIL %s: pack_schedule returned %d (%s)\n", full, (int)st, bsattn_last_error());
            ++g_fail;
        }
        bsattn_layout_destroy(lay);
    }
    if (g_fail) {
        std::fprintf(stderr, "%d failures\n", g_fail);
        return 1;
    }
    std::printf("OK %d cases\n", done);
    return 0;
}
