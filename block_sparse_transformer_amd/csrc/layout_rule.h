// layout_rule.h -- the per-row block rule, evaluated identically on host and device.
//
// BigBird page ("BigBird 稀疏注意力机制解析：如何突破 Transformer 的序列长度限制"),
// section 核心实现: global positions see and are seen by everything, a sliding
// window of neighbours, and random remote links.  Rows are block indices of
// 64-token blocks (SQA page, "Transformer计算效率优化：SQA稀疏注意力机制详解",
// sections 3.1 and 5).
//
// Row i of head h, for a non-global i:
//   E      = W(i) U G, W(i) = [max(0,i-wh), min(nb-1,i+wh)], G the global blocks
//   n      = nb - |E| candidates: the blocks outside E, in ascending order
//   take   = min(r, n) random blocks by a partial Fisher-Yates shuffle of the
//            candidates; draw j swaps positions j and j + (u_j mod (n-j)),
//            u_j = splitmix64 output j+1 from the row state
//            s = sm(sm(sm(seed) ^ h) ^ i), sm(x) = splitmix64 output 1 from x.
//   row    = sort(E U chosen).
// A global row is every block.  The shuffle is simulated sparsely: only the
// <= 2*take positions it touches are stored, and an untouched position p
// holds the p-th block outside E, so nothing of size nb is materialised.
//
// splitmix64: Steele, Lea & Flood, OOPSLA 2014 (state += golden gamma, then
// Stafford's Mix13 output function); arithmetic modulo 2^64.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSR_HD __host__ __device__
#else
#define BSR_HD
#endif

namespace bsattn {

constexpr int kMaxWindowBlocks = 63;
constexpr int kMaxGlobal = 64;
constexpr int kMaxRandom = 64;
constexpr int kMaxExcluded = kMaxWindowBlocks + kMaxGlobal;

constexpr uint64_t kGoldenGamma = 0x9E3779B97F4A7C15ull;

BSR_HD inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// First output of a splitmix64 generator in state x.
BSR_HD inline uint64_t splitmix_first(uint64_t x) { return mix64(x + kGoldenGamma); }

struct RowRule {
    int32_t nb;          // blocks per side
    int32_t wh;          // window half-width in blocks
    int32_t r;           // random blocks per row
    int32_t ng;          // number of global blocks
    uint64_t seed;
    int32_t g[kMaxGlobal];   // global blocks, ascending, distinct
};

BSR_HD inline bool rule_is_global(const RowRule& R, int32_t i) {
    for (int32_t a = 0; a < R.ng; ++a)
        if (R.g[a] == i) return true;
    return false;
}

// Ascending E = W(i) U G into e[]; returns |E|.
BSR_HD inline int32_t rule_excluded(const RowRule& R, int32_t i, int32_t* e) {
    const int32_t lo = i - R.wh < 0 ? 0 : i - R.wh;
    const int32_t hi = i + R.wh > R.nb - 1 ? R.nb - 1 : i + R.wh;
    int32_t n = 0, a = 0;
    int32_t w = lo;
    while (w <= hi || a < R.ng) {
        int32_t x;
        if (a >= R.ng || (w <= hi && w < R.g[a])) {
            x = w++;
        } else if (w > hi || R.g[a] < w) {
            x = R.g[a++];
        } else {            // equal
            x = w++;
            ++a;
        }
        e[n++] = x;
    }
    return n;
}

// p-th (0-based) block in [0, nb) outside the ascending set e[0..ne).
BSR_HD inline int32_t rule_select(const int32_t* e, int32_t ne, int32_t p) {
    int32_t x = p;
    for (int32_t a = 0; a < ne; ++a) {
        if (e[a] <= x) ++x;
        else break;
    }
    return x;
}

BSR_HD inline int32_t rule_row_count(const RowRule& R, int32_t h, int32_t i) {
    if (rule_is_global(R, i)) return R.nb;
    int32_t e[kMaxExcluded];
    const int32_t ne = rule_excluded(R, i, e);
    const int32_t n = R.nb - ne;
    return ne + (R.r < n ? R.r : n);
}

// Writes the ascending row into out[] (capacity rule_row_count) and returns its length.
BSR_HD inline int32_t rule_row_fill(const RowRule& R, int32_t h, int32_t i, int32_t* out) {
    if (rule_is_global(R, i)) {
        for (int32_t j = 0; j < R.nb; ++j) out[j] = j;
        return R.nb;
    }
    int32_t e[kMaxExcluded];
    const int32_t ne = rule_excluded(R, i, e);
    const int32_t n = R.nb - ne;
    const int32_t take = R.r < n ? R.r : n;

    // Sparse partial Fisher-Yates over candidate positions [0, n).
    int32_t pos[2 * kMaxRandom], val[2 * kMaxRandom];
    int32_t nmap = 0;
    int32_t chosen[kMaxRandom];
    uint64_t state = splitmix_first(splitmix_first(splitmix_first(R.seed) ^ (uint64_t)(uint32_t)h) ^
                                    (uint64_t)(uint32_t)i);
    for (int32_t j = 0; j < take; ++j) {
        state += kGoldenGamma;
        const uint64_t u = mix64(state);
        const int32_t t = j + (int32_t)(u % (uint64_t)(n - j));
        int32_t vj = -1, vt = -1, sj = -1, st = -1;
        for (int32_t a = 0; a < nmap; ++a) {
            if (pos[a] == j) sj = a;
            if (pos[a] == t) st = a;
        }
        vj = sj >= 0 ? val[sj] : rule_select(e, ne, j);
        vt = st >= 0 ? val[st] : rule_select(e, ne, t);
        // position j takes vt (final), position t takes vj
        if (sj < 0) { sj = nmap; pos[nmap] = j; ++nmap; }
        val[sj] = vt;
        if (t != j) {
            if (st < 0) { st = nmap; pos[nmap] = t; ++nmap; }
            val[st] = vj;
        }
        chosen[j] = vt;
    }
    // insertion sort of the chosen blocks (take <= 64)
    for (int32_t a = 1; a < take; ++a) {
        const int32_t x = chosen[a];
        int32_t b = a - 1;
        while (b >= 0 && chosen[b] > x) { chosen[b + 1] = chosen[b]; --b; }
        chosen[b + 1] = x;
    }
    // merge the two ascending, disjoint lists
    int32_t a = 0, c = 0, o = 0;
    while (a < ne || c < take) {
        if (c >= take || (a < ne && e[a] < chosen[c])) out[o++] = e[a++];
        else out[o++] = chosen[c++];
    }
    return o;
}

// Tile row i (64 tokens) of a rule on 32-token blocks: the tiles j that hold a
// block of rule row 2 i or 2 i + 1, ascending, each with its quarter bits (bit
// 2 a + b: query half a, key half b).  cols / subs may be null (count only).
// Returns the row length.
BSR_HD inline int32_t sub_tile_row(const RowRule& R, int32_t h, int32_t i, int32_t* cols, uint8_t* subs) {
    constexpr int32_t kCap = kMaxExcluded + kMaxRandom;   // bound on a non-global rule row
    int32_t l0[kCap], l1[kCap];
    const bool g0 = rule_is_global(R, 2 * i), g1 = rule_is_global(R, 2 * i + 1);
    const int32_t n0 = g0 ? R.nb : rule_row_fill(R, h, 2 * i, l0);
    const int32_t n1 = g1 ? R.nb : rule_row_fill(R, h, 2 * i + 1, l1);
    int32_t a0 = 0, a1 = 0, n = 0;
    while (a0 < n0 || a1 < n1) {
        const int32_t b0 = a0 < n0 ? (g0 ? a0 : l0[a0]) : 0x7fffffff;
        const int32_t b1 = a1 < n1 ? (g1 ? a1 : l1[a1]) : 0x7fffffff;
        const int32_t j = (b0 < b1 ? b0 : b1) / 2;
        int32_t sub = 0;
        while (a0 < n0 && (g0 ? a0 : l0[a0]) / 2 == j) { sub |= 1 << ((g0 ? a0 : l0[a0]) % 2); ++a0; }
        while (a1 < n1 && (g1 ? a1 : l1[a1]) / 2 == j) { sub |= 1 << (2 + (g1 ? a1 : l1[a1]) % 2); ++a1; }
        if (cols) {
            cols[n] = j;
            subs[n] = (uint8_t)sub;
        }
        ++n;
    }
    return n;
}

// Tile row i of a rule on 128-token blocks: rule row i / 2 with every block c
// spanning tiles 2 c and 2 c + 1 (expanded in place, from the back).  out may
// be null (count only).  Returns the row length.
BSR_HD inline int32_t wide_tile_row_fill(const RowRule& R, int32_t h, int32_t i, int32_t* out) {
    if (!out) return 2 * rule_row_count(R, h, i / 2);
    const int32_t n = rule_row_fill(R, h, i / 2, out);
    for (int32_t c = n - 1; c >= 0; --c) {
        const int32_t v = out[c];
        out[2 * c + 1] = 2 * v + 1;
        out[2 * c] = 2 * v;
    }
    return 2 * n;
}

// Token-granular pattern: the rule above on 1-token blocks (window [t-w, t+w]
// clipped, global tokens G of any number, r random tokens per non-global row
// from the same per-row stream with the token index in place of the block
// index).  The excluded set is one interval plus G, so the p-th candidate is
// found by binary search over G instead of from a materialised list.
struct TokenRule {
    int32_t L;           // tokens
    int32_t w;           // window half-width in tokens
    int32_t r;           // random tokens per row (<= kMaxRandom)
    uint64_t seed;
    const int32_t* g;    // global tokens, ascending, distinct
    int32_t ng;
};

// Number of global tokens < x.
BSR_HD inline int32_t token_g_below(const TokenRule& R, int32_t x) {
    int32_t lo = 0, hi = R.ng;
    while (lo < hi) {
        const int32_t mid = (lo + hi) / 2;
        if (R.g[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

BSR_HD inline bool token_is_global(const TokenRule& R, int32_t t) {
    const int32_t k = token_g_below(R, t);
    return k < R.ng && R.g[k] == t;
}

// The q-th (0-based) token outside G: q + k, k = #{i : g[i] - i <= q} (g[i] - i
// is non-decreasing for ascending distinct g).
BSR_HD inline int32_t token_nonglobal_select(const TokenRule& R, int32_t q) {
    int32_t lo = 0, hi = R.ng;
    while (lo < hi) {
        const int32_t mid = (lo + hi) / 2;
        if (R.g[mid] - mid <= q) lo = mid + 1;
        else hi = mid;
    }
    return q + lo;
}

// Random tokens of row t of head h, ascending, into out[] (capacity r);
// returns how many (0 for a global row).
BSR_HD inline int32_t token_links_fill(const TokenRule& R, int32_t h, int32_t t, int32_t* out) {
    if (token_is_global(R, t)) return 0;
    const int32_t lo = t - R.w < 0 ? 0 : t - R.w;
    const int32_t hi = t + R.w > R.L - 1 ? R.L - 1 : t + R.w;
    const int32_t before = lo - token_g_below(R, lo);            // candidates left of the window
    const int32_t upto = (hi + 1) - token_g_below(R, hi + 1);    // non-global tokens in [0, hi]
    const int32_t n = (R.L - R.ng) - (upto - before);
    const int32_t take = R.r < n ? R.r : n;
    auto cand = [&](int32_t p) {
        return token_nonglobal_select(R, p < before ? p : p - before + upto);
    };
    int32_t pos[2 * kMaxRandom], val[2 * kMaxRandom];
    int32_t nmap = 0;
    uint64_t state = splitmix_first(splitmix_first(splitmix_first(R.seed) ^ (uint64_t)(uint32_t)h) ^
                                    (uint64_t)(uint32_t)t);
    for (int32_t j = 0; j < take; ++j) {
        state += kGoldenGamma;
        const uint64_t u = mix64(state);
        const int32_t x = j + (int32_t)(u % (uint64_t)(n - j));
        int32_t sj = -1, sx = -1;
        for (int32_t a = 0; a < nmap; ++a) {
            if (pos[a] == j) sj = a;
            if (pos[a] == x) sx = a;
        }
        const int32_t vj = sj >= 0 ? val[sj] : cand(j);
        const int32_t vx = sx >= 0 ? val[sx] : cand(x);
        if (sj < 0) { sj = nmap; pos[nmap] = j; ++nmap; }
        val[sj] = vx;
        if (x != j) {
            if (sx < 0) { sx = nmap; pos[nmap] = x; ++nmap; }
            val[sx] = vj;
        }
        out[j] = vx;
    }
    for (int32_t a = 1; a < take; ++a) {   // insertion sort (take <= 64)
        const int32_t y = out[a];
        int32_t b = a - 1;
        while (b >= 0 && out[b] > y) { out[b + 1] = out[b]; --b; }
        out[b + 1] = y;
    }
    return take;
}

// Band layout: key blocks touched by |t - s| <= band for query block i.
BSR_HD inline int32_t band_row_fill(int32_t nb, int32_t block, int32_t band, int32_t i, int32_t* out) {
    const int32_t L = nb * block;
    int32_t lo_tok = i * block - band;
    int32_t hi_tok = i * block + block - 1 + band;
    if (lo_tok < 0) lo_tok = 0;
    if (hi_tok > L - 1) hi_tok = L - 1;
    int32_t o = 0;
    for (int32_t j = lo_tok / block; j <= hi_tok / block; ++j) {
        if (out) out[o] = j;
        ++o;
    }
    return o;
}

}  // namespace bsattn
