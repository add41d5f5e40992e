// Host check of the one-launch grid orders.  Every workgroup index of a
// launch goes through the decode the kernel runs (grid_order.hpp) with the
// arguments the C ABI plans (planning.hpp), and the check asks:
//   - coverage: every item of the launch is run by exactly one workgroup;
//   - order: every item comes after each item it waits for (the hardware
//     dispatches workgroups in index order, so waits on lower indices end);
//   - bounds: every index an item derives (sequence, row, chunk, workspace
//     word, first logit of its chunk) is inside its array.
// Prints "ok <cases>" and exits 0, or prints the first failures and exits 1.
// With argument N > 0 the check plants mistake N in the arguments it hands
// the decodes (never in the decodes themselves) and must then fail.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "grid_order.hpp"
#include "planning.hpp"

using namespace sv;

static long g_fail = 0, g_cases = 0;
static int g_mutant = 0;  // the planted mistake, 0 for none
#define CHECK(c, ...)                                                  \
    do {                                                               \
        if (!(c)) {                                                    \
            if (g_fail++ < 20) {                                       \
                fprintf(stderr, "FAIL line %d (%s): ", __LINE__, #c); \
                fprintf(stderr, __VA_ARGS__);                          \
                fputc('\n', stderr);                                   \
            }                                                          \
        }                                                              \
    } while (0)

// ------------------------------------------------------------------ fast division

static void check_fastdiv(std::mt19937_64 &rng) {
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + static_cast<uint32_t>(rng() % 0x7fffffffu));
    for (int e = 12; e < 31; ++e) {
        ds.push_back(1u << e);
        ds.push_back((1u << e) - 1);
        ds.push_back((1u << e) + 1);
    }
    for (uint32_t d : ds) {
        FastDiv f = make_fastdiv(d);
        if (g_mutant == 1 && d > 1) f.m -= 1;  // a multiplier one too small
        auto one = [&](uint64_t n) {
            if (n >= 0x80000000ull) return;
            const uint32_t q = fdiv(static_cast<uint32_t>(n), f);
            CHECK(q == n / d, "n=%llu d=%u got %u", static_cast<unsigned long long>(n), d, q);
        };
        for (uint64_t k : {0ull, 1ull, 2ull, 3ull, 1000ull, 0x7fffffffull / d, 0x7fffffffull / d - 1})
            for (int64_t dn = -1; dn <= 1; ++dn) one(k * d + dn);
        for (int i = 0; i < 64; ++i) one(rng() % 0x80000000ull);
        one(0x7fffffff);
    }
    ++g_cases;
}

// ------------------------------------------------------------------ chain verify

struct ChainShape {
    int32_t B, K, V;
    spec_dtype dt;
};

static void check_chain(const ChainShape &c) {
    Plan plan;
    if (!make_plan(SPEC_MODE_CHAIN, c.B, c.K, c.V, c.dt, plan)) {
        fprintf(stderr, "shape B=%d K=%d V=%d rejected\n", c.B, c.K, c.V);
        ++g_fail;
        return;
    }
    ++g_cases;
    if (c.B == 0) return;
    ChainArgs a{};
    a.B = c.B;
    a.K = c.K;
    a.V = c.V;
    a.chunk = plan.chunk;
    a.nchunk = plan.nchunk;
    a.nchunk2 = plan.nchunk2;
    chain_grid_fields(plan, c.K, a);
    const int64_t B = c.B, K = c.K, V = c.V, R = 2 * K + 1, nch = plan.nchunk, D = a.D;
    // The workspace regions fit the plan, in order.
    CHECK(plan.off_partial >= kWorkspaceHeader, "partials overlap the header");
    CHECK(plan.off_partial + static_cast<size_t>(B * R * nch) * 16 <= plan.off_sums, "partials");
    CHECK(plan.off_sums + static_cast<size_t>(B * plan.nchunk2) * 16 <= plan.off_rec, "sums");
    CHECK(plan.off_rec + static_cast<size_t>(B) * kRecWords * 8 <= plan.bytes, "records");
    // Every chunk holds logits: its first element is inside the row.
    CHECK((nch - 1) * plan.chunk < V && nch * plan.chunk >= V, "statistics chunks of V=%d", c.V);
    CHECK((D - 1) * plan.chunk2 < V && D * plan.chunk2 >= V, "draw chunks of V=%d", c.V);

    // The draws of the two-phase form (also the fallback of the one-call form).
    {
        ChainArgs m = a;
        if (g_mutant == 5) m.fd_D = make_fastdiv(a.D + 1);  // draw items per sequence off by one
        const uint32_t n = chain_draw_grid(m);
        std::vector<int64_t> res(B, -1), draw(B * D, -1), fin(B, -1), bon(B, -1);
        for (uint32_t g = 0; g < n; ++g) {
            const ChainItem it = chain_draw_item(g, m);
            CHECK(it.b < B, "draw grid g=%u b=%u", g, it.b);
            if (it.b >= B) continue;
            int64_t *slot = nullptr;
            if (it.kind == kItemResolver) slot = &res[it.b];
            else if (it.kind == kItemFinisher) slot = &fin[it.b];
            else if (it.kind == kItemBonus) slot = &bon[it.b];
            else if (it.kind == kItemDraw && it.p < D) slot = &draw[it.b * D + it.p];
            CHECK(slot && *slot < 0, "draw grid g=%u kind=%d b=%u p=%u twice or out of range", g, it.kind,
                  it.b, it.p);
            if (slot) *slot = g;
        }
        for (int64_t b = 0; b < B; ++b) {
            CHECK(res[b] >= 0 && fin[b] >= 0 && bon[b] >= 0, "draw grid b=%lld missing", (long long)b);
            for (int64_t p = 0; p < D; ++p) {
                CHECK(draw[b * D + p] > res[b], "draw before its resolver b=%lld", (long long)b);
                CHECK(fin[b] > draw[b * D + p], "finisher before a draw b=%lld", (long long)b);
            }
            CHECK(bon[b] > res[b], "bonus before its resolver");
        }
    }

    const uint32_t total = chain_schedule(a);
    if (total == 0) return;  // too large for one grid: the two phases run
    if (g_mutant == 2) a.fd_S1 = make_fastdiv(a.S);      // blocks of S, not S + 1
    if (g_mutant == 3 && B > 1) a.bon_end -= 1;           // bonus statistics end early
    if (g_mutant == 4) a.fd_D = make_fastdiv(a.D + 1);   // draw items per sequence off by one
    CHECK(total == chain_fused_grid(a), "grid %u vs %u", total, chain_fused_grid(a));
    std::vector<int64_t> st(B * R * nch, -1), res(B, -1), draw(B * D, -1), fin(B, -1), bon(B, -1);
    for (uint32_t g = 0; g < total; ++g) {
        const ChainItem it = chain_fused_item(g, a);
        CHECK(it.b < B, "g=%u b=%u", g, it.b);
        if (it.b >= B) continue;
        int64_t *slot = nullptr;
        if (it.kind == kItemStats) {
            CHECK(it.p < a.S, "g=%u p=%u", g, it.p);
            int row = -1, ch = -1;
            chain_stats_row(it.p, a, row, ch);
            CHECK(row >= 0 && row < R && row != K && ch >= 0 && ch < nch, "g=%u row=%d ch=%d", g, row, ch);
            if (row >= 0 && row < R && ch >= 0 && ch < nch) slot = &st[(it.b * R + row) * nch + ch];
        } else if (it.kind == kItemBonusStats) {
            CHECK(it.p < nch, "g=%u bonus chunk %u", g, it.p);
            if (it.p < nch) slot = &st[(it.b * R + K) * nch + it.p];
        } else if (it.kind == kItemResolver) {
            slot = &res[it.b];
        } else if (it.kind == kItemDraw) {
            CHECK(it.p < D, "g=%u draw chunk %u", g, it.p);
            if (it.p < D) slot = &draw[it.b * D + it.p];
        } else if (it.kind == kItemFinisher) {
            slot = &fin[it.b];
        } else {
            CHECK(it.kind == kItemBonus, "g=%u kind %d", g, it.kind);
            slot = &bon[it.b];
        }
        CHECK(slot && *slot < 0, "g=%u kind=%d b=%u p=%u twice", g, it.kind, it.b, it.p);
        if (slot) *slot = g;
    }
    for (int64_t b = 0; b < B; ++b) {
        int64_t last_rows = -1, last_bonus_row = -1, last_draw = -1;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t ch = 0; ch < nch; ++ch) {
                const int64_t p = st[(b * R + r) * nch + ch];
                CHECK(p >= 0, "b=%lld row=%lld ch=%lld never run", (long long)b, (long long)r, (long long)ch);
                (r == K ? last_bonus_row : last_rows) = std::max(r == K ? last_bonus_row : last_rows, p);
            }
        CHECK(res[b] >= 0 && fin[b] >= 0 && bon[b] >= 0, "b=%lld missing an item", (long long)b);
        // The resolver reads the statistics of rows 0..K-1 and K+1..2K.
        CHECK(res[b] > last_rows, "b=%lld resolver before its statistics", (long long)b);
        for (int64_t p = 0; p < D; ++p) {
            CHECK(draw[b * D + p] > res[b], "b=%lld draw %lld before its resolver", (long long)b,
                  (long long)p);
            last_draw = std::max(last_draw, draw[b * D + p]);
        }
        CHECK(fin[b] > last_draw && fin[b] > res[b], "b=%lld finisher too early", (long long)b);
        CHECK(bon[b] > res[b] && bon[b] > last_bonus_row, "b=%lld bonus item too early", (long long)b);
    }
}

// The position-major one-launch order (early exit), K >= 2.
static void check_chain_pm(const ChainShape &c) {
    Plan plan;
    if (!make_plan(SPEC_MODE_CHAIN, c.B, c.K, c.V, c.dt, plan) || c.B == 0 || c.K < 2) return;
    ChainArgs a{};
    a.B = c.B;
    a.K = c.K;
    a.V = c.V;
    a.chunk = plan.chunk;
    a.nchunk = plan.nchunk;
    a.nchunk2 = plan.nchunk2;
    chain_grid_fields(plan, c.K, a);
    const uint32_t total = chain_pm_schedule(a);
    if (total == 0) return;  // the sequence-major order runs instead
    ++g_cases;
    if (g_mutant == 8) a.fd_nch = make_fastdiv(a.nchunk + 1);  // the bonus rows' decode off by one
    const int64_t B = c.B, K = c.K, R = 2 * K + 1, nch = plan.nchunk, D = a.D;
    const Grid3 grid = chain_pm_grid(a);
    CHECK(static_cast<uint64_t>(grid.x) * grid.y * grid.z == total, "pm grid %u x %u x %u vs %u", grid.x,
          grid.y, grid.z, total);
    CHECK(plan.off_pairs >= plan.off_rec + static_cast<size_t>(B) * kRecWords * 8, "pairs overlap records");
    CHECK(plan.off_gate >= plan.off_pairs + static_cast<size_t>(B * K) * 8, "gate lines overlap pairs");
    CHECK(plan.off_gate % kGateLineBytes == 0, "gate lines not line-aligned");
    CHECK(plan.off_gate + static_cast<size_t>(B * K) * kGateLineBytes <= plan.bytes,
          "gate lines past the workspace");
    std::vector<int64_t> st(B * R * nch, -1), pr(B * K, -1), draw(B * D, -1), fin(B, -1), bon(B, -1);
    // The arguments the decode sees (a planted mistake narrows its rows).
    ChainArgs dec = a;
    if (g_mutant == 9 && dec.nchunk > 1) dec.nchunk -= 1;  // slabs decoded one chunk too narrow
    int64_t last_real = -1, first_none = -1;
    for (uint32_t g = 0; g < total; ++g) {
        // The flattened index the hardware hands out: x fastest, then y, then z.
        const uint32_t x = g % grid.x, y = (g / grid.x) % grid.y, z = g / (grid.x * grid.y);
        int row = -1, ch = -1;
        const ChainItem it = chain_pm_item(x, y, z, dec, row, ch);
        if (it.kind == kItemNone) {
            CHECK(z >= K, "pm g=%u empty slot among the positions", g);
            if (first_none < 0) first_none = g;
            continue;
        }
        last_real = g;
        CHECK(it.b < B, "pm g=%u b=%u", g, it.b);
        if (it.b >= B) continue;
        int64_t *slot = nullptr;
        if (it.kind == kItemStats) {
            int prow = -1, pch = -1;
            chain_stats_row(it.p, a, prow, pch);
            CHECK(prow == row && pch == ch, "pm g=%u row %d/%d ch %d/%d", g, row, prow, ch, pch);
            CHECK(z < K && row >= 0 && row < R && row != K && ch >= 0 && ch < nch, "pm g=%u row=%d ch=%d", g,
                  row, ch);
            if (row >= 0 && row < R && ch >= 0 && ch < nch) slot = &st[(it.b * R + row) * nch + ch];
        } else if (it.kind == kItemBonusStats) {
            CHECK(it.p < nch, "pm g=%u bonus chunk %u", g, it.p);
            if (it.p < nch) slot = &st[(it.b * R + K) * nch + it.p];
        } else if (it.kind == kItemPair) {
            CHECK(it.p < K, "pm g=%u position %u", g, it.p);
            if (it.p < K) slot = &pr[it.b * K + it.p];
        } else if (it.kind == kItemDraw) {
            CHECK(it.p < D, "pm g=%u draw chunk %u", g, it.p);
            if (it.p < D) slot = &draw[it.b * D + it.p];
        } else if (it.kind == kItemFinisher) {
            slot = &fin[it.b];
        } else {
            CHECK(it.kind == kItemBonus, "pm g=%u kind %d", g, it.kind);
            slot = &bon[it.b];
        }
        CHECK(slot && *slot < 0, "pm g=%u kind=%d b=%u p=%u twice", g, it.kind, it.b, it.p);
        if (slot) *slot = g;
    }
    for (int64_t b = 0; b < B; ++b) {
        int64_t last_pr = -1, last_draw = -1, last_bonus_row = -1;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t ch = 0; ch < nch; ++ch) {
                const int64_t p = st[(b * R + r) * nch + ch];
                CHECK(p >= 0, "pm b=%lld row=%lld ch=%lld never run", (long long)b, (long long)r, (long long)ch);
                if (r == K) last_bonus_row = std::max(last_bonus_row, p);
            }
        for (int64_t k = 0; k < K; ++k) {
            const int64_t p = pr[b * K + k];
            CHECK(p >= 0, "pm b=%lld pair %lld missing", (long long)b, (long long)k);
            // after the statistics of its two rows and the earlier positions' resolvers
            for (int64_t ch = 0; ch < nch; ++ch) {
                CHECK(p > st[(b * R + k) * nch + ch] && p > st[(b * R + K + 1 + k) * nch + ch],
                      "pm b=%lld pair %lld before its rows", (long long)b, (long long)k);
            }
            if (k > 0) CHECK(p > pr[b * K + k - 1], "pm b=%lld pair %lld before pair %lld", (long long)b,
                             (long long)k, (long long)(k - 1));
            // position k's outcome comes before position k + 1's rows
            if (k + 1 < K)
                for (int64_t ch = 0; ch < nch; ++ch)
                    CHECK(p < st[(b * R + k + 1) * nch + ch] && p < st[(b * R + K + 2 + k) * nch + ch],
                          "pm b=%lld pair %lld after its gated rows", (long long)b, (long long)k);
            last_pr = std::max(last_pr, p);
        }
        for (int64_t p = 0; p < D; ++p) {
            CHECK(draw[b * D + p] > last_pr, "pm b=%lld draw before the record", (long long)b);
            last_draw = std::max(last_draw, draw[b * D + p]);
        }
        CHECK(fin[b] > last_draw && fin[b] > last_pr, "pm b=%lld finisher too early", (long long)b);
        CHECK(bon[b] > last_pr && bon[b] > last_bonus_row, "pm b=%lld bonus item too early", (long long)b);
    }
    CHECK(first_none < 0 || first_none > last_real, "pm empty slot %lld before item %lld", (long long)first_none,
          (long long)last_real);
}

// ------------------------------------------------------------------ greedy chain, static tree

static void check_argmax(spec_mode mode, int32_t B, int32_t KN, int32_t V, spec_dtype dt) {
    Plan plan;
    CHECK(make_plan(mode, B, KN, V, dt, plan), "argmax shape rejected");
    ++g_cases;
    if (B == 0) return;
    const int64_t rows = plan.rows, nch = plan.nchunk, per = rows / B;
    CHECK(rows % B == 0, "rows %lld per sequence", (long long)rows);
    CHECK((nch - 1) * plan.chunk < V && nch * plan.chunk >= V, "argmax chunks");
    CHECK(plan.off_partial + static_cast<size_t>(rows * nch) * 16 <= plan.bytes, "argmax partials");
    if (mode == SPEC_MODE_TREE) {
        // The node-major order: an outcome word per node, then a gate line
        // per node, and a grid (chunks + 1) x trees x nodes.
        CHECK(plan.off_pairs >= plan.off_partial + static_cast<size_t>(rows * nch) * 16, "node outcomes overlap");
        CHECK(plan.off_gate >= plan.off_pairs + static_cast<size_t>(rows) * 8, "node gates overlap");
        CHECK(plan.off_gate % kGateLineBytes == 0, "node gates not line-aligned");
        CHECK(plan.off_gate + static_cast<size_t>(rows) * kGateLineBytes <= plan.bytes, "node gates past the workspace");
        const Grid3 g = tree_node_major_grid(static_cast<int32_t>(nch), B, KN);
        CHECK(static_cast<int64_t>(g.x) * g.y * g.z == (nch + 1) * rows, "node-major grid");
    }
    // Argmax items only; the last chunk of a sequence's last row resolves it.
    const uint32_t n = argmax_only_grid(rows, nch);
    const uint32_t per_dec = static_cast<uint32_t>(g_mutant == 10 ? per + 1 : per);  // rows a sequence, as decoded
    const FastDiv fd_nch = make_fastdiv(static_cast<uint32_t>(nch)), fd_per = make_fastdiv(per_dec);
    std::vector<int64_t> am(rows * nch, -1), res(B, -1);
    for (uint32_t g = 0; g < n; ++g) {
        const ArgmaxItem it = argmax_item_of(g, static_cast<uint32_t>(nch), fd_nch, static_cast<uint32_t>(rows));
        CHECK(it.argmax && it.row < rows && it.ch < nch, "g=%u", g);
        if (!(it.argmax && it.row < rows && it.ch < nch)) continue;
        CHECK(am[it.row * nch + it.ch] < 0, "g=%u twice", g);
        am[it.row * nch + it.ch] = g;
        uint32_t b = 0;
        if (argmax_resolves(it.row, it.ch, static_cast<uint32_t>(nch), per_dec, fd_per, b)) {
            CHECK(b < static_cast<uint32_t>(B), "g=%u resolves %u", g, b);
            if (b < static_cast<uint32_t>(B)) {
                CHECK(res[b] < 0, "g=%u resolves %u twice", g, b);
                res[b] = g;
            }
        }
    }
    for (int64_t b = 0; b < B; ++b) {
        CHECK(res[b] >= 0, "resolve %lld missing", (long long)b);
        for (int64_t r = b * per; r < (b + 1) * per; ++r)
            for (int64_t ch = 0; ch < nch; ++ch)
                CHECK(am[r * nch + ch] >= 0 && am[r * nch + ch] <= res[b], "row %lld ch %lld after its resolve",
                      (long long)r, (long long)ch);
    }
}

// ------------------------------------------------------------------ per-sequence trees

// The compact order's wavefront arithmetic, lane by lane: counts through the
// kernel's own lane_tree_rows, the inclusive scan and the first lane whose
// total passes R, then the kernel's lane_row walk.
template <int P>
static uint32_t locate_row_host(const std::vector<int32_t> &count, int B, int Nmax, uint32_t R,
                                uint32_t &b, uint32_t &v) {
    int n[64][P], incl[64], s[64];
    int run = 0;
    for (int lane = 0; lane < 64; ++lane) {
        lane_tree_rows<P>(count.data(), B, Nmax, lane, n[lane]);
        s[lane] = 0;
        for (int j = 0; j < P; ++j) s[lane] += n[lane][j];
        run += s[lane];
        incl[lane] = run;
    }
    const uint32_t T = static_cast<uint32_t>(incl[63]);
    if (R < T) {
        int L = 0;
        while (!(static_cast<uint32_t>(incl[L]) > R)) ++L;
        const uint32_t r = R - static_cast<uint32_t>(incl[L] - s[L]);
        lane_row<P>(r, static_cast<uint32_t>(L) * P, [&](int j) { return static_cast<uint32_t>(n[L][j]); }, b, v);
    }
    return T;
}

static void check_tree_dyn(int32_t B, int32_t Nmax, int32_t V, spec_dtype dt, std::mt19937_64 &rng,
                           int count_mode) {
    Plan plan;
    CHECK(make_plan(SPEC_MODE_TREE_DYN, B, Nmax, V, dt, plan), "tree_dyn shape rejected");
    ++g_cases;
    if (B == 0) return;
    {
        // The node-major order: an outcome word and a gate line per node slot.
        const int64_t rows = plan.rows, nch = plan.nchunk;
        CHECK(plan.off_pairs >= plan.off_partial + static_cast<size_t>(rows * nch) * 16, "node outcomes overlap");
        CHECK(plan.off_gate >= plan.off_pairs + static_cast<size_t>(rows) * 8, "node gates overlap");
        CHECK(plan.off_gate % kGateLineBytes == 0, "node gates not line-aligned");
        CHECK(plan.off_gate + static_cast<size_t>(rows) * kGateLineBytes <= plan.bytes, "node gates past the workspace");
    }
    // Node counts: in range, or out of range both ways (clamped to [1, Nmax]).
    std::vector<int32_t> count(B);
    for (auto &c : count) {
        if (count_mode == 0) c = 1 + static_cast<int32_t>(rng() % Nmax);
        else if (count_mode == 1) c = Nmax;
        else c = static_cast<int32_t>(rng() % (Nmax + 8)) - 4;
    }
    const uint32_t nch = static_cast<uint32_t>(plan.nchunk), rows = static_cast<uint32_t>(plan.rows);
    CHECK(rows == static_cast<uint32_t>(B) * Nmax, "rows");
    const uint32_t n = argmax_grid(rows, nch, B);
    std::vector<int64_t> am(static_cast<size_t>(rows) * nch, -1), res(B, -1);
    // The divisors as the library makes them for the launch.
    const FastDiv fd_nch = make_fastdiv(nch), fd_nmax = make_fastdiv(static_cast<uint32_t>(Nmax));
    for (uint32_t g = 0; g < n; ++g) {
        TreeDynItem it;
        if (B <= kCompactTrees) {
            const uint32_t R = fdiv(g, fd_nch);
            CHECK(R == g / nch, "g=%u row %u", g, R);
            uint32_t b = 0, v = 0;
            const uint32_t T = B <= 64 ? locate_row_host<1>(count, B, Nmax, R, b, v)
                                       : locate_row_host<kCountsPerLane>(count, B, Nmax, R, b, v);
            it = tree_dyn_compact_item(g, R, nch, T, b, v, B, g_mutant == 6 ? Nmax - 1 : Nmax);
        } else {
            it = tree_dyn_full_item(g, nch, fd_nch, rows, Nmax, fd_nmax, count.data());
        }
        CHECK(!(it.argmax && it.resolve), "g=%u both", g);
        if (it.argmax) {
            const uint32_t b = it.row / Nmax, v = it.row % Nmax;
            CHECK(it.row < rows && it.ch < nch, "g=%u row %u ch %u", g, it.row, it.ch);
            if (it.row < rows && it.ch < nch) {
                CHECK(static_cast<int>(v) < tree_rows(count[b], Nmax), "g=%u padding row b=%u v=%u read", g, b, v);
                CHECK(am[static_cast<size_t>(it.row) * nch + it.ch] < 0, "g=%u twice", g);
                am[static_cast<size_t>(it.row) * nch + it.ch] = g;
            }
        } else if (it.resolve) {
            CHECK(it.row < static_cast<uint32_t>(B), "g=%u resolve %u", g, it.row);
            if (it.row < static_cast<uint32_t>(B)) {
                CHECK(res[it.row] < 0, "g=%u resolve twice", g);
                res[it.row] = g;
            }
        }
    }
    for (int32_t b = 0; b < B; ++b) {
        CHECK(res[b] >= 0, "resolve %d missing", b);
        const int nr = tree_rows(count[b], Nmax);
        for (int v = 0; v < Nmax; ++v)
            for (uint32_t ch = 0; ch < nch; ++ch) {
                const int64_t p = am[(static_cast<size_t>(b) * Nmax + v) * nch + ch];
                if (v < nr) CHECK(p >= 0 && p < res[b], "b=%d v=%d ch=%u", b, v, ch);
                else CHECK(p < 0, "padding b=%d v=%d read", b, v);
            }
    }
}

// ------------------------------------------------------------------ top-k

static void check_topk(int32_t rows, int32_t V, int32_t k, spec_dtype dt) {
    Plan plan;
    CHECK(make_plan(SPEC_MODE_TOPK, rows, k, V, dt, plan), "topk shape rejected");
    ++g_cases;
    if (rows == 0) return;
    const int64_t nch = plan.nchunk, G = (rows + 3) / 4, L = topk_lag(rows, plan.nchunk);
    CHECK(L >= 1 && L <= G, "lag %lld of %lld groups", (long long)L, (long long)G);
    CHECK((nch - 1) * plan.chunk < V && nch * plan.chunk >= V, "topk chunks");
    CHECK(plan.off_partial + static_cast<size_t>(rows * nch) * kMaxTopK * 16 <= plan.bytes, "topk lists");
    const uint32_t n = topk_grid(rows, nch);
    std::vector<int64_t> chunk(rows * nch, -1), merge(G, -1);
    const int64_t nch_dec = g_mutant == 7 ? nch + 1 : nch;  // chunks per row, as the decode sees them
    const FastDiv fd_nch = make_fastdiv(static_cast<uint32_t>(nch_dec)),
                  fd_blk = make_fastdiv(static_cast<uint32_t>(kTopkGroupRows * nch_dec + 1));
    for (uint32_t g = 0; g < n; ++g) {
        const TopkItem it = topk_item(g, rows, nch_dec, L, fd_nch, fd_blk);
        if (it.mgroup < 0) {
            CHECK(it.row >= 0 && it.row < rows && it.ch >= 0 && it.ch < nch, "g=%u row %lld ch %lld", g,
                  (long long)it.row, (long long)it.ch);
            if (it.row >= 0 && it.row < rows && it.ch >= 0 && it.ch < nch) {
                CHECK(chunk[it.row * nch + it.ch] < 0, "g=%u twice", g);
                chunk[it.row * nch + it.ch] = g;
            }
        } else {
            CHECK(it.mgroup < G, "g=%u merge group %lld of %lld", g, (long long)it.mgroup, (long long)G);
            if (it.mgroup < G) {
                CHECK(merge[it.mgroup] < 0, "g=%u merge twice", g);
                merge[it.mgroup] = g;
            }
        }
    }
    for (int64_t q = 0; q < G; ++q) {
        CHECK(merge[q] >= 0, "merge %lld missing", (long long)q);
        for (int64_t r = q * 4; r < std::min<int64_t>(rows, q * 4 + 4); ++r)
            for (int64_t ch = 0; ch < nch; ++ch)
                CHECK(chunk[r * nch + ch] >= 0 && chunk[r * nch + ch] < merge[q], "row %lld ch %lld", (long long)r,
                      (long long)ch);
    }
}

int main(int argc, char **argv) {
    if (argc > 1) g_mutant = atoi(argv[1]);
    std::mt19937_64 rng(20260214);
    check_fastdiv(rng);
    const spec_dtype BF = SPEC_DTYPE_BF16, F = SPEC_DTYPE_F32;
    // The benchmark workloads, then edges: K = 0, B = 1, V = 1, ragged V,
    // K at its limit, V at its limits, large B.
    const ChainShape chains[] = {
        {8, 4, 1024, F},       {64, 5, 128256, BF},  {256, 8, 151936, F},  {3, 0, 5000, BF},
        {1, 5, 128256, BF},    {5, 3, 4099, F},      {2, 2, 1, F},         {4, 64, 2000, BF},
        {2, 3, 1 << 19, BF},   {2, 3, 1 << 18, F},   {2, 3, (1 << 19) - 1, BF}, {4096, 4, 32000, BF},
        {1, 0, 1, F},          {0, 4, 100, F},       {7, 1, 2048, F},      {7, 1, 2049, F},
        {9, 2, 4096, BF},      {9, 2, 4097, BF},     {128, 1, 4096, F},    {3, 64, 300000, BF},
        {8, 3, 1 << 19, BF},   {8, 3, 1 << 18, F},   {1, 64, 1 << 19, BF},
    };
    for (const auto &c : chains) {
        check_chain(c);
        check_chain_pm(c);
    }
    for (int i = 0; i < 300; ++i) {
        const int32_t B = 1 + static_cast<int32_t>(rng() % 96), K = static_cast<int32_t>(rng() % 17);
        const spec_dtype dt = (rng() & 1) ? BF : F;
        const int32_t vmax = dt == BF ? (1 << 19) : (1 << 18);
        const int32_t V = 1 + static_cast<int32_t>(rng() % (i < 150 ? 20000 : vmax));
        check_chain({B, K, V, dt});
        check_chain_pm({B, K, V, dt});
    }
    const int32_t argmax_shapes[][3] = {{64, 5, 32000}, {8, 0, 1}, {1, 64, 128256}, {3, 7, 8193},
                                        {32, 45, 128256}, {5, 1, 4096}, {300, 3, 100},
                                        {1, 1, 1 << 26}, {1, 2, 1 << 26}, {1, 4, 1 << 26}};
    for (const auto &s : argmax_shapes) {
        check_argmax(SPEC_MODE_GREEDY, s[0], s[1], s[2], BF);
        check_argmax(SPEC_MODE_GREEDY, s[0], s[1], s[2], F);
        if (s[1] >= 1) check_argmax(SPEC_MODE_TREE, s[0], s[1], s[2], BF);
    }
    const int32_t tree_shapes[][3] = {{32, 64, 128256}, {1, 1, 10}, {64, 7, 9000}, {65, 7, 9000},
                                      {255, 5, 3000},   {256, 5, 3000}, {257, 5, 3000}, {300, 3, 20000},
                                      {4, 256, 5000},   {100, 16, 16384}};
    for (const auto &s : tree_shapes)
        for (int mode = 0; mode < 3; ++mode) check_tree_dyn(s[0], s[1], s[2], BF, rng, mode);
    const int32_t topk_shapes[][3] = {{512, 128256, 8}, {1, 1, 1}, {3, 100, 8}, {4, 4096, 5},
                                      {5, 8193, 8},     {1202, 20001, 5}, {403, 140000, 8},
                                      {97, 128256, 8},  {33, 524288, 8}, {3001, 100, 8}, {8, 4097, 1}};
    for (const auto &s : topk_shapes) {
        check_topk(s[0], s[1], s[2], BF);
        check_topk(s[0], s[1], s[2], F);
    }
    for (int i = 0; i < 100; ++i) {
        const int32_t rows = 1 + static_cast<int32_t>(rng() % 3000), V = 8 + static_cast<int32_t>(rng() % 300000);
        check_topk(rows, V, 1 + static_cast<int32_t>(rng() % 8), (rng() & 1) ? BF : F);
    }
    if (g_fail) {
        fprintf(stderr, "%ld failures\n", g_fail);
        return 1;
    }
    printf("ok %ld\n", g_cases);
    return 0;
}
