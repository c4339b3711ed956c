// Host check of the launch-epoch arithmetic of the look-back records
// (nonlinear_rnn_solve_pararnn_amd/csrc/tags.hpp), built by
// tests/test_epoch.py.  Prints "ok" and exits 0 when every check passes.
//
//  1. Every tag of a period is a signalling-NaN bit pattern, and no two
//     epochs of a period share a tag.
//  2. The header word after the draws of a launch: one epoch per launch, the
//     epoch advances once per launch and returns to 0 after kTagPeriod
//     launches; exactly the last launch of a period is a wrap launch.
//  3. The clear ranges cover every word past the header except the kept
//     range, for every position of the kept range.
//  4. A model of a workspace over several periods (a short period, random
//     launches that read records before writing their own, as the look-back
//     does): with the clear at each wrap launch no read ever matches a record
//     that another launch wrote; without it, some read does (the hazard the
//     clear removes).
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <vector>

#include "tags.hpp"

using namespace prn;

static int fails = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            if (fails < 20) fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

static bool is_snan(uint32_t t) {
    return (t & 0x7f800000u) == 0x7f800000u && (t & 0x00400000u) == 0 && (t & 0x007fffffu) != 0;
}

static void check_tags() {
    uint32_t prev_pos = 0, prev_neg = 0;
    for (uint32_t e = 0; e < kTagPeriod; ++e) {
        const uint32_t t = launch_tag(e);
        CHECK(is_snan(t));
        // strictly increasing within each sign half, halves told apart by
        // the sign bit: injective over the period
        if (t & 0x80000000u) {
            CHECK(e >= kTagHalf);
            if (e > kTagHalf) CHECK(t > prev_neg);
            prev_neg = t;
        } else {
            CHECK(e < kTagHalf);
            if (e > 0) CHECK(t > prev_pos);
            prev_pos = t;
        }
        CHECK(t != 0u);  // a zero-filled word never carries a tag
    }
    CHECK(launch_tag(kTagHalf - 1) == 0x7fbfffffu);
    CHECK(launch_tag(kTagHalf) == 0xff800001u);
    CHECK(launch_tag(kTagPeriod - 1) == 0xffbfffffu);
}

// Draws of one launch against a header word: returns the epoch every draw
// saw (or ~0u if they differed) and whether it was a wrap launch.
static uint32_t run_launch(uint64_t &hdr, uint32_t draws, uint32_t period, bool &wrap) {
    uint32_t seen = ~0u - 1;
    bool same = true;
    for (uint32_t d = 0; d < draws; ++d) {
        const uint64_t old = hdr;
        hdr = old + 1;  // the atomic increment
        const uint32_t idx = (uint32_t)old, epoch = (uint32_t)(old >> 32);
        if (idx + 1 == draws) hdr = header_after_draw(idx, epoch, draws, period);
        if (seen == ~0u - 1) seen = epoch;
        same = same && seen == epoch;
        CHECK(idx == d);
    }
    wrap = is_wrap_launch(seen, period);
    return same ? seen : ~0u;
}

static void check_header() {
    std::mt19937_64 rng(1);
    for (uint32_t period : {2u, 3u, 7u, 1000u}) {
        uint64_t hdr = 0;
        for (uint32_t l = 0; l < 3 * period + 5; ++l) {
            const uint32_t draws = 1 + (uint32_t)(rng() % 300);
            bool wrap = false;
            const uint32_t e = run_launch(hdr, draws, period, wrap);
            CHECK(e == l % period);
            CHECK(wrap == (l % period == period - 1));
            CHECK((uint32_t)hdr == 0);  // count reset for the next launch
            CHECK((uint32_t)(hdr >> 32) == (l + 1) % period);
        }
    }
    // the real period: the launch at epoch kTagPeriod - 1 wraps to 0
    CHECK(next_epoch(kTagPeriod - 1) == 0);
    CHECK(is_wrap_launch(kTagPeriod - 1));
    CHECK(!is_wrap_launch(kTagPeriod - 2));
    CHECK(!is_wrap_launch(0));
    CHECK(header_after_draw(9, kTagPeriod - 1, 10) == 0);
    CHECK(header_after_draw(3, 5, 10) == ((uint64_t)5 << 32 | 4));
}

static void check_clear_ranges() {
    for (uint64_t words = 0; words < 40; ++words)
        for (uint64_t lo = 0; lo < 44; ++lo)
            for (uint64_t hi = 0; hi < 44; ++hi) {
                const ClearRanges r = clear_ranges(words, lo, hi);
                for (uint64_t w = 0; w < words; ++w) {
                    const bool c = (w >= r.lo0 && w < r.hi0) || (w >= r.lo1 && w < r.hi1);
                    const bool keep = lo < hi && w >= lo && w < hi;
                    CHECK(c == (w >= kHeaderWords && !keep));
                }
                CHECK(r.hi0 <= r.lo1 || r.lo1 >= r.hi1 || r.lo0 >= r.hi0);  // disjoint
                CHECK(r.hi0 <= words && r.hi1 <= words);
            }
}

// Workspace model: `words` record slots, each a 64-bit word tag:payload.
// Each launch draws a random region (base, size) of the workspace as its
// record area, reads random slots of it before writing them (a look-back
// that polls records not yet published) and then writes every slot of it
// with its tag.  A read whose tag equals the launch's own tag and that this
// launch has not written is a stale match.  Returns the stale matches seen.
static uint64_t model(uint32_t period, bool clear_at_wrap, uint64_t seed) {
    const uint64_t words = 64;
    std::vector<uint64_t> ws(words, 0);
    std::mt19937_64 rng(seed);
    uint64_t hdr = 0, stale = 0;
    for (int l = 0; l < 40 * (int)period; ++l) {
        bool wrap = false;
        const uint32_t epoch = run_launch(hdr, 1 + (uint32_t)(rng() % 8), period, wrap);
        const uint32_t tag = launch_tag(epoch);
        const uint64_t base = kHeaderWords + rng() % (words - kHeaderWords);
        const uint64_t size = 1 + rng() % (words - base);
        std::vector<bool> mine(words, false);
        for (uint64_t k = 0; k < size; ++k) {
            const uint64_t w = base + rng() % size;  // poll before publishing
            if (!mine[w] && (uint32_t)(ws[w] >> 32) == tag) ++stale;
            const uint64_t v = base + k;  // publish
            ws[v] = ((uint64_t)tag << 32) | (uint32_t)rng();
            mine[v] = true;
        }
        if (wrap && clear_at_wrap) {
            const ClearRanges r = clear_ranges(words, 0, 0);
            for (uint64_t w = r.lo0; w < r.hi0; ++w) ws[w] = 0;
            for (uint64_t w = r.lo1; w < r.hi1; ++w) ws[w] = 0;
        }
    }
    return stale;
}

static void check_model() {
    uint64_t without = 0;
    for (uint32_t period : {2u, 3u, 5u})
        for (uint64_t seed = 1; seed <= 50; ++seed) {
            CHECK(model(period, true, seed) == 0);
            without += model(period, false, seed);
        }
    CHECK(without > 0);  // the model does see the hazard when nothing clears
}

int main() {
    check_tags();
    check_header();
    check_clear_ranges();
    check_model();
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
