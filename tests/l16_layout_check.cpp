// Host-side check of the L = 16 kernel's index math (l16_layout.h), compiled with g++
// by test_l16_layout.py.  Verifies, exhaustively over all 2^16 slots:
//  - state_of(p, .) is a bijection slots -> states and slot_of(p, .) is its inverse;
//  - the four registers of a group at step p hold the four predecessors of one group
//    (states that differ only in the oldest digit) at p-1, and the successors with
//    new digit b = 0..3 at p;
//  - the transposition moves the value of each state at p = 3 to the slot that holds
//    the same state at p = 0;
//  - LDS staging addresses are in range, distinct within a round, agree between the
//    writing and the reading side, and every wave instruction touches distinct banks
//    (64 banks per wave, 32 per half wave);
//  - the k*V = 4 half-step patterns place the metric on the even half-steps and list
//    every metric group once, in processing order.
#define __host__
#define __device__
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "l16_layout.h"

using namespace tcq::l16;

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            if (fails < 20) std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

int main() {
    // bijection and inverse
    for (int p = 0; p <= 3; ++p) {
        std::vector<int> seen(1 << 16, 0);
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t l = 0; l < 64; ++l)
                for (uint32_t r = 0; r < 128; ++r) {
                    uint32_t s = state_of(p, w, l, r);
                    CHECK(s < (1u << 16));
                    seen[s]++;
                    Slot q = slot_of(p, s);
                    CHECK(q.w == w && q.l == l && q.r == r);
                }
        for (int s = 0; s < (1 << 16); ++s) CHECK(seen[s] == 1);
    }
    // group structure
    for (int p = 1; p <= 3; ++p)
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t l = 0; l < 64; ++l)
                for (uint32_t g = 0; g < 32; ++g) {
                    uint32_t x = state_of(p - 1, w, l, group_reg(p, g, 0)) & 0x3FFFu;
                    for (uint32_t j = 0; j < 4; ++j) {
                        uint32_t r = group_reg(p, g, j);
                        CHECK(r < 128);
                        CHECK(reg_group(p, r) == g);
                        // predecessor j of the group: (j << 14) | x
                        CHECK(state_of(p - 1, w, l, r) == ((j << 14) | x));
                        // successor with new digit b = j: (x << 2) | j
                        CHECK(state_of(p, w, l, r) == ((x << 2) | j));
                    }
                }
    // transposition
    {
        std::set<uint32_t> dests;
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t l = 0; l < 64; ++l)
                for (uint32_t r = 0; r < 128; ++r) {
                    Slot d = transpose_dest(w, l, r);
                    CHECK(d.w < 8 && d.l < 64 && d.r < 128);
                    CHECK(state_of(3, w, l, r) == state_of(0, d.w, d.l, d.r));
                    CHECK(((d.r & 1u) == ((r >> 6) & 1u)));  // round split
                    dests.insert((d.w << 13) | (d.l << 7) | d.r);
                    CHECK(lds_write_lane(w, l) + lds_write_reg(r) ==
                          lds_read_lane(d.w, d.l) + lds_read_reg(d.r));
                }
        CHECK(dests.size() == (1u << 16));
    }
    // LDS addresses: range, injectivity per round, banks
    for (uint32_t rho = 0; rho < 2; ++rho) {
        std::vector<int> used(kLdsDwords, 0);
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t r = 0; r < 128; ++r) {
                if (((r >> 6) & 1u) != rho) continue;
                std::set<uint32_t> b64, b32lo, b32hi;
                for (uint32_t l = 0; l < 64; ++l) {
                    uint32_t a = lds_write_lane(w, l) + lds_write_reg(r);
                    CHECK(a < kLdsDwords);
                    if (a < kLdsDwords) used[a]++;
                    b64.insert(a % 64);
                    (l < 32 ? b32lo : b32hi).insert(a % 32);
                }
                CHECK(b64.size() == 64 && b32lo.size() == 32 && b32hi.size() == 32);
            }
        int dup = 0;
        for (auto u : used) dup += (u > 1);
        CHECK(dup == 0);
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t r = 0; r < 128; ++r) {
                if ((r & 1u) != rho) continue;
                std::set<uint32_t> b64, b32lo, b32hi;
                for (uint32_t l = 0; l < 64; ++l) {
                    uint32_t a = lds_read_lane(w, l) + lds_read_reg(r);
                    CHECK(a < kLdsDwords);
                    if (a < kLdsDwords) CHECK(used[a] == 1);
                    b64.insert(a % 64);
                    (l < 32 ? b32lo : b32hi).insert(a % 32);
                }
                CHECK(b64.size() == 64 && b32lo.size() == 32 && b32hi.size() == 32);
            }
    }
    // segment order: every (step, group) exactly once per super-step; step 1/2 halves
    // follow register bit 0, step 3 halves follow register bit 6; backpointer slots
    // are distinct per (step, group)
    for (int p = 1; p <= 3; ++p) {
        std::set<uint32_t> gs, slots;
        for (int seg = 0; seg < 6; ++seg) {
            if (seg_step(seg) != p) continue;
            for (int i = 0; i < 16; ++i) {
                uint32_t g = seg_group(seg, i);
                CHECK(g < 32);
                gs.insert(g);
                CHECK(bp_half(p, g) == (uint32_t)seg_half(seg));
                CHECK(bp_shift(p, g) == 2u * (15u - (uint32_t)i));
                slots.insert(bp_half(p, g) * 32 + bp_shift(p, g));
                for (uint32_t b = 0; b < 4; ++b) {
                    uint32_t r = group_reg(p, g, b);
                    if (p < 3) CHECK((r & 1u) == (uint32_t)seg_half(seg));
                    else CHECK(((r >> 6) & 1u) == (uint32_t)seg_half(seg));
                }
            }
        }
        CHECK(gs.size() == 32 && slots.size() == 32);
    }
    // naming: each LDS round reads into the physical registers it wrote out
    for (int m = 0; m < 2; ++m)
        for (int rho = 0; rho < 2; ++rho) {
            std::set<uint32_t> out, in;
            for (uint32_t r = 0; r < 128; ++r) {
                if (((r >> 6) & 1u) == (uint32_t)rho) out.insert(phys(m, r));
                if ((r & 1u) == (uint32_t)rho) in.insert(phys(1 - m, r));
            }
            CHECK(out == in && out.size() == 64);
        }
    for (uint32_t r = 0; r < 128; ++r) CHECK(phys(1, phys(1, r)) == r && phys(0, r) == r);
    // k*V = 3: bijection, group structure (8 predecessors (j << 13) | x, successors
    // (x << 3) | b), transposition after two steps, segments and backpointer slots
    for (int p = 0; p <= 2; ++p) {
        std::vector<int> seen(1 << 16, 0);
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t l = 0; l < 64; ++l)
                for (uint32_t r = 0; r < 128; ++r) {
                    uint32_t st = state_of3(p, w, l, r);
                    seen[st]++;
                    Slot q = slot_of3(p, st);
                    CHECK(q.w == w && q.l == l && q.r == r);
                }
        for (int st = 0; st < (1 << 16); ++st) CHECK(seen[st] == 1);
    }
    for (int p = 1; p <= 2; ++p)
        for (uint32_t w = 0; w < 8; ++w)
            for (uint32_t l = 0; l < 64; ++l)
                for (uint32_t g = 0; g < 16; ++g) {
                    uint32_t x = state_of3(p - 1, w, l, group_reg3(p, g, 0)) & 0x1FFFu;
                    for (uint32_t j = 0; j < 8; ++j) {
                        uint32_t r = group_reg3(p, g, j);
                        CHECK(r < 128 && reg_group3(p, r) == g);
                        CHECK(state_of3(p - 1, w, l, r) == ((j << 13) | x));
                        CHECK(state_of3(p, w, l, r) == ((x << 3) | j));
                    }
                }
    for (uint32_t w = 0; w < 8; ++w)
        for (uint32_t l = 0; l < 64; ++l)
            for (uint32_t r = 0; r < 128; ++r) {
                Slot d = transpose_dest(w, l, r);
                CHECK(state_of3(2, w, l, r) == state_of3(0, d.w, d.l, d.r));
            }
    for (int p = 1; p <= 2; ++p) {
        std::set<uint32_t> gs, slots;
        for (int seg = 0; seg < 4; ++seg) {
            if (seg3_step(seg) != p) continue;
            for (int i = 0; i < 8; ++i) {
                uint32_t g = seg3_group(seg, i);
                CHECK(g < 16);
                gs.insert(g);
                CHECK(bp3_half(p, g) == (uint32_t)seg3_half(seg));
                CHECK(bp3_shift(p, g) == 3u * (7u - (uint32_t)i));
                slots.insert(bp3_half(p, g) * 32 + bp3_shift(p, g));
                for (uint32_t b = 0; b < 8; ++b) {
                    uint32_t r = group_reg3(p, g, b);
                    if (p == 1) CHECK((r & 1u) == (uint32_t)seg3_half(seg));
                    else CHECK(((r >> 6) & 1u) == (uint32_t)seg3_half(seg));
                }
            }
        }
        CHECK(gs.size() == 16 && slots.size() == 16);
    }
    // k*V = 4 half-steps: the metric positions of each pattern cover every metric group
    // once, in processing order, and the pattern follows the half-step parity
    for (int mp = 0; mp <= 1; ++mp) {
        std::set<uint32_t> seen;
        int expect = 0;
        for (int seg = 0; seg < 6; ++seg) {
            CHECK(seg_has_metric(mp, seg) == (((seg_step(seg) + mp) % 2) == 0));
            if (!seg_has_metric(mp, seg)) continue;
            CHECK(metric_index(mp, seg) == expect);
            CHECK(metric_seg(mp, expect) == seg);
            for (int i = 0; i < 16; ++i)
                seen.insert(static_cast<uint32_t>(seg_step(seg)) * 64u + seg_group(seg, i));
            ++expect;
        }
        CHECK(expect * 16 == metric_groups(mp));
        CHECK((int)seen.size() == metric_groups(mp));
        for (int q = mp; q < mp + 8; q += 2)
            for (int seg = 0; seg < 6; ++seg)
                CHECK(seg_has_metric(q & 1, seg) == ((3 * q + seg_step(seg)) % 2 == 0));
        // ring sizes 8 V divide the positions of every super-step
        for (int V = 1; V <= 2; ++V) CHECK((metric_groups(mp) * V) % (8 * V) == 0);
    }
    if (fails) {
        std::printf("%d failures\n", fails);
        return 1;
    }
    std::printf("l16 layout ok\n");
    return 0;
}
