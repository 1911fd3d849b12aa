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
//    every metric group once, in processing order;
//  - the k*V = 4 relabelling of the state commutes with the shift and makes the two
//    half-step minima pick the lowest predecessor index;
//  - the transposition rounds spread over the segments touch no register the segment
//    they run in uses, refill exactly the registers they freed, and the k*V = 4
//    kernel's interleaved segment pairs respect every register dependency.
#define __host__
#define __device__
#include <cstdio>
#include <cstdlib>
#include <set>
#include <utility>
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


// Registers (physical, one lane) of a group of 2-bit step p and of 3-bit step p under
// naming nm.
static std::set<uint32_t> group_regs2(int nm, int p, uint32_t g) {
    std::set<uint32_t> out;
    for (uint32_t b = 0; b < 4; ++b) out.insert(phys(nm, group_reg(p, g, b)));
    return out;
}
static std::set<uint32_t> group_regs3(int nm, int p, uint32_t g) {
    std::set<uint32_t> out;
    for (uint32_t b = 0; b < 8; ++b) out.insert(phys(nm, group_reg3(p, g, b)));
    return out;
}
static bool disjoint(const std::set<uint32_t> &a, const std::set<uint32_t> &b) {
    for (uint32_t x : a)
        if (b.count(x)) return false;
    return true;
}

// The transposition rounds spread over the segments (kernels_l16*.hip, l16_device.h):
// the registers a round writes out while a segment runs are not touched by that
// segment's groups, the registers a round reads back are exactly those it freed, and in
// the k*V = 4 kernel's interleaved segment pairs every step-2 group comes after the
// step-1 groups whose registers it reads, with no later step-1 group writing them.
static void check_spread_rounds() {
    for (int nm = 0; nm < 2; ++nm) {
        // round 1 of the previous transposition: logical r[6] = 1 of naming 1 - nm
        std::set<uint32_t> r1w, r0w, r1r, r0r;
        for (uint32_t i = 0; i < 64; ++i) r1w.insert(phys(1 - nm, 64 + i));
        for (uint32_t i = 0; i < 64; ++i) r0w.insert(phys(nm, i));
        for (uint32_t g2 = 0; g2 < 16; ++g2)
            for (uint32_t b = 0; b < 4; ++b) {
                // round_read_group<1 - nm, 1, g2> and <nm, 0, g2> targets
                r1r.insert(phys(nm, group_reg(1, 2 * g2 + 1, b)));
                r0r.insert(phys(1 - nm, group_reg(1, 2 * g2, b)));
            }
        CHECK(r1w == r1r);  // round 1 refills exactly the registers it wrote out
        CHECK(r0w == r0r);  // so does round 0
        // k*V = 2 and 4: segments 0-1 (steps 1-2, even groups) while round 1 is written;
        // segment 2 (step 1, odd groups) refills round 1
        for (int seg = 0; seg < 2; ++seg)
            for (int i = 0; i < 16; ++i)
                CHECK(disjoint(group_regs2(nm, seg_step(seg), seg_group(seg, i)), r1w));
        // segment 4 (step 3, groups 0..15) writes round 0 one group behind: group I's
        // registers are logical 4I .. 4I + 3, and no later group of segments 4-5 uses them
        for (uint32_t g = 0; g < 16; ++g) {
            std::set<uint32_t> own;
            for (uint32_t b = 0; b < 4; ++b) own.insert(phys(nm, 4 * g + b));
            CHECK(own == group_regs2(nm, 3, seg_group(4, g)));
            for (uint32_t h = g + 1; h < 32; ++h)
                CHECK(disjoint(own, group_regs2(nm, 3, h)));
        }
        // segment 5 (step 3, groups 16..31) while round 0 is read back
        for (int i = 0; i < 16; ++i)
            CHECK(disjoint(group_regs2(nm, 3, seg_group(5, i)), r0r));
        // k*V = 3: segment 0 (step 1, even groups) while round 1 is written; segment 2
        // (step 2, groups 0..7) writes round 0 one group behind (group g = registers
        // 8g .. 8g + 7); segment 3 (groups 8..15) while round 0 is read back
        for (int i = 0; i < 8; ++i) {
            CHECK(disjoint(group_regs3(nm, 1, seg3_group(0, i)), r1w));
            std::set<uint32_t> own;
            for (uint32_t b = 0; b < 8; ++b) own.insert(phys(nm, 8 * i + b));
            CHECK(own == group_regs3(nm, 2, seg3_group(2, i)));
            CHECK(disjoint(group_regs3(nm, 2, seg3_group(3, i)), r0r));
        }
        std::set<uint32_t> r1r3;
        for (int i = 0; i < 8; ++i)
            for (uint32_t b = 0; b < 8; ++b) r1r3.insert(phys(nm, group_reg3(1, seg3_group(1, i), b)));
        CHECK(r1r3 == r1w);
        // k*V = 4 segment pairs (SA = 0: even groups, 2: odd): order of the 32 groups
        for (int sa = 0; sa <= 2; sa += 2) {
            std::vector<std::pair<int, int>> order;  // (step, index within its segment)
            for (int k = 0; k < 32; ++k) order.push_back({pair_step(k), pair_index(k)});
            std::vector<int> pos1(16, -1), pos2(16, -1);
            for (int k = 0; k < 32; ++k) (order[k].first == 1 ? pos1 : pos2)[order[k].second] = k;
            for (int i = 0; i < 16; ++i) CHECK(pos1[i] >= 0 && pos2[i] >= 0);
            for (int i = 1; i < 16; ++i) CHECK(pos1[i] > pos1[i - 1] && pos2[i] > pos2[i - 1]);
            for (int j = 0; j < 16; ++j) {
                const auto rd = group_regs2(nm, 2, seg_group(sa + 1, j));
                for (int i = 0; i < 16; ++i) {
                    const auto wr = group_regs2(nm, 1, seg_group(sa, i));
                    // a step-1 group sharing registers with step-2 group j comes first
                    if (!disjoint(rd, wr)) CHECK(pos1[i] < pos2[j]);
                }
            }
            if (sa == 2) {
                // round 1 is read into step-1 group i + 3 before step-1 group i: no group
                // placed between the read and step-1 group i + 3 touches its registers
                for (int i = 0; i + 3 < 16; ++i) {
                    const auto tgt = group_regs2(nm, 1, seg_group(sa, i + 3));
                    for (int k = pos1[i]; k < pos1[i + 3]; ++k) {
                        const auto &o = order[k];
                        const auto regs = group_regs2(nm, o.first, seg_group(sa + o.first - 1, o.second));
                        CHECK(disjoint(regs, tgt));
                    }
                }
            }
        }
    }
}

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
    // k*V = 4 relabelling P (halves of every nibble exchanged): an involution that
    // commutes with the 4-bit shift, so the relabelled trellis has the same paths; its
    // first half-step drops j_lo (bits 13:12 of the true state), the second j_hi.
    for (uint32_t s = 0; s < (1u << 16); ++s) {
        CHECK(nibble_halves_swap(nibble_halves_swap(s)) == s);
        CHECK((nibble_halves_swap(s) >> 14) == ((s >> 12) & 3u));
        CHECK(((nibble_halves_swap(s) >> 12) & 3u) == (s >> 14));
        for (uint32_t b = 0; b < 16; ++b)
            CHECK(nibble_halves_swap(((s << 4) | b) & 0xFFFFu) ==
                  (((nibble_halves_swap(s) << 4) | nibble_halves_swap(b)) & 0xFFFFu));
    }
    // Two-stage minimum over j = 4 j_hi + j_lo: first, per j_hi, the lowest j_lo of
    // minimum cost; then the lowest j_hi of minimum cost.  It picks the lowest j of
    // minimum cost, for every cost vector with values in {0, 1, 2} on a 16-way group
    // (sampled: the 2^16 vectors over {0, 1} and 3^8 patterns spread over the group).
    auto check_two_stage = [&](const int (&c)[16]) {
        int best = 0;
        for (int j = 1; j < 16; ++j)
            if (c[j] < c[best]) best = j;
        int m1[4], a1[4];
        for (int hi = 0; hi < 4; ++hi) {
            a1[hi] = 0;
            for (int lo = 1; lo < 4; ++lo)
                if (c[4 * hi + lo] < c[4 * hi + a1[hi]]) a1[hi] = lo;
            m1[hi] = c[4 * hi + a1[hi]];
        }
        int hi_best = 0;
        for (int hi = 1; hi < 4; ++hi)
            if (m1[hi] < m1[hi_best]) hi_best = hi;
        CHECK(4 * hi_best + a1[hi_best] == best);
    };
    for (uint32_t m = 0; m < (1u << 16); ++m) {
        int c[16];
        for (int j = 0; j < 16; ++j) c[j] = (m >> j) & 1u;
        check_two_stage(c);
    }
    for (uint32_t m = 0; m < 6561; ++m) {
        int c[16];
        uint32_t t = m;
        for (int j = 0; j < 8; ++j) {
            c[2 * j] = t % 3;
            c[2 * j + 1] = (t % 3 + j) % 3;
            t /= 3;
        }
        check_two_stage(c);
    }
    check_spread_rounds();
    if (fails) {
        std::printf("%d failures\n", fails);
        return 1;
    }
    std::printf("l16 layout ok\n");
    return 0;
}
