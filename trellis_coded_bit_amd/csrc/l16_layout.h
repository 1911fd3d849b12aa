// Register / lane / wave layout of the L = 16, k*V = 2 forward kernel.
//
// One workgroup of 8 waves holds the 2^16 path costs of one coding block, 128 per
// lane: slot (w, l, r) = (wave 0..7, lane 0..63, register 0..127).  The 16-bit state is
// read as eight base-4 digits, oldest (bits 15..14) first.  A "super-step" is three
// trellis steps; at its start the digits are placed as
//
//     digit 7 (oldest) A = r[5:4]     digit 3  n2 = w[2:1]
//     digit 6          B = r[3:2]     digit 2  (nh, z) = (l[5], r[6])
//     digit 5          C = r[1:0]     digit 1  r1 = l[3:2]
//     digit 4   n1 = (w[0], l[4])     digit 0  r2 = l[1:0]
//
// Step 1 of the super-step takes the minimum over A (the four predecessors of a group
// differ only in the oldest digit), and writes the four successors into the same four
// registers with the new digit in A's place; steps 2 and 3 do the same with B and C.
// After step p (p = 1, 2, 3) the state held by a slot is the digit sequence
// [A, B, C, n1, n2, D2, r1, r2] rotated left by p, D2 = 2 nh + z.  Every compare and
// select of the super-step therefore stays inside one lane.
//
// After three steps the oldest digits are n1, n2, D2 (in lanes, waves and z); a fixed
// bit permutation of (w, l, r) -- the "transposition", done through LDS -- brings them
// into A, B, C and restores the layout above for the next super-step.
#pragma once

#include <cstdint>

namespace tcq {
namespace l16 {

constexpr int kWaves = 8;
constexpr int kLanes = 64;
constexpr int kRegs = 128;
constexpr int kGroupsPerLane = 32;  // 128 registers / 4 successors

struct Slot {
    uint32_t w, l, r;
};

__host__ __device__ constexpr uint32_t bit(uint32_t x, int b) { return (x >> b) & 1u; }

// Digits [A, B, C, n1, n2, D2, r1, r2] of slot (w, l, r) at a super-step start.
__host__ __device__ constexpr uint32_t seq_digit(uint32_t w, uint32_t l, uint32_t r, int k) {
    return k == 0   ? (r >> 4) & 3u
           : k == 1 ? (r >> 2) & 3u
           : k == 2 ? r & 3u
           : k == 3 ? (bit(w, 0) << 1) | bit(l, 4)
           : k == 4 ? (w >> 1) & 3u
           : k == 5 ? (bit(l, 5) << 1) | bit(r, 6)
           : k == 6 ? (l >> 2) & 3u
                    : l & 3u;
}

// State held by slot (w, l, r) after p steps of the current super-step (p = 0..3).
__host__ __device__ constexpr uint32_t state_of(int p, uint32_t w, uint32_t l, uint32_t r) {
    uint32_t s = 0;
    for (int k = 0; k < 8; ++k) s = (s << 2) | seq_digit(w, l, r, (k + p) & 7);
    return s;
}

// Inverse of state_of.
__host__ __device__ constexpr Slot slot_of(int p, uint32_t s) {
    uint32_t seq[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < 8; ++k) {
        const uint32_t digit = (s >> (2 * (7 - k))) & 3u;  // k-th oldest digit
        seq[(k + p) & 7] = digit;
    }
    const uint32_t r = seq[2] | (seq[1] << 2) | (seq[0] << 4) | ((seq[5] & 1u) << 6);
    const uint32_t l = seq[7] | (seq[6] << 2) | ((seq[3] & 1u) << 4) | ((seq[5] >> 1) << 5);
    const uint32_t w = (seq[3] >> 1) | (seq[4] << 1);
    return Slot{w, l, r};
}

// Bit position (within r) of the digit replaced at step p of a super-step (p = 1..3).
__host__ __device__ constexpr int active_shift(int p) { return p == 1 ? 4 : (p == 2 ? 2 : 0); }

// Register of successor b of the lane's group g at step p: g's five bits fill the
// register bits other than the active digit, in ascending order.
__host__ __device__ constexpr uint32_t group_reg(int p, uint32_t g, uint32_t b) {
    const int a = active_shift(p);
    const uint32_t low = g & ((1u << a) - 1u);
    const uint32_t high = g >> a;
    return low | (b << a) | (high << (a + 2));
}

// Group index of register r at step p (inverse of group_reg in its first argument).
__host__ __device__ constexpr uint32_t reg_group(int p, uint32_t r) {
    const int a = active_shift(p);
    return (r & ((1u << a) - 1u)) | ((r >> (a + 2)) << a);
}

// ---------------------------------------------------------------------------------
// k*V = 3.  A super-step is two steps of three bits; the six register bits r[5:0]
// still hold the oldest six state bits at its start, so the layout above, the
// transposition and the LDS staging are unchanged.  After p steps the state is the
// start-of-super-step state rotated left by 3p bits.  Step 1 replaces r[5:3], step 2
// r[2:0]; a group is the 8 registers that differ in those bits.
// ---------------------------------------------------------------------------------
__host__ __device__ constexpr uint32_t rotl16(uint32_t s, int k) {
    k &= 15;
    return ((s << k) | (s >> ((16 - k) & 15))) & 0xFFFFu;
}
__host__ __device__ constexpr uint32_t state_of3(int p, uint32_t w, uint32_t l, uint32_t r) {
    return rotl16(state_of(0, w, l, r), 3 * p);
}
__host__ __device__ constexpr Slot slot_of3(int p, uint32_t s) {
    return slot_of(0, rotl16(s, 16 - ((3 * p) & 15)));
}
__host__ __device__ constexpr int active_shift3(int p) { return p == 1 ? 3 : 0; }
// register of successor b (0..7) of group g (0..15) at step p; g fills the other four
// register bits in ascending order
__host__ __device__ constexpr uint32_t group_reg3(int p, uint32_t g, uint32_t b) {
    const int a = active_shift3(p);
    const uint32_t low = g & ((1u << a) - 1u);
    const uint32_t high = g >> a;
    return low | (b << a) | (high << (a + 3));
}
__host__ __device__ constexpr uint32_t reg_group3(int p, uint32_t r) {
    const int a = active_shift3(p);
    return (r & ((1u << a) - 1u)) | ((r >> (a + 3)) << a);
}
// Segment order of a k*V = 3 super-step: four segments of 8 groups.
//   segment : 0      1      2       3
//   step    : 1      1      2       2
//   groups  : even   odd    0..7    8..15
// (step-1 groups split by r[0], the round of the preceding transposition; step-2
// groups by r[6], the round of the following one)
__host__ __device__ constexpr int seg3_step(int seg) { return seg < 2 ? 1 : 2; }
__host__ __device__ constexpr int seg3_half(int seg) { return seg & 1; }
__host__ __device__ constexpr uint32_t seg3_group(int seg, int i) {
    return seg < 2 ? 2u * i + (seg & 1) : 8u * (seg & 1) + i;
}
// backpointers: per lane and step two 32-bit words, 3 bits per group, the segment's
// first group in the top bits (bits 31..24 unused)
__host__ __device__ constexpr uint32_t bp3_half(int p, uint32_t g) {
    return p == 1 ? (g & 1u) : (g >> 3);
}
__host__ __device__ constexpr uint32_t bp3_shift(int p, uint32_t g) {
    return 3u * (7u - (p == 1 ? (g >> 1) : (g & 7u)));
}

// Processing order of a super-step: six segments of 16 groups each.  Splitting steps
// 1 and 2 by the parity of g (= bit 0 of the register, = the LDS round of the
// preceding transposition) lets half the trellis advance two steps while the other
// half is still in transit; step 3 is split by g < 16 (= r[6], the round of the
// following transposition) so the first half can be written out early.
//   segment : 0      1      2      3      4      5
//   step    : 1      2      1      2      3      3
//   groups  : even   even   odd    odd    0..15  16..31
__host__ __device__ constexpr int seg_step(int seg) {
    return (seg == 0 || seg == 2) ? 1 : ((seg == 1 || seg == 3) ? 2 : 3);
}
__host__ __device__ constexpr int seg_half(int seg) {
    return (seg == 0 || seg == 1 || seg == 4) ? 0 : 1;
}
// i-th group (i = 0..15) of a segment
__host__ __device__ constexpr uint32_t seg_group(int seg, int i) {
    return seg_step(seg) == 3 ? 16u * seg_half(seg) + i : 2u * i + seg_half(seg);
}
// Backpointer word of step p: per lane two 32-bit words (halves), 2 bits per group,
// the segment's first group in the top bits.
__host__ __device__ constexpr uint32_t bp_half(int p, uint32_t g) {
    return p == 3 ? (g >> 4) : (g & 1u);
}
__host__ __device__ constexpr uint32_t bp_shift(int p, uint32_t g) {
    return 2u * (15u - (p == 3 ? (g & 15u) : (g >> 1)));
}

// ---------------------------------------------------------------------------------
// k*V = 4 run as 2-bit half-steps (kernels_l16h.hip) on a relabelled state: bits [3:2]
// and [1:0] of every nibble exchanged.  The map is a permutation of bit positions, so
// it is its own inverse and the image of an OR is the OR of the images.
// ---------------------------------------------------------------------------------
__host__ __device__ constexpr uint32_t nibble_halves_swap(uint32_t x) {
    return ((x & 0x33333333u) << 2) | ((x >> 2) & 0x33333333u);
}

// ---------------------------------------------------------------------------------
// k*V = 4 run as 2-bit half-steps (kernels_l16h.hip): super-step q covers half-steps
// 3q + 1 .. 3q + 3 and the metric sits on the even ones, i.e. on step P of the
// super-step when q + P is even.  MP = q mod 2 is the super-step's pattern.
// ---------------------------------------------------------------------------------
// Metric groups of a super-step in processing order.  MP = q mod 2.
//   MP = 0: step 2 only  -> segments 1, 3          (32 groups)
//   MP = 1: steps 1 and 3 -> segments 0, 2, 4, 5   (64 groups)
__host__ __device__ constexpr int metric_groups(int mp) { return mp ? 64 : 32; }
__host__ __device__ constexpr int metric_seg(int mp, int j) {
    return mp ? (j == 0 ? 0 : (j == 1 ? 2 : (j == 2 ? 4 : 5))) : (j == 0 ? 1 : 3);
}
// does segment SEG of a super-step with pattern MP carry the metric?
__host__ __device__ constexpr bool seg_has_metric(int mp, int seg) {
    return ((seg_step(seg) + mp) & 1) == 0;
}
// index of segment SEG among the metric segments of pattern MP
__host__ __device__ constexpr int metric_index(int mp, int seg) {
    return mp ? (seg == 0 ? 0 : (seg == 2 ? 1 : (seg == 4 ? 2 : 3))) : (seg == 1 ? 0 : 1);
}


// k*V = 4: a step-1 segment and the step-2 segment after it (segments 0-1 or 2-3, one
// of them a plain half-step) are processed as one interleaved sequence of 32 groups.
// Step-2 group j reads the registers that step-1 groups C + 4b + 16 r[6] wrote (C its
// two low register bits), i.e. groups 0..7 for j < 8 and 8..15 for j >= 8, so: step-1
// groups 0..7; then step-2 group j and step-1 group 8 + j in turn (j = 0..7); then
// step-2 groups 8..15.  Slot k (0..31) holds the group pair_index(k) of half-step
// pair_step(k) (1 or 2).
__host__ __device__ constexpr int pair_step(int k) {
    return k < 8 ? 1 : (k < 24 ? ((k - 8) % 2 == 0 ? 2 : 1) : 2);
}
__host__ __device__ constexpr int pair_index(int k) {
    return k < 8 ? k : (k < 24 ? ((k - 8) % 2 == 0 ? (k - 8) / 2 : 8 + (k - 8) / 2) : k - 16);
}

// Register naming.  Odd super-steps keep logical register r in physical register
// phys(1, r) = r with bits 0 and 6 swapped.  A transposition round then refills exactly
// the physical registers it has just written out: round 0 moves logical r[6] = 0 into
// logical r'[0] = 0, and phys(m, {r[6] = 0}) = phys(1 - m, {r'[0] = 0}) for m = 0, 1.
__host__ __device__ constexpr uint32_t phys(int naming, uint32_t r) {
    return naming ? ((r & 0x3Eu) | (bit(r, 0) << 6) | bit(r, 6)) : r;
}

// Destination of the value in slot (w, l, r) at the end of a super-step (p = 3).
__host__ __device__ constexpr Slot transpose_dest(uint32_t w, uint32_t l, uint32_t r) {
    const uint32_t rn = bit(r, 6) | (bit(l, 5) << 1) | (bit(w, 1) << 2) | (bit(w, 2) << 3) |
                        (bit(l, 4) << 4) | (bit(w, 0) << 5) | (bit(r, 4) << 6);
    const uint32_t ln = bit(r, 0) | (bit(r, 1) << 1) | (bit(r, 2) << 2) | (bit(r, 3) << 3) |
                        (bit(l, 2) << 4) | (bit(r, 5) << 5);
    const uint32_t wn = bit(l, 3) | (bit(l, 0) << 1) | (bit(l, 1) << 2);
    return Slot{wn, ln, rn};
}

// LDS staging of the transposition: two rounds, split on r[6] of the source (= bit 0
// of the destination register).  Within a round a value's dword address is
//     l2 + 2 * (33 * row + col) + 2112 * other
// with row = l0 + 2 l1 + 4 l3 + 8 l4 + 16 l5, col = r0 + 2 r1 + 4 r2 + 8 r3 + 16 r5,
// other = w0 + 2 w1 + 4 w2 + 8 r4 (source coordinates).  The padding (33 instead of 32)
// makes every write and every read of a wave touch 64 different banks, and each half
// wave 32 different banks.
constexpr uint32_t kLdsDwords = 2112u * 16u;  // one round: 33792 dwords = 132 KiB

__host__ __device__ constexpr uint32_t lds_write_lane(uint32_t w, uint32_t l) {
    const uint32_t row = bit(l, 0) | (bit(l, 1) << 1) | (bit(l, 3) << 2) | (bit(l, 4) << 3) |
                         (bit(l, 5) << 4);
    return bit(l, 2) + 66u * row + 2112u * (bit(w, 0) | (bit(w, 1) << 1) | (bit(w, 2) << 2));
}
__host__ __device__ constexpr uint32_t lds_write_reg(uint32_t r) {
    const uint32_t col = bit(r, 0) | (bit(r, 1) << 1) | (bit(r, 2) << 2) | (bit(r, 3) << 3) |
                         (bit(r, 5) << 4);
    return 2u * col + 2112u * 8u * bit(r, 4);
}
// The same address expressed in destination coordinates (w', l', r').
__host__ __device__ constexpr uint32_t lds_read_lane(uint32_t w, uint32_t l) {
    const uint32_t col = bit(l, 0) | (bit(l, 1) << 1) | (bit(l, 2) << 2) | (bit(l, 3) << 3) |
                         (bit(l, 5) << 4);
    const uint32_t rowpart = bit(w, 1) | (bit(w, 2) << 1) | (bit(w, 0) << 2);
    return bit(l, 4) + 2u * col + 66u * rowpart;
}
__host__ __device__ constexpr uint32_t lds_read_reg(uint32_t r) {
    const uint32_t rowpart = (bit(r, 4) << 3) | (bit(r, 1) << 4);
    const uint32_t other = bit(r, 5) | (bit(r, 2) << 1) | (bit(r, 3) << 2) | (bit(r, 6) << 3);
    return 66u * rowpart + 2112u * other;
}

}  // namespace l16
}  // namespace tcq
