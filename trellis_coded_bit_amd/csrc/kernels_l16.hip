// L = 16, k*V = 2, V = 1 forward kernel: the coding block's 2^16 path costs live in
// VGPRs (128 per lane, one 8-wave workgroup per block), every add-compare-select of a
// step happens inside a lane, and the cost vector is re-laid out through LDS once
// every three steps (layout and proofs of its index math: l16_layout.h).
//
// The step (Pingala-8 post, Viterbi paragraph; bitshift structure from the QTIP
// abstract; d-weighted branch metric from the CurveTQ abstract):
//   predecessors of group x are (j << 14) | x, j = 0..3; keep the smallest cost, lowest
//   j on ties; successor (x << 2) | b gets  fmaf(fl(d * e), e, m), e = fl(w - C[s']).
// All states start at cost +0, which is the free start (see kernels_generic.hip).
//
// Codebook: per step, each lane needs the four successor values of each of its 32
// groups.  A prepare kernel writes three permuted copies of the table (one per step of
// the super-step) so that these reads are one coalesced 16-byte load per lane per group
// from an L2-resident 768 KiB array.
#include <hip/hip_runtime.h>

#include "l16_device.h"
#include "l16_layout.h"
#include "tcq.h"
#include "tcq_internal.h"

#include <utility>

namespace tcq {
namespace {

using namespace l16;

// Context with the backpointer words addressed through a buffer descriptor (lane offset in
// a register, step and half in the scalar offset): no 64-bit address per store.
struct CtxL : Ctx {
    BpBuf bpb;
};

// Groups of codebook in flight.  Measured on MI355X with the transposition rounds spread
// over the segments: 12 deep for both searches (a 16-deep ring leaves the weighted
// kernel short of registers, and it spills in the loop: 193.5 against 172.1 ms at
// 4096 x 4096; at d = 1 16 deep gains nothing).
template <bool WEIGHTED>
constexpr int kRing = 12;

__global__ __launch_bounds__(256) void l16_prepare_kernel(const float *__restrict__ C,
                                                          float4 *__restrict__ out) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 3 * kCopy) return;
    const int p = idx / kCopy + 1;
    const int rem = idx % kCopy;
    const uint32_t w = rem / (kGroupsPerLane * kLanes);
    const uint32_t g = (rem / kLanes) % kGroupsPerLane;
    const uint32_t l = rem % kLanes;
    const uint32_t s = state_of(p, w, l, group_reg(p, g, 0));  // successor with b = 0
    const float *src = C + s;                                // s, s+1, s+2, s+3
    out[idx] = make_float4(src[0], src[1], src[2], src[3]);
}

// Codebook copy entry for group g of step P: a raw buffer load whose per-lane offset
// (voff = 16 * lane) is shared by every load and whose group/step offset is a scalar.
// The low part of the offset ((g mod 4) KiB) goes to the instruction's immediate field,
// so a super-step needs only 24 distinct scalar offsets.
template <int P>
__device__ __forceinline__ float4 cb_load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int g) {
    constexpr int kEntry = static_cast<int>(sizeof(float4));
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        rs, voff + (g & 3) * kLanes * kEntry, ((P - 1) * kCopy + (g & ~3) * kLanes) * kEntry, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}

// The codebook entries are consumed in the fixed segment order of a super-step
// (position k = 16 * segment + i, 96 per super-step); a ring of D loads runs
// ahead of the consumer, across segment and super-step boundaries.
constexpr int kPositions = 96;
// the ring runs across super-steps: position k lives in slot k mod D in every
// super-step only if the ring size divides the positions per super-step
static_assert(kPositions % kRing<false> == 0 && kPositions % kRing<true> == 0,
              "ring size must divide a super-step");

template <int K>
__device__ __forceinline__ float4 cb_load_pos(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    constexpr int k = K % kPositions;
    return cb_load<seg_step(k / 16)>(rs, voff, seg_group(k / 16, k % 16));
}

template <int K0, int D, int... I>
__device__ __forceinline__ void ring_prime(float4 (&ring)[D], __amdgpu_buffer_rsrc_t rs,
                                           uint32_t voff, std::integer_sequence<int, I...>) {
    ((ring[(K0 + I) % D] = cb_load_pos<K0 + I>(rs, voff)), ...);
}

// Fill the ring with positions K0 .. K0 + D - 1.
template <int K0, int D>
__device__ __forceinline__ void ring_fill(float4 (&ring)[D], __amdgpu_buffer_rsrc_t rs,
                                          uint32_t voff) {
    ring_prime<K0>(ring, rs, voff, std::make_integer_sequence<int, D>{});
}

// Path costs are non-negative floats (sums of d * e * e >= 0 starting from +0, never
// -0), so their bit patterns order exactly like their values: minima and compares run
// on the unsigned bit patterns, which needs no NaN canonicalization.
//
// One group (I-th of segment SEG) under register naming NM.  `wt`/`dt` are the step's
// weight and d; two backpointer bits are shifted into `acc`.
template <int SEG, bool WEIGHTED, int NM, int I>
__device__ __forceinline__ void acs_group(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                          __amdgpu_buffer_rsrc_t rs, uint32_t voff, float wt,
                                          float dt, uint32_t &acc) {
    constexpr int P = seg_step(SEG);
    constexpr int k = 16 * SEG + I;
    constexpr uint32_t g = seg_group(SEG, I);
    // at most kRing codebook loads in flight: later loads stay below this point
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    constexpr int D = kRing<WEIGHTED>;
    const float4 c = ring[k % D];
    ring[k % D] = cb_load_pos<k + D>(rs, voff);
    constexpr int r0 = phys(NM, group_reg(P, g, 0)), r1 = phys(NM, group_reg(P, g, 1));
    constexpr int r2 = phys(NM, group_reg(P, g, 2)), r3 = phys(NM, group_reg(P, g, 3));
    const uint32_t u0 = J[r0], u1 = J[r1], u2 = J[r2], u3 = J[r3];
    uint64_t chi, b0;
    const uint32_t mu = argmin4(u0, u1, u2, u3, chi, b0);
    acc = shift_in(shift_in(acc, chi), b0);
    const float m = __uint_as_float(mu);
    const float e0 = wt - c.x, e1 = wt - c.y, e2 = wt - c.z, e3 = wt - c.w;
    J[r0] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e0 : e0, e0, m));
    J[r1] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e1 : e1, e1, m));
    J[r2] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e2 : e2, e2, m));
    J[r3] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e3 : e3, e3, m));
}

template <int SEG, bool WEIGHTED, int NM, int... I>
__device__ __forceinline__ void acs_segment_impl(uint32_t (&J)[kRegs],
                                                 float4 (&ring)[kRing<WEIGHTED>],
                                                 __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                 float wt, float dt, const BpBuf &bpb,
                                                 int bp_word, std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    (acs_group<SEG, WEIGHTED, NM, I>(J, ring, rs, voff, wt, dt, acc), ...);
    bpb.store(bp_word, acc);
}

template <int SEG, bool WEIGHTED, int NM>
__device__ __forceinline__ void acs_segment(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                            const CtxL &cx, int t0, const StepIn &in) {
    constexpr int P = seg_step(SEG);
    const int t = t0 + P - 1;  // 0-based step index
    acs_segment_impl<SEG, WEIGHTED, NM>(J, ring, cx.rs, cx.voff, in.w[P - 1], in.d[P - 1],
                                        cx.bpb, 2 * kThreads * t + seg_half(SEG),
                                        std::make_integer_sequence<int, 16>{});
}

template <int SEG, bool WEIGHTED, int NM, class X, int... I>
__device__ __forceinline__ void acs_segment_x_impl(uint32_t (&J)[kRegs],
                                                   float4 (&ring)[kRing<WEIGHTED>],
                                                   const CtxL &cx, float wt, float dt,
                                                   int bp_word, const X &x,
                                                   std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    ((acs_group<SEG, WEIGHTED, NM, I>(J, ring, cx.rs, cx.voff, wt, dt, acc),
      x.template step<I>(J, cx)),
     ...);
    cx.bpb.store(bp_word, acc);
}
// acs_segment with LDS work X interleaved.
template <int SEG, bool WEIGHTED, int NM, class X>
__device__ __forceinline__ void acs_segment_x(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                              const CtxL &cx, int t0, const StepIn &in,
                                              const X &x) {
    constexpr int P = seg_step(SEG);
    const int t = t0 + P - 1;
    acs_segment_x_impl<SEG, WEIGHTED, NM>(J, ring, cx, in.w[P - 1], in.d[P - 1],
                                          2 * kThreads * t + seg_half(SEG), x,
                                          std::make_integer_sequence<int, 16>{});
}
// Segment 2 (step 1 of the odd groups) with round 1 of the transposition read into the
// registers it consumes: the four values of group i + kReadAhead are requested before
// group i is computed, so at most 4 * (kReadAhead + 1) reads are in flight (the LDS
// wait counter counts at most 15) and each group waits only for its own values.
constexpr int kReadAhead = 3;
template <bool WEIGHTED, int NM, int I>
__device__ __forceinline__ void seg2_group(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                           const CtxL &cx, float wt, float dt, uint32_t &acc) {
    if constexpr (I + kReadAhead < 16) round_read_group<1 - NM, 1, I + kReadAhead>(J, cx);
    acs_group<2, WEIGHTED, NM, I>(J, ring, cx.rs, cx.voff, wt, dt, acc);
}
template <bool WEIGHTED, int NM, int... I>
__device__ __forceinline__ void seg2_reading(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                             const CtxL &cx, int t0, const StepIn &in,
                                             std::integer_sequence<int, I...>) {
    round_read_groups<1 - NM, 1>(J, cx, std::make_integer_sequence<int, kReadAhead>{});
    uint32_t acc = 0;
    (seg2_group<WEIGHTED, NM, I>(J, ring, cx, in.w[0], in.d[0], acc), ...);
    cx.bpb.store(2 * kThreads * t0 + seg_half(2), acc);
}

// Super-step (steps t0+1 .. t0+3) under naming NM, with the weights (and d) of its three
// steps in `in`; those of the next super-step are requested into `next`.  On entry the
// even registers hold round 0 of the previous transposition, and round 1 of it is still
// in the registers of naming 1 - NM with r[6] = 1 (the odd groups of this naming, which
// segments 0 and 1 do not touch): segments 0 and 1 write it to LDS as they go, segment 2
// reads it back group by group.  Segment 4 (step 3 of the r[6] = 0 half) writes round 0
// of this super-step's transposition as its groups finish, and segment 5 (the r[6] = 1
// half) reads it back into the same registers.  On exit round 1 is left in registers
// for the next super-step (or the tail) to write.
template <bool WEIGHTED, int NM>
__device__ __forceinline__ void super_step(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                           const CtxL &cx, int t0, const StepIn &in,
                                           StepIn &next) {
    acs_segment_x<0, WEIGHTED, NM>(J, ring, cx, t0, in, WriteLds<1 - NM, 1, 2, 0>{});
    acs_segment_x<1, WEIGHTED, NM>(J, ring, cx, t0, in, WriteLds<1 - NM, 1, 2, 32>{});
    __syncthreads();  // round-1 values written by every wave
    seg2_reading<WEIGHTED, NM>(J, ring, cx, t0, in, std::make_integer_sequence<int, 16>{});
    acs_segment<3, WEIGHTED, NM>(J, ring, cx, t0, in);
    __syncthreads();  // every wave has read round 1
    acs_segment_x<4, WEIGHTED, NM>(J, ring, cx, t0, in, WriteRound0Lagged<NM, 4>{});
    round_write_range<NM, 0, 60, 4>(J, cx);
    next = load_steps<WEIGHTED>(cx, t0 + 3);  // complete by the barrier below
    __syncthreads();  // round-0 values written by every wave
    acs_segment_x<5, WEIGHTED, NM>(J, ring, cx, t0, in, ReadLds<NM, 0, 1>{});
    __syncthreads();  // every wave has read round 0
}

// The last R = 1 or 2 steps (segments 0..3 in order; for one step the ring is refilled
// where the order departs from a full super-step), under naming NM.  Round 1 of the last
// transposition (naming 1 - NM) is written first, in one go (this runs once per block).
template <bool WEIGHTED, int NM, int R>
__device__ __forceinline__ void tail_steps(uint32_t (&J)[kRegs], float4 (&ring)[kRing<WEIGHTED>],
                                           const CtxL &cx, int t0, const StepIn &in) {
    round_write<1 - NM, 1>(J, cx);
    acs_segment<0, WEIGHTED, NM>(J, ring, cx, t0, in);
    if constexpr (R == 2) acs_segment<1, WEIGHTED, NM>(J, ring, cx, t0, in);
    __syncthreads();
    round_read<1 - NM, 1>(J, cx);
    if constexpr (R == 1) ring_fill<32>(ring, cx.rs, cx.voff);
    acs_segment<2, WEIGHTED, NM>(J, ring, cx, t0, in);
    if constexpr (R == 2) acs_segment<3, WEIGHTED, NM>(J, ring, cx, t0, in);
}

// Register part of the state a register holds after step P of a super-step, and the
// lane's lowest (cost, state).
template <int P>
struct lane_argmin_key {
    static constexpr uint32_t of(int r) {
        return state_of(P, 0, 0, static_cast<uint32_t>(r));
    }
};
template <int P, int NM>
__device__ __forceinline__ void lane_argmin(const uint32_t (&J)[kRegs], uint32_t w,
                                            uint32_t l, uint32_t &bv, uint32_t &bi) {
    lane_best<lane_argmin_key<P>, NM>(J, state_of(P, w, l, 0), bv, bi);
}

// R = n mod 3, the steps after the last whole super-step: a template argument, so that
// each instantiation has one tail (with the three tails in one kernel the compiler merged
// their register assignments and spilled to scratch at the joins).
template <bool WEIGHTED, int R>
__global__ __launch_bounds__(kThreads, 1) void acs_l16_kernel(
    const float *__restrict__ W, int64_t ldw, const float *__restrict__ d,
    const float4 *__restrict__ cb, int n, int64_t blocks_per_row, int64_t block0,
    uint2 *__restrict__ bp, int64_t bp_per_block, uint32_t *__restrict__ send,
    float *__restrict__ cost_out) {
    const uint32_t tid = threadIdx.x;
    const uint32_t w = tid >> 6;
    const uint32_t l = tid & 63;
    const int64_t blk = block0 + blockIdx.x;
    const int64_t row = blk / blocks_per_row;
    const int64_t col = blk % blocks_per_row;

    CtxL cx;
    static_cast<Ctx &>(cx) = make_ctx(W, ldw, WEIGHTED ? d : nullptr, cb, n, row, col, w, l,
                                      bp + blockIdx.x * bp_per_block);
    cx.bpb = make_bpbuf(bp + blockIdx.x * bp_per_block, bp_per_block, w, l);

    uint32_t J[kRegs];  // fp32 costs held as their bit patterns
#pragma unroll
    for (int r = 0; r < kRegs; ++r) J[r] = 0u;
    float4 ring[kRing<WEIGHTED>];
    ring_fill<0>(ring, cx.rs, cx.voff);

    // Every super-step ends with a transposition whose second round is written and read
    // during the next one; the all-zero start is staged the same way (whatever registers
    // the first super-step writes out hold zeros), so all super-steps run the same
    // branch-free code.  Super-steps alternate between namings 1 and 0 so that the last
    // one runs under naming 1 and the tail under naming 0.
#pragma unroll
    for (int r = 0; r < kRegs; ++r) asm volatile("" : "+v"(J[r]));  // keep the zeros opaque
    const int Q = n / 3;  // n % 3 == R: the launcher picks the instantiation
    StepIn in = load_steps<WEIGHTED>(cx, 0);
    if (Q & 1) {
        StepIn next;
        super_step<WEIGHTED, 1>(J, ring, cx, 0, in, next);
        in = next;
    }
    for (int q = Q & 1; q < Q; q += 2) {
        StepIn mid, next;
        super_step<WEIGHTED, 0>(J, ring, cx, 3 * q, in, mid);
        super_step<WEIGHTED, 1>(J, ring, cx, 3 * q + 3, mid, next);
        in = next;
    }
    if constexpr (R == 1) {
        tail_steps<WEIGHTED, 0, 1>(J, ring, cx, 3 * Q, in);
    } else if constexpr (R == 2) {
        tail_steps<WEIGHTED, 0, 2>(J, ring, cx, 3 * Q, in);
    } else {
        round_write<1, 1>(J, cx);  // the last round (zeros if there was no super-step)
        __syncthreads();
        round_read<1, 1>(J, cx);
    }

    uint32_t bv = 0xFFFFFFFFu;  // above every finite or infinite cost pattern
    uint32_t bi = 0xFFFFFFFFu;
    // final layout: step R of a super-step (R = 0: its start) under naming 0
    lane_argmin<R, 0>(J, w, l, bv, bi);
    block_select(bv, bi, w, l, send + blockIdx.x, cost_out + blk);
}

// Remembered predecessor index j of state s at step t (1-based): s_{t-1} = (j << 14) |
// (s >> 2).
__device__ __forceinline__ uint32_t bp_choice(const uint2 *bpb, int t, uint32_t s) {
    const int p = (t - 1) % 3 + 1;
    const Slot sl = slot_of(p, s);
    const uint32_t g = reg_group(p, sl.r);
    const uint2 word = bpb[(t - 1) * kThreads + sl.w * kLanes + sl.l];
    const uint32_t bits = bp_half(p, g) ? word.y : word.x;
    return (bits >> bp_shift(p, g)) & 3u;
}

// One wave per block: follow the remembered predecessors back from the end state and
// pack the 2-bit chunks b_1..b_n, MSB first, into MSB-first words.  n counts 2-bit
// steps: the half-step view of k*V = 4 has twice the steps of the block, up to
// 2 * TCQ_MAX_STEPS.  With swap_halves (the relabelled trellis of the k*V = 4 kernel,
// whose state has the two halves of every nibble exchanged) the end state is given as a
// true state and converted first, and the start state and every packed word are
// converted back at the end.  Three steps per memory round trip: with s_t known, lane 0 reads
// the choice at step t for s_t, lanes 1..4 the choice at step t-1 for each of the four
// possible s_{t-1}, and lanes 5..20 the choice at step t-2 for each of the sixteen
// possible s_{t-2}; the three reads are independent, and the wave then picks the path
// they determine.  (Four blocks per 256-thread workgroup were slower: 497 against
// 470 us at 16384 blocks of 256 steps.)
__global__ __launch_bounds__(64) void traceback_l16_kernel(
    const uint2 *__restrict__ bp, int64_t bp_per_block, const uint32_t *__restrict__ send,
    int n, int nwords, int64_t block0, uint32_t *__restrict__ bitstream,
    uint32_t *__restrict__ start_state, int swap_halves) {
    __shared__ uint8_t chunk[2 * TCQ_MAX_STEPS];
    const int lane = threadIdx.x;
    const uint2 *bpb = bp + blockIdx.x * bp_per_block;
    const int64_t blk = block0 + blockIdx.x;
    uint32_t s = send[blockIdx.x];  // s_t, the same in every lane
    if (swap_halves) s = nibble_halves_swap(s);
    int t = n;
    while (t >= 1) {
        // this lane's candidate: level 0 is s_t itself, level 1 s_{t-1} = (j0 << 14) |
        // (s_t >> 2), level 2 s_{t-2} = (j1 << 14) | (s_{t-1} >> 2)
        int lvl = -1;
        uint32_t c = 0;
        if (lane == 0) {
            lvl = 0;
            c = s;
        } else if (lane < 5) {
            lvl = 1;
            c = (static_cast<uint32_t>(lane - 1) << 14) | (s >> 2);
        } else if (lane < 21) {
            lvl = 2;
            const uint32_t j0 = static_cast<uint32_t>(lane - 5) >> 2;
            const uint32_t j1 = static_cast<uint32_t>(lane - 5) & 3u;
            c = (j1 << 14) | (((j0 << 14) | (s >> 2)) >> 2);
        }
        uint32_t jb = 0;
        if (lvl >= 0 && t - lvl >= 1) jb = bp_choice(bpb, t - lvl, c);
        const uint32_t j0 = __builtin_amdgcn_readlane(jb, 0);
        if (lane == 0) chunk[t - 1] = static_cast<uint8_t>(s & 3u);
        const uint32_t s1 = (j0 << 14) | (s >> 2);
        if (t == 1) {
            s = s1;
            break;
        }
        const uint32_t j1 = __builtin_amdgcn_readlane(jb, 1 + static_cast<int>(j0));
        if (lane == 0) chunk[t - 2] = static_cast<uint8_t>(s1 & 3u);
        const uint32_t s2 = (j1 << 14) | (s1 >> 2);
        if (t == 2) {
            s = s2;
            break;
        }
        const uint32_t j2 =
            __builtin_amdgcn_readlane(jb, 5 + 4 * static_cast<int>(j0) + static_cast<int>(j1));
        if (lane == 0) chunk[t - 3] = static_cast<uint8_t>(s2 & 3u);
        s = (j2 << 14) | (s2 >> 2);
        t -= 3;
    }
    if (lane == 0) start_state[blk] = swap_halves ? nibble_halves_swap(s) : s;
    __syncthreads();
    for (int wi = lane; wi < nwords; wi += 64) {
        uint32_t word = 0;
        for (int q = 0; q < 16; ++q) {
            const int ci = wi * 16 + q;
            if (ci < n) word |= static_cast<uint32_t>(chunk[ci]) << (30 - 2 * q);
        }
        bitstream[blk * nwords + wi] = swap_halves ? nibble_halves_swap(word) : word;
    }
}

constexpr size_t kLdsBytes = kLdsDwords * sizeof(float);

// Codebook-stream ceiling of the forward kernel: the same codebook loads (descriptor,
// offsets, order, ring of kRing<false> loads in flight, one 8-wave workgroup per block) with
// the arithmetic, LDS traffic and backpointer stores taken out.  Each lane folds what it
// loads into one word (one xor per loaded dword, so every load stays live) and stores it
// at the end.  Its rate of codebook bytes is what the L2 delivers to the compute units
// for this access pattern: 4 bytes per state update of the forward kernel.
template <int K>
__device__ __forceinline__ void probe_position(float4 (&ring)[kRing<false>],
                                               __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                               uint32_t &x) {
    constexpr int D = kRing<false>;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const float4 c = ring[K % D];
    ring[K % D] = cb_load_pos<K + D>(rs, voff);
    x ^= __float_as_uint(c.x) ^ __float_as_uint(c.y) ^ __float_as_uint(c.z) ^
         __float_as_uint(c.w);
    asm volatile("" : "+v"(x));  // consumed here, not in a tree at the end
}

template <int... I>
__device__ __forceinline__ void probe_positions(float4 (&ring)[kRing<false>],
                                                __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                uint32_t &x, std::integer_sequence<int, I...>) {
    (probe_position<I>(ring, rs, voff, x), ...);
}

__global__ __launch_bounds__(kThreads, 1) void l16_stream_probe_kernel(const float4 *cb,
                                                                       int super_steps,
                                                                       uint32_t *out) {
    const uint32_t tid = threadIdx.x;
    const uint32_t wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float4 *>(cb + wu * (kCopy / kWaves)), 0,
        3 * kCopy * static_cast<int>(sizeof(float4)), 0x00020000);
    const uint32_t voff = (tid & 63) * static_cast<uint32_t>(sizeof(float4));
    float4 ring[kRing<false>];
    ring_fill<0>(ring, rs, voff);
    uint32_t x = 0;
    for (int q = 0; q < super_steps; ++q)
        probe_positions(ring, rs, voff, x, std::make_integer_sequence<int, kPositions>{});
    out[static_cast<int64_t>(blockIdx.x) * kThreads + tid] = x;
}

}  // namespace

bool l16_supported(const Problem &p) { return p.L == 16 && p.kv == 2 && p.V == 1; }

size_t l16_fixed_bytes(const Problem &) { return 3 * sizeof(float4) * kCopy; }

size_t l16_bp_bytes(const Problem &p) {
    return static_cast<size_t>(p.n) * kThreads * sizeof(uint2);
}

hipError_t launch_l16_prepare(const Problem &, const float *C, char *ws, hipStream_t s) {
    const int total = 3 * kCopy;
    hipLaunchKernelGGL(l16_prepare_kernel, dim3((total + 255) / 256), dim3(256), 0, s, C,
                       reinterpret_cast<float4 *>(ws));
    return hipGetLastError();
}

hipError_t launch_acs_l16(const Problem &p, const Plan &pl, const float *W, const float *d,
                          int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s) {
    char *per = ws + pl.fixed;
    uint2 *bp = reinterpret_cast<uint2 *>(per);
    uint32_t *send = reinterpret_cast<uint32_t *>(per + nb * pl.bp_bytes);
    const float4 *cb = reinterpret_cast<const float4 *>(ws);
    const int64_t bp_per_block = static_cast<int64_t>(pl.bp_bytes / sizeof(uint2));
    using Kern = void (*)(const float *, int64_t, const float *, const float4 *, int, int64_t,
                          int64_t, uint2 *, int64_t, uint32_t *, float *);
    static constexpr Kern kKernels[2][3] = {
        {acs_l16_kernel<false, 0>, acs_l16_kernel<false, 1>, acs_l16_kernel<false, 2>},
        {acs_l16_kernel<true, 0>, acs_l16_kernel<true, 1>, acs_l16_kernel<true, 2>}};
    const Kern kern = kKernels[d ? 1 : 0][p.n % 3];
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kLdsBytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), kLdsBytes, s, W,
                       p.ldw, d, cb, p.n, p.blocks_per_row, block0, bp, bp_per_block, send,
                       cost);
    return hipGetLastError();
}

size_t l16_stream_probe_bytes(int64_t blocks) {
    return 3 * sizeof(float4) * kCopy + static_cast<size_t>(blocks) * kThreads * 4;
}

hipError_t launch_l16_stream_probe(int64_t blocks, int super_steps, char *ws, hipStream_t s) {
    const float4 *cb = reinterpret_cast<const float4 *>(ws);
    uint32_t *out = reinterpret_cast<uint32_t *>(ws + 3 * sizeof(float4) * kCopy);
    // the forward kernel's LDS allocation (unused here), so that one workgroup of 8 waves
    // runs per compute unit, as in the forward kernel
    const void *kern = reinterpret_cast<const void *>(l16_stream_probe_kernel);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kLdsBytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(l16_stream_probe_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), kLdsBytes, s, cb, super_steps, out);
    return hipGetLastError();
}

hipError_t launch_traceback_l16(const Problem &p, const Plan &pl, int64_t block0, int64_t nb,
                                const char *ws, uint32_t *bitstream, uint32_t *start_state,
                                hipStream_t s, bool swap_halves) {
    const char *per = ws + pl.fixed;
    const uint2 *bp = reinterpret_cast<const uint2 *>(per);
    const uint32_t *send = reinterpret_cast<const uint32_t *>(per + nb * pl.bp_bytes);
    const int nwords = (p.k * p.T + 31) / 32;
    hipLaunchKernelGGL(traceback_l16_kernel, dim3(static_cast<unsigned>(nb)), dim3(64), 0, s, bp,
                       static_cast<int64_t>(pl.bp_bytes / sizeof(uint2)), send, p.n, nwords,
                       block0, bitstream, start_state, swap_halves ? 1 : 0);
    return hipGetLastError();
}

}  // namespace tcq
