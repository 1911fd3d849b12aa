// L = 16, k*V = 3, V = 1 forward kernel (the 3-bit code).  Same organisation as the
// k*V = 2 kernel (kernels_l16.hip): the block's 2^16 costs in VGPRs, a super-step of
// in-lane add-compare-select (here two steps of three bits, 8 predecessors per group),
// then the same LDS transposition.  Layout, group structure and segment order:
// l16_layout.h (the "k*V = 3" part); shared device pieces: l16_device.h.
//
// The step (Pingala-8 post, Viterbi paragraph; bitshift structure from the QTIP
// abstract; weighted metric from the CurveTQ abstract): predecessors of group x are
// (j << 13) | x, j = 0..7; keep the smallest cost, lowest j on ties; successor
// (x << 3) | b gets fmaf(fl(d * e), e, m), e = fl(w - C[s']).
#include <hip/hip_runtime.h>

#include <utility>

#include "l16_device.h"
#include "l16_layout.h"
#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

using namespace l16;

constexpr int kGroups3 = 16;  // groups per lane and step
constexpr int kPrefetch3 = 8;    // float4 codebook loads in flight (4 groups)
constexpr int kPositions3 = 64;  // float4 loads per super-step (2 steps x 16 groups x 2)
// the ring runs across super-steps: position k lives in slot k mod kPrefetch3 in every
// super-step only if the ring size divides the positions per super-step
static_assert(kPositions3 % kPrefetch3 == 0, "ring size must divide a super-step");

// Codebook copies for k*V = 3: for step p (1, 2), per (wave, group, half, lane) one
// float4 holding successors 4h .. 4h+3 of the group: 2 copies of 16384 float4.
__global__ __launch_bounds__(256) void l16k3_prepare_kernel(const float *__restrict__ C,
                                                            float4 *__restrict__ out) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 2 * kCopy) return;
    const int p = idx / kCopy + 1;
    const int rem = idx % kCopy;
    const uint32_t w = rem / (kGroups3 * 2 * kLanes);
    const uint32_t g = (rem / (2 * kLanes)) % kGroups3;
    const uint32_t h = (rem / kLanes) % 2;
    const uint32_t l = rem % kLanes;
    const uint32_t s = state_of3(p, w, l, group_reg3(p, g, 0)) + 4u * h;
    const float *src = C + s;
    out[idx] = make_float4(src[0], src[1], src[2], src[3]);
}

// load for position k of a super-step: segment k / 16, group (k % 16) / 2, half k % 2
template <int K>
__device__ __forceinline__ float4 cb3_load_pos(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    constexpr int k = K % kPositions3;
    constexpr int seg = k / 16;
    constexpr int P = seg3_step(seg);
    constexpr int e = static_cast<int>(seg3_group(seg, (k % 16) / 2)) * 2 + (k % 2);
    constexpr int kEntry = static_cast<int>(sizeof(float4));
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        rs, voff + (e & 3) * kLanes * kEntry, ((P - 1) * kCopy + (e & ~3) * kLanes) * kEntry, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}

template <int K0, int... I>
__device__ __forceinline__ void ring3_prime(float4 (&ring)[kPrefetch3], __amdgpu_buffer_rsrc_t rs,
                                            uint32_t voff, std::integer_sequence<int, I...>) {
    ((ring[(K0 + I) % kPrefetch3] = cb3_load_pos<K0 + I>(rs, voff)), ...);
}

template <int K0>
__device__ __forceinline__ void ring3_fill(float4 (&ring)[kPrefetch3], __amdgpu_buffer_rsrc_t rs,
                                           uint32_t voff) {
    ring3_prime<K0>(ring, rs, voff, std::make_integer_sequence<int, kPrefetch3>{});
}

__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// One group (I-th of segment SEG) under naming NM: 8-way minimum with the lowest index
// on ties, three backpointer bits shifted in.  The minimum takes four VALU minimums
// (three of them v_min3); seven equality compares against it give masks e0 .. e6, and
// the index j of the first set mask is assembled on the SALU (13 operations):
//   bit 2 of j = no match among 0..3;  bit 1 = first match in 2..3, or none in 0..5;
//   bit 0 = none of: e0, e2 without e0|e1, e4 without a match in 0..3, e6 without one
//           in 0..5.
// Bit 2 is stored inverted (the mask "a match among 0..3" as it is, one operation fewer)
// and the traceback flips it back.  (A tournament of pairwise minimums and strict
// compares gives the same index with three more VALU operations per group; it ran 2 %
// slower at 4096 x 14336, and storing bit 2 as it is 1 % slower.)
template <int SEG, bool WEIGHTED, int NM, int I>
__device__ __forceinline__ void acs3_group(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                           __amdgpu_buffer_rsrc_t rs, uint32_t voff, float wt,
                                           float dt, uint32_t &acc) {
    constexpr int P = seg3_step(SEG);
    constexpr int k = 16 * SEG + 2 * I;
    constexpr uint32_t g = seg3_group(SEG, I);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const float4 ca = ring[k % kPrefetch3];
    const float4 cbv = ring[(k + 1) % kPrefetch3];
    ring[k % kPrefetch3] = cb3_load_pos<k + kPrefetch3>(rs, voff);
    ring[(k + 1) % kPrefetch3] = cb3_load_pos<k + 1 + kPrefetch3>(rs, voff);
    constexpr int r0 = phys(NM, group_reg3(P, g, 0)), r1 = phys(NM, group_reg3(P, g, 1));
    constexpr int r2 = phys(NM, group_reg3(P, g, 2)), r3 = phys(NM, group_reg3(P, g, 3));
    constexpr int r4 = phys(NM, group_reg3(P, g, 4)), r5 = phys(NM, group_reg3(P, g, 5));
    constexpr int r6 = phys(NM, group_reg3(P, g, 6)), r7 = phys(NM, group_reg3(P, g, 7));
    const uint32_t u0 = J[r0], u1 = J[r1], u2 = J[r2], u3 = J[r3];
    const uint32_t u4 = J[r4], u5 = J[r5], u6 = J[r6], u7 = J[r7];
    const uint32_t mu = umin(umin(umin(umin(u0, u1), u2), umin(umin(u3, u4), u5)),
                             umin(u6, u7));
    const uint64_t e0 = __ballot(u0 == mu), e1 = __ballot(u1 == mu);
    const uint64_t e2 = __ballot(u2 == mu), e3 = __ballot(u3 == mu);
    const uint64_t e4 = __ballot(u4 == mu), e5 = __ballot(u5 == mu);
    const uint64_t e6 = __ballot(u6 == mu);
    const uint64_t t01 = e0 | e1, t23 = e2 | e3, t45 = e4 | e5;
    const uint64_t a03 = t01 | t23;  // a match among 0..3: index bit 2 clear
    const uint64_t y = ~(a03 | t45);
    const uint64_t b1 = (t23 & ~t01) | y;
    const uint64_t b0 = ~((e0 | (e2 & ~t01)) | ((e4 & ~a03) | (e6 & y)));
    acc = shift_in(shift_in(shift_in(acc, a03), b1), b0);
    const float m = __uint_as_float(mu);
    const float e[8] = {wt - ca.x, wt - ca.y, wt - ca.z, wt - ca.w,
                        wt - cbv.x, wt - cbv.y, wt - cbv.z, wt - cbv.w};
    J[r0] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[0] : e[0], e[0], m));
    J[r1] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[1] : e[1], e[1], m));
    J[r2] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[2] : e[2], e[2], m));
    J[r3] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[3] : e[3], e[3], m));
    J[r4] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[4] : e[4], e[4], m));
    J[r5] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[5] : e[5], e[5], m));
    J[r6] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[6] : e[6], e[6], m));
    J[r7] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e[7] : e[7], e[7], m));
    // order within the group: the minimums and compares, then the scalar assembly of the
    // three index bits interleaved one for one with the independent vector work (with two
    // waves per SIMD the compare -> SALU -> carry-in chain is otherwise exposed)
    __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
}

template <int SEG, bool WEIGHTED, int NM, int... I>
__device__ __forceinline__ void acs3_segment_impl(uint32_t (&J)[kRegs],
                                                  float4 (&ring)[kPrefetch3],
                                                  __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                  float wt, float dt, uint32_t *bp_word,
                                                  std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    (acs3_group<SEG, WEIGHTED, NM, I>(J, ring, rs, voff, wt, dt, acc), ...);
    *bp_word = acc;
}

// acs3_segment with LDS work X issued after each group (l16_device.h).
template <int SEG, bool WEIGHTED, int NM, class X, int... I>
__device__ __forceinline__ void acs3_segment_x_impl(uint32_t (&J)[kRegs],
                                                    float4 (&ring)[kPrefetch3], const Ctx &cx,
                                                    float wt, float dt, uint32_t *bp_word,
                                                    const X &x, std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    ((acs3_group<SEG, WEIGHTED, NM, I>(J, ring, cx.rs, cx.voff, wt, dt, acc),
      x.template step<I>(J, cx)),
     ...);
    *bp_word = acc;
}
template <int SEG, bool WEIGHTED, int NM, class X>
__device__ __forceinline__ void acs3_segment_x(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                               const Ctx &cx, int t0, const StepIn &in,
                                               const X &x) {
    constexpr int P = seg3_step(SEG);
    const int t = t0 + P - 1;
    acs3_segment_x_impl<SEG, WEIGHTED, NM>(J, ring, cx, in.w[P - 1], in.d[P - 1],
                                           cx.bp + 2 * kThreads * t + seg3_half(SEG), x,
                                           std::make_integer_sequence<int, 8>{});
}

template <int SEG, bool WEIGHTED, int NM>
__device__ __forceinline__ void acs3_segment(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                             const Ctx &cx, int t0, const StepIn &in) {
    constexpr int P = seg3_step(SEG);
    const int t = t0 + P - 1;
    acs3_segment_impl<SEG, WEIGHTED, NM>(J, ring, cx.rs, cx.voff, in.w[P - 1], in.d[P - 1],
                                         cx.bp + 2 * kThreads * t + seg3_half(SEG),
                                         std::make_integer_sequence<int, 8>{});
}

// The eight registers of step-1 group g = 2 I + RHO (the registers segment RHO of a
// super-step consumes together), read from transposition round RHO.
template <int NM, int RHO, int I>
__device__ __forceinline__ void round_read_group3(uint32_t (&J)[kRegs], const Ctx &cx) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        constexpr uint32_t g = 2u * I + RHO;
        const uint32_t r = group_reg3(1, g, b);
        const uint32_t off = 4u * lds_read_reg(r);
        const uint32_t k = off / (4u * 2112u * 4u);
        J[phys(1 - NM, r)] = lds_get(cx.rb[k], off - k * 4u * 2112u * 4u);
    }
}

// Segment 1 (step 1 of the odd groups) with round 1 of the transposition read into the
// registers it consumes: the eight values of group i + 1 are requested before group i
// is computed, so at most 16 reads are in flight (the LDS wait counter counts at most
// 15) and each group waits only for its own values.
template <bool WEIGHTED, int NM, int I>
__device__ __forceinline__ void seg1_group3(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                            const Ctx &cx, float wt, float dt, uint32_t &acc) {
    if constexpr (I + 1 < 8) round_read_group3<1 - NM, 1, I + 1>(J, cx);
    acs3_group<1, WEIGHTED, NM, I>(J, ring, cx.rs, cx.voff, wt, dt, acc);
}
template <bool WEIGHTED, int NM, int... I>
__device__ __forceinline__ void seg1_reading3(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                              const Ctx &cx, int t0, const StepIn &in,
                                              std::integer_sequence<int, I...>) {
    round_read_group3<1 - NM, 1, 0>(J, cx);
    uint32_t acc = 0;
    (seg1_group3<WEIGHTED, NM, I>(J, ring, cx, in.w[0], in.d[0], acc), ...);
    cx.bp[2 * kThreads * t0 + seg3_half(1)] = acc;
}

// Super-step (steps t0+1, t0+2) under naming NM, with the weights (and d) of its two
// steps in `in`; those of the next super-step are requested into `next` and complete at
// a barrier (a wait for a scalar load would also wait for every LDS operation in flight).
// The transposition rounds are spread over the segments as in kernels_l16.hip: segment 0
// (even step-1 groups) writes round 1 of the previous transposition, which is still in
// the odd groups' registers; segment 1 reads it back; segment 2 (step 2, the r[6] = 0
// half) writes round 0 as its groups finish and segment 3 (the r[6] = 1 half) reads it
// back.  Round 1 is left in registers for the next super-step (or the tail).
template <bool WEIGHTED, int NM>
__device__ __forceinline__ void super_step3(uint32_t (&J)[kRegs], float4 (&ring)[kPrefetch3],
                                            const Ctx &cx, int t0, const StepIn &in,
                                            StepIn &next) {
    acs3_segment_x<0, WEIGHTED, NM>(J, ring, cx, t0, in, WriteLds<1 - NM, 1, 8, 0>{});
    __syncthreads();  // round-1 values written by every wave
    seg1_reading3<WEIGHTED, NM>(J, ring, cx, t0, in, std::make_integer_sequence<int, 8>{});
    __syncthreads();  // every wave has read round 1
    acs3_segment_x<2, WEIGHTED, NM>(J, ring, cx, t0, in, WriteRound0Lagged<NM, 8>{});
    round_write_range<NM, 0, 56, 8>(J, cx);
    next = load_steps<WEIGHTED>(cx, t0 + 2);
    __syncthreads();  // round-0 values written by every wave
    acs3_segment_x<3, WEIGHTED, NM>(J, ring, cx, t0, in, ReadLds<NM, 0, 2>{});
    __syncthreads();  // every wave has read round 0
}

// Register part of the state a register holds after step P of a 3-bit super-step, and the
// lane's lowest (cost, state).
template <int P>
struct lane_argmin3_key {
    static constexpr uint32_t of(int r) {
        return state_of3(P, 0, 0, static_cast<uint32_t>(r));
    }
};
template <int P, int NM>
__device__ __forceinline__ void lane_argmin3(const uint32_t (&J)[kRegs], uint32_t w,
                                             uint32_t l, uint32_t &bv, uint32_t &bi) {
    lane_best<lane_argmin3_key<P>, NM>(J, state_of3(P, w, l, 0), bv, bi);
}

// R = n mod 2 (one step after the last whole super-step, or none): a template argument,
// so that each instantiation has one tail and no merged register assignment.
template <bool WEIGHTED, int R>
__global__ __launch_bounds__(kThreads, 1) void acs_l16k3_kernel(
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
    const Ctx cx = make_ctx(W, ldw, WEIGHTED ? d : nullptr, cb, n, row, col, w, l,
                            bp + blockIdx.x * bp_per_block);

    uint32_t J[kRegs];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) J[r] = 0u;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) asm volatile("" : "+v"(J[r]));
    float4 ring[kPrefetch3];
    ring3_fill<0>(ring, cx.rs, cx.voff);
    // the all-zero start is round 1 of a transposition that the first super-step (or the
    // tail) writes out as it goes

    const int Q = n / 2;  // n % 2 == R: the launcher picks the instantiation
    StepIn in = load_steps<WEIGHTED>(cx, 0);
    if (Q & 1) {
        StepIn next;
        super_step3<WEIGHTED, 1>(J, ring, cx, 0, in, next);
        in = next;
    }
    for (int q = Q & 1; q < Q; q += 2) {
        StepIn mid, next;
        super_step3<WEIGHTED, 0>(J, ring, cx, 2 * q, in, mid);
        super_step3<WEIGHTED, 1>(J, ring, cx, 2 * q + 2, mid, next);
        in = next;
    }
    if constexpr (R == 1) {  // one more step: segments 0 and 1 under naming 0
        acs3_segment_x<0, WEIGHTED, 0>(J, ring, cx, 2 * Q, in, WriteLds<1, 1, 8, 0>{});
        __syncthreads();
        round_read<1, 1>(J, cx);
        acs3_segment<1, WEIGHTED, 0>(J, ring, cx, 2 * Q, in);
    } else {
        round_write<1, 1>(J, cx);
        __syncthreads();
        round_read<1, 1>(J, cx);
    }

    uint32_t bv = 0xFFFFFFFFu;
    uint32_t bi = 0xFFFFFFFFu;
    lane_argmin3<R, 0>(J, w, l, bv, bi);
    block_select(bv, bi, w, l, send + blockIdx.x, cost_out + blk);
}

// One wave per block: follow the remembered predecessors back and pack the 3-bit chunks
// b_1..b_n (MSB first) into MSB-first words.
__global__ __launch_bounds__(64) void traceback_l16k3_kernel(
    const uint2 *__restrict__ bp, int64_t bp_per_block, const uint32_t *__restrict__ send,
    int n, int nwords, int64_t block0, uint32_t *__restrict__ bitstream,
    uint32_t *__restrict__ start_state) {
    __shared__ uint8_t chunk[TCQ_MAX_STEPS];
    const int lane = threadIdx.x;
    const uint2 *bpb = bp + blockIdx.x * bp_per_block;
    const int64_t blk = block0 + blockIdx.x;
    // Two steps per memory round trip: with s_t known, lane 0 reads the choice at step t
    // for s_t and lanes 1..8 the choice at step t-1 for each of the eight possible
    // s_{t-1} = (j << 13) | (s_t >> 3); the wave then picks the path they determine.
    uint32_t s = send[blockIdx.x];  // s_t, the same in every lane
    int t = n;
    while (t >= 1) {
        int lvl = -1;
        uint32_t c = 0;
        if (lane == 0) {
            lvl = 0;
            c = s;
        } else if (lane < 9) {
            lvl = 1;
            c = (static_cast<uint32_t>(lane - 1) << 13) | (s >> 3);
        }
        uint32_t jb = 0;
        if (lvl >= 0 && t - lvl >= 1) {
            const int tt = t - lvl;
            const int p = (tt - 1) % 2 + 1;
            const Slot sl = slot_of3(p, c);
            const uint32_t g = reg_group3(p, sl.r);
            const uint2 word = bpb[(tt - 1) * kThreads + sl.w * kLanes + sl.l];
            const uint32_t bits = bp3_half(p, g) ? word.y : word.x;
            jb = ((bits >> bp3_shift(p, g)) & 7u) ^ 4u;  // bit 2 is stored inverted
        }
        const uint32_t j0 = __builtin_amdgcn_readlane(jb, 0);
        if (lane == 0) chunk[t - 1] = static_cast<uint8_t>(s & 7u);
        const uint32_t s1 = (j0 << 13) | (s >> 3);
        if (t == 1) {
            s = s1;
            break;
        }
        const uint32_t j1 = __builtin_amdgcn_readlane(jb, 1 + static_cast<int>(j0));
        if (lane == 0) chunk[t - 2] = static_cast<uint8_t>(s1 & 7u);
        s = (j1 << 13) | (s1 >> 3);
        t -= 2;
    }
    if (lane == 0) start_state[blk] = s;
    __syncthreads();
    const int total = 3 * n;
    for (int wi = lane; wi < nwords; wi += 64) {
        uint32_t word = 0;
        for (int q = 0; q < 32; ++q) {
            const int pos = wi * 32 + q;
            if (pos < total) {
                const int ci = pos / 3;
                const int within = 2 - pos % 3;
                word |= ((static_cast<uint32_t>(chunk[ci]) >> within) & 1u) << (31 - q);
            }
        }
        bitstream[blk * nwords + wi] = word;
    }
}

constexpr size_t kLdsBytes = kLdsDwords * sizeof(float);

}  // namespace

bool l16k3_supported(const Problem &p) { return p.L == 16 && p.kv == 3 && p.V == 1; }

size_t l16k3_fixed_bytes(const Problem &) { return 2 * sizeof(float4) * kCopy; }

size_t l16k3_bp_bytes(const Problem &p) {
    return static_cast<size_t>(p.n) * kThreads * sizeof(uint2);
}

hipError_t launch_l16k3_prepare(const Problem &, const float *C, char *ws, hipStream_t s) {
    const int total = 2 * kCopy;
    hipLaunchKernelGGL(l16k3_prepare_kernel, dim3((total + 255) / 256), dim3(256), 0, s, C,
                       reinterpret_cast<float4 *>(ws));
    return hipGetLastError();
}

hipError_t launch_acs_l16k3(const Problem &p, const Plan &pl, const float *W, const float *d,
                            int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s) {
    char *per = ws + pl.fixed;
    uint2 *bp = reinterpret_cast<uint2 *>(per);
    uint32_t *send = reinterpret_cast<uint32_t *>(per + nb * pl.bp_bytes);
    const float4 *cb = reinterpret_cast<const float4 *>(ws);
    const int64_t bp_per_block = static_cast<int64_t>(pl.bp_bytes / sizeof(uint2));
    using Kern = void (*)(const float *, int64_t, const float *, const float4 *, int, int64_t,
                          int64_t, uint2 *, int64_t, uint32_t *, float *);
    static constexpr Kern kKernels[2][2] = {{acs_l16k3_kernel<false, 0>, acs_l16k3_kernel<false, 1>},
                                            {acs_l16k3_kernel<true, 0>, acs_l16k3_kernel<true, 1>}};
    const Kern kern = kKernels[d ? 1 : 0][p.n % 2];
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kLdsBytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), kLdsBytes, s, W,
                       p.ldw, d, cb, p.n, p.blocks_per_row, block0, bp, bp_per_block, send,
                       cost);
    return hipGetLastError();
}

hipError_t launch_traceback_l16k3(const Problem &p, const Plan &pl, int64_t block0, int64_t nb,
                                  const char *ws, uint32_t *bitstream, uint32_t *start_state,
                                  hipStream_t s) {
    const char *per = ws + pl.fixed;
    const uint2 *bp = reinterpret_cast<const uint2 *>(per);
    const uint32_t *send = reinterpret_cast<const uint32_t *>(per + nb * pl.bp_bytes);
    const int nwords = (p.k * p.T + 31) / 32;
    hipLaunchKernelGGL(traceback_l16k3_kernel, dim3(static_cast<unsigned>(nb)), dim3(64), 0, s,
                       bp, static_cast<int64_t>(pl.bp_bytes / sizeof(uint2)), send, p.n, nwords,
                       block0, bitstream, start_state);
    return hipGetLastError();
}

}  // namespace tcq
