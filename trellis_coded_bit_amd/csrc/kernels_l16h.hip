// L = 16, k*V = 4 forward kernel (k = 2, V = 2: the 8B-MLP shape; also k = 4, V = 1).
//
// A step that shifts in four bits is two "half-steps" of two bits.  The predecessors of
// s = (x << 4) | b are (j << 12) | x, j = 0..15; write j = 4 j_hi + j_lo.  The kernel runs
// the trellis on a relabelled state: each 4-bit chunk of the state is stored with its two
// 2-bit halves exchanged, P(s) (P swaps bits [3:2] and [1:0] of every nibble; P = P^-1).
// A 4-bit shift of s is a 4-bit shift of P(s), so every path and cost is unchanged; but
// the first half-step of a step now drops the oldest 2-bit digit of P(s), which is j_lo,
// and the second drops j_hi.  The first half-step (no cost added) keeps, for every j_hi,
// the lowest j_lo of minimum cost; the second (which adds the branch metric of the whole
// step on the true state, C[P(.)]) keeps the lowest j_hi of minimum cost.  Together they
// keep the smallest j = 4 j_hi + j_lo of minimum cost: the 16-way lowest-index rule.  The
// minima are exact, so every cost is the one the 16-way search gives.  The half-step
// chunks come out as (low half, high half) of each true chunk, so the traceback swaps the
// halves of every nibble of the packed stream and of the start state; the end state is
// chosen by the lowest true index.  The start state comes out below 2^12 because all
// costs start equal.
//
// So the kernel is the k*V = 2 kernel (kernels_l16.hip, layout in l16_layout.h) run over
// 2n half-steps, with the metric only on even half-steps: half-step h = 3q + P of
// super-step q carries a metric when q + P is even (P = 2 for even q, P = 1 and 3 for
// odd q).  Metric: for v = 0..V-1 in order, e = fl(w - C[s][v]); acc = fmaf(fl(d e), e,
// acc), starting from the kept predecessor cost (the encoder's chain).
#include <hip/hip_runtime.h>

#include <utility>

#include "l16_device.h"
#include "l16_layout.h"
#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

using namespace l16;

// The shared per-block context plus backpointer stores through a buffer descriptor.
struct CtxH : Ctx {
    BpBuf bpb;
};

// Codebook copies: for step P (1..3) and coordinate v, per (wave, group, lane) one float4
// with coordinate v of the group's four successors: 3 V copies of kCopy float4.
template <int V>
__global__ __launch_bounds__(256) void l16h_prepare_kernel(const float *__restrict__ C,
                                                           float4 *__restrict__ out) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 3 * V * kCopy) return;
    const int pv = idx / kCopy;
    const int p = pv / V + 1;
    const int v = pv % V;
    const int rem = idx % kCopy;
    const uint32_t w = rem / (kGroupsPerLane * kLanes);
    const uint32_t g = (rem / kLanes) % kGroupsPerLane;
    const uint32_t l = rem % kLanes;
    // successors s .. s + 3 of the relabelled trellis: true states P(s + b)
    const uint32_t s = state_of(p, w, l, group_reg(p, g, 0));
    out[idx] = make_float4(C[static_cast<size_t>(nibble_halves_swap(s)) * V + v],
                           C[static_cast<size_t>(nibble_halves_swap(s + 1)) * V + v],
                           C[static_cast<size_t>(nibble_halves_swap(s + 2)) * V + v],
                           C[static_cast<size_t>(nibble_halves_swap(s + 3)) * V + v]);
}

// Codebook loads in flight: 4 groups.  Measured on MI355X at 14336 x 4096, V = 2: 663 ms
// against 671 ms with 8 groups (whose 64 registers of ring push the kernel into scratch)
// and 669 ms with 2.  The ring size divides the 32 V and 64 V positions of a super-step.
template <int V>
struct Ring {
    static constexpr int kSize = 4 * V;
};

// Codebook load for metric position K of a super-step with pattern MP (positions run
// over the metric groups in processing order, V loads per group; positions past the
// end of the super-step belong to the next one, whose pattern is 1 - MP).
template <int V, int MP, int K>
__device__ __forceinline__ float4 cbh_load_pos(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    constexpr int cnt = metric_groups(MP) * V;
    constexpr int mp = K < cnt ? MP : 1 - MP;
    constexpr int k = K < cnt ? K : K - cnt;
    constexpr int mg = k / V;
    constexpr int v = k % V;
    constexpr int seg = metric_seg(mp, mg / 16);
    constexpr int P = seg_step(seg);
    constexpr int g = static_cast<int>(seg_group(seg, mg % 16));
    constexpr int kEntry = static_cast<int>(sizeof(float4));
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(
        rs, voff + (g & 3) * kLanes * kEntry,
        (((P - 1) * V + v) * kCopy + (g & ~3) * kLanes) * kEntry, 0);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                       __uint_as_float(x[3]));
}

template <int V, int MP, int K0, int... I>
__device__ __forceinline__ void ringh_prime(float4 (&ring)[Ring<V>::kSize],
                                            __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                            std::integer_sequence<int, I...>) {
    ((ring[(K0 + I) % Ring<V>::kSize] = cbh_load_pos<V, MP, K0 + I>(rs, voff)), ...);
}

// One group (I-th of segment SEG) of a half-step without metric: the four successors all
// take the kept predecessor cost.  No scheduling barrier between these groups (they load
// no codebook values), so the compare -> SALU -> carry-in chain of one group overlaps the
// minimums of the next.
template <int SEG, int NM, int I>
__device__ __forceinline__ void acsh_group_plain(uint32_t (&J)[kRegs], uint32_t &acc) {
    constexpr int P = seg_step(SEG);
    constexpr uint32_t g = seg_group(SEG, I);
    constexpr int r0 = phys(NM, group_reg(P, g, 0)), r1 = phys(NM, group_reg(P, g, 1));
    constexpr int r2 = phys(NM, group_reg(P, g, 2)), r3 = phys(NM, group_reg(P, g, 3));
    const uint32_t u0 = J[r0], u1 = J[r1], u2 = J[r2], u3 = J[r3];
    uint64_t chi, b0;
    const uint32_t mu = argmin4(u0, u1, u2, u3, chi, b0);
    acc = shift_in(shift_in(acc, chi), b0);
    J[r0] = mu;
    J[r1] = mu;
    J[r2] = mu;
    J[r3] = mu;
}

// One group of a half-step with metric (V coordinates per successor).
template <int SEG, bool WEIGHTED, int NM, int V, int MP, int I>
__device__ __forceinline__ void acsh_group_metric(uint32_t (&J)[kRegs],
                                                  float4 (&ring)[Ring<V>::kSize],
                                                  __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                  const float (&wt)[2], const float (&dt)[2],
                                                  uint32_t &acc) {
    constexpr int RS = Ring<V>::kSize;
    constexpr int P = seg_step(SEG);
    constexpr int k = (16 * metric_index(MP, SEG) + I) * V;  // first position of the group
    constexpr uint32_t g = seg_group(SEG, I);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    float4 c[V];
#pragma unroll
    for (int v = 0; v < V; ++v) c[v] = ring[(k + v) % RS];
    if constexpr (V == 1) {
        ring[k % RS] = cbh_load_pos<V, MP, k + RS>(rs, voff);
    } else {
        ring[k % RS] = cbh_load_pos<V, MP, k + RS>(rs, voff);
        ring[(k + 1) % RS] = cbh_load_pos<V, MP, k + 1 + RS>(rs, voff);
    }
    constexpr int r0 = phys(NM, group_reg(P, g, 0)), r1 = phys(NM, group_reg(P, g, 1));
    constexpr int r2 = phys(NM, group_reg(P, g, 2)), r3 = phys(NM, group_reg(P, g, 3));
    const uint32_t u0 = J[r0], u1 = J[r1], u2 = J[r2], u3 = J[r3];
    uint64_t chi, b0;
    const uint32_t mu = argmin4(u0, u1, u2, u3, chi, b0);
    acc = shift_in(shift_in(acc, chi), b0);
    float a0 = __uint_as_float(mu), a1 = a0, a2 = a0, a3 = a0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const float e0 = wt[v] - c[v].x, e1 = wt[v] - c[v].y;
        const float e2 = wt[v] - c[v].z, e3 = wt[v] - c[v].w;
        a0 = __builtin_fmaf(WEIGHTED ? dt[v] * e0 : e0, e0, a0);
        a1 = __builtin_fmaf(WEIGHTED ? dt[v] * e1 : e1, e1, a1);
        a2 = __builtin_fmaf(WEIGHTED ? dt[v] * e2 : e2, e2, a2);
        a3 = __builtin_fmaf(WEIGHTED ? dt[v] * e3 : e3, e3, a3);
    }
    J[r0] = __float_as_uint(a0);
    J[r1] = __float_as_uint(a1);
    J[r2] = __float_as_uint(a2);
    J[r3] = __float_as_uint(a3);
}

template <int SEG, bool WEIGHTED, int NM, int V, int MP, int... I>
__device__ __forceinline__ void acsh_segment_impl(uint32_t (&J)[kRegs],
                                                  float4 (&ring)[Ring<V>::kSize],
                                                  const CtxH &cx, const float (&wt)[2],
                                                  const float (&dt)[2], int bp_word,
                                                  std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    if constexpr (seg_has_metric(MP, SEG)) {
        (acsh_group_metric<SEG, WEIGHTED, NM, V, MP, I>(J, ring, cx.rs, cx.voff, wt, dt, acc),
         ...);
    } else {
        (acsh_group_plain<SEG, NM, I>(J, acc), ...);
    }
    cx.bpb.store(bp_word, acc);
}

// Weights and d of the full steps under the three half-steps of a super-step (index
// P - 1; only the metric half-steps use them), held in scalar registers.  Requested one
// super-step ahead so that they complete at a workgroup barrier: a wait for a scalar
// load is also a wait for every LDS operation in flight.
struct StepInH {
    float w[3][2], d[3][2];
};
// Half-steps h0 .. h0 + 2; the full step of half-step h is h >> 1, clamped to the block.
template <bool WEIGHTED, int V>
__device__ __forceinline__ StepInH load_h(const CtxH &cx, int h0) {
    StepInH s;
    const int last = cx.nw / V - 1;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int t = (h0 + p) >> 1 < last ? (h0 + p) >> 1 : last;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            s.w[p][v] = v < V ? cx.wcol[t * V + v] : 0.0f;
            s.d[p][v] = WEIGHTED && v < V ? cx.dcol[t * V + v] : 1.0f;
        }
    }
    return s;
}

// Segment SEG of super-step q (half-steps 3q + 1 .. 3q + 3), pattern MP = q mod 2.
template <int SEG, bool WEIGHTED, int NM, int V, int MP>
__device__ __forceinline__ void acsh_segment(uint32_t (&J)[kRegs],
                                             float4 (&ring)[Ring<V>::kSize], const CtxH &cx,
                                             int h0, const StepInH &in) {
    constexpr int P = seg_step(SEG);
    const int h = h0 + P - 1;  // 0-based half-step index
    acsh_segment_impl<SEG, WEIGHTED, NM, V, MP>(J, ring, cx, in.w[P - 1], in.d[P - 1],
                                                2 * kThreads * h + seg_half(SEG),
                                                std::make_integer_sequence<int, 16>{});
}

// Group I of segment SEG, with or without the metric as the pattern says.
template <int SEG, bool WEIGHTED, int NM, int V, int MP, int I>
__device__ __forceinline__ void acsh_group(uint32_t (&J)[kRegs], float4 (&ring)[Ring<V>::kSize],
                                           const CtxH &cx, const StepInH &in, uint32_t &acc) {
    constexpr int P = seg_step(SEG);
    if constexpr (seg_has_metric(MP, SEG))
        acsh_group_metric<SEG, WEIGHTED, NM, V, MP, I>(J, ring, cx.rs, cx.voff, in.w[P - 1],
                                                       in.d[P - 1], acc);
    else
        acsh_group_plain<SEG, NM, I>(J, acc);
}

// Segment SEG with LDS work X issued after each group (l16_device.h).
template <int SEG, bool WEIGHTED, int NM, int V, int MP, class X, int... I>
__device__ __forceinline__ void acsh_segment_x_impl(uint32_t (&J)[kRegs],
                                                    float4 (&ring)[Ring<V>::kSize],
                                                    const CtxH &cx, const StepInH &in,
                                                    int bp_word, const X &x,
                                                    std::integer_sequence<int, I...>) {
    uint32_t acc = 0;
    ((acsh_group<SEG, WEIGHTED, NM, V, MP, I>(J, ring, cx, in, acc), x.template step<I>(J, cx)),
     ...);
    cx.bpb.store(bp_word, acc);
}
template <int SEG, bool WEIGHTED, int NM, int V, int MP, class X>
__device__ __forceinline__ void acsh_segment_x(uint32_t (&J)[kRegs],
                                               float4 (&ring)[Ring<V>::kSize], const CtxH &cx,
                                               int h0, const StepInH &in, const X &x) {
    constexpr int P = seg_step(SEG);
    const int h = h0 + P - 1;
    acsh_segment_x_impl<SEG, WEIGHTED, NM, V, MP>(J, ring, cx, in, 2 * kThreads * h + seg_half(SEG),
                                                  x, std::make_integer_sequence<int, 16>{});
}

// Segments SA (half-step 1) and SA + 1 (half-step 2) of one half of the groups (SA = 0:
// even groups, SA = 2: odd), interleaved in the order pair_step / pair_index of
// l16_layout.h (every step-2 group after the step-1 groups it reads).  One of the two
// carries the metric, the other only the minimum: the plain groups' compare -> SALU ->
// carry-in chains overlap the metric groups' arithmetic instead of running back to
// back.  Each segment keeps its own group order, so the codebook ring and the
// backpointer words are as in the segment-by-segment order.  READS: round 1 of the
// transposition is read into the step-1 groups three groups ahead (the odd half), the
// first three before the call.  X issues its LDS work after each of the 32 groups.
template <int SA, bool WEIGHTED, int NM, int V, int MP, bool READS, int I>
__device__ __forceinline__ void pair_step1(uint32_t (&J)[kRegs], float4 (&ring)[Ring<V>::kSize],
                                           const CtxH &cx, const StepInH &in, uint32_t &acc) {
    if constexpr (READS && I + 3 < 16) round_read_group<1 - NM, 1, I + 3>(J, cx);
    acsh_group<SA, WEIGHTED, NM, V, MP, I>(J, ring, cx, in, acc);
}
template <int SA, bool WEIGHTED, int NM, int V, int MP, bool READS, int K, class X>
__device__ __forceinline__ void pair_slot(uint32_t (&J)[kRegs], float4 (&ring)[Ring<V>::kSize],
                                          const CtxH &cx, const StepInH &in, uint32_t &acc1,
                                          uint32_t &acc2, const X &x) {
    constexpr int I = pair_index(K);
    if constexpr (pair_step(K) == 1)
        pair_step1<SA, WEIGHTED, NM, V, MP, READS, I>(J, ring, cx, in, acc1);
    else
        acsh_group<SA + 1, WEIGHTED, NM, V, MP, I>(J, ring, cx, in, acc2);
    x.template step<K>(J, cx);
}
template <int SA, bool WEIGHTED, int NM, int V, int MP, bool READS, class X, int... K>
__device__ __forceinline__ void acsh_pair_impl(uint32_t (&J)[kRegs],
                                               float4 (&ring)[Ring<V>::kSize], const CtxH &cx,
                                               int h0, const StepInH &in, const X &x,
                                               std::integer_sequence<int, K...>) {
    if constexpr (READS) round_read_groups<1 - NM, 1>(J, cx, std::make_integer_sequence<int, 3>{});
    uint32_t acc1 = 0, acc2 = 0;
    (pair_slot<SA, WEIGHTED, NM, V, MP, READS, K>(J, ring, cx, in, acc1, acc2, x), ...);
    cx.bpb.store(2 * kThreads * h0 + seg_half(SA), acc1);
    cx.bpb.store(2 * kThreads * (h0 + 1) + seg_half(SA + 1), acc2);
}
template <int SA, bool WEIGHTED, int NM, int V, int MP, bool READS, class X>
__device__ __forceinline__ void acsh_pair(uint32_t (&J)[kRegs], float4 (&ring)[Ring<V>::kSize],
                                          const CtxH &cx, int h0, const StepInH &in,
                                          const X &x) {
    acsh_pair_impl<SA, WEIGHTED, NM, V, MP, READS>(J, ring, cx, h0, in, x,
                                                   std::make_integer_sequence<int, 32>{});
}
// No LDS work between the groups.
struct NoLds {
    template <int I>
    __device__ __forceinline__ void step(uint32_t (&)[kRegs], const Ctx &) const {}
};

// Super-step under naming NM and pattern MP, with the weights of its half-steps in `in`
// and those of the next super-step requested into `next`; the transposition rounds are
// spread over the segments as in kernels_l16.hip (round 1 of the previous transposition
// written by segments 0 and 1 and read by segment 2, round 0 written behind segment 4
// and read by segment 5, round 1 left in registers for the next super-step or the tail).
template <bool WEIGHTED, int NM, int V, int MP>
__device__ __forceinline__ void super_step_h(uint32_t (&J)[kRegs],
                                             float4 (&ring)[Ring<V>::kSize], const CtxH &cx,
                                             int h0, const StepInH &in, StepInH &next) {
    acsh_pair<0, WEIGHTED, NM, V, MP, false>(J, ring, cx, h0, in, WriteLds<1 - NM, 1, 2, 0>{});
    __syncthreads();  // round-1 values written by every wave
    acsh_pair<2, WEIGHTED, NM, V, MP, true>(J, ring, cx, h0, in, NoLds{});
    __syncthreads();  // every wave has read round 1
    acsh_segment_x<4, WEIGHTED, NM, V, MP>(J, ring, cx, h0, in, WriteRound0Lagged<NM, 4>{});
    round_write_range<NM, 0, 60, 4>(J, cx);
    next = load_h<WEIGHTED, V>(cx, h0 + 3);
    __syncthreads();  // round-0 values written by every wave
    acsh_segment_x<5, WEIGHTED, NM, V, MP>(J, ring, cx, h0, in, ReadLds<NM, 0, 1>{});
    __syncthreads();  // every wave has read round 0
}

// The last R = 1 or 2 half-steps (segments 0..3 in order) under naming 0.  The metric
// positions they use are the first ones of their pattern, in order, so the ring needs
// no refill.
template <bool WEIGHTED, int V, int MP, int R>
__device__ __forceinline__ void tail_h(uint32_t (&J)[kRegs], float4 (&ring)[Ring<V>::kSize],
                                       const CtxH &cx, int h0, const StepInH &in) {
    round_write<1, 1>(J, cx);  // round 1 of the last transposition, in one go
    acsh_segment<0, WEIGHTED, 0, V, MP>(J, ring, cx, h0, in);
    if constexpr (R == 2) acsh_segment<1, WEIGHTED, 0, V, MP>(J, ring, cx, h0, in);
    __syncthreads();
    round_read<1, 1>(J, cx);
    acsh_segment<2, WEIGHTED, 0, V, MP>(J, ring, cx, h0, in);
    if constexpr (R == 2) acsh_segment<3, WEIGHTED, 0, V, MP>(J, ring, cx, h0, in);
}

// Register part of the true state (halves of every nibble swapped back) a register holds
// after half-step P: ties between end states go to the lowest true index.
template <int P>
struct lane_argmin_h_key {
    static constexpr uint32_t of(int r) {
        return nibble_halves_swap(state_of(P, 0, 0, static_cast<uint32_t>(r)));
    }
};
template <int P, int NM>
__device__ __forceinline__ void lane_argmin_h(const uint32_t (&J)[kRegs], uint32_t w,
                                              uint32_t l, uint32_t &bv, uint32_t &bi) {
    lane_best<lane_argmin_h_key<P>, NM>(J, nibble_halves_swap(state_of(P, w, l, 0)), bv, bi);
}

// n = full steps per block; the kernel runs 2n half-steps.
// R = 2n mod 3, the half-steps after the last whole super-step, is a template argument,
// so that each instantiation has one loop and one tail (with the tails chosen at run
// time the compiler merged their register assignments and spilled to scratch at the
// joins).  It also fixes the pattern QP = Q mod 2 of the last whole super-step: 2n = 3Q
// + R is even, so Q and R have the same parity.
template <bool WEIGHTED, int V, int R>
__global__ __launch_bounds__(kThreads, 1) void acs_l16h_kernel(
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
    CtxH cx;
    static_cast<Ctx &>(cx) = make_ctx(W, ldw, WEIGHTED ? d : nullptr, cb, n * V, row, col, w,
                                      l, bp + blockIdx.x * bp_per_block, 3 * V);
    cx.bpb = make_bpbuf(bp + blockIdx.x * bp_per_block, bp_per_block, w, l);

    uint32_t J[kRegs];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) J[r] = 0u;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) asm volatile("" : "+v"(J[r]));
    constexpr int RS = Ring<V>::kSize;
    float4 ring[RS];
    ringh_prime<V, 0, 0>(ring, cx.rs, cx.voff, std::make_integer_sequence<int, RS>{});
    // the all-zero start is round 1 of a transposition that the first super-step (or the
    // tail) writes out as it goes

    const int nh = 2 * n;
    const int Q = nh / 3;  // nh % 3 == R: the launcher picks the instantiation
    constexpr int QP = R % 2;  // == Q % 2
    StepInH in = load_h<WEIGHTED, V>(cx, 0);
    if constexpr (QP == 1) {
        StepInH next;
        super_step_h<WEIGHTED, 1, V, 0>(J, ring, cx, 0, in, next);
        in = next;
        for (int q = 1; q < Q; q += 2) {
            StepInH mid, nx;
            super_step_h<WEIGHTED, 0, V, 1>(J, ring, cx, 3 * q, in, mid);
            super_step_h<WEIGHTED, 1, V, 0>(J, ring, cx, 3 * q + 3, mid, nx);
            in = nx;
        }
    } else {
        for (int q = 0; q < Q; q += 2) {
            StepInH mid, nx;
            super_step_h<WEIGHTED, 0, V, 0>(J, ring, cx, 3 * q, in, mid);
            super_step_h<WEIGHTED, 1, V, 1>(J, ring, cx, 3 * q + 3, mid, nx);
            in = nx;
        }
    }
    // the tail is super-step Q, pattern Q mod 2
    if constexpr (R == 1) {
        tail_h<WEIGHTED, V, QP, 1>(J, ring, cx, 3 * Q, in);
    } else if constexpr (R == 2) {
        tail_h<WEIGHTED, V, QP, 2>(J, ring, cx, 3 * Q, in);
    } else {
        round_write<1, 1>(J, cx);
        __syncthreads();
        round_read<1, 1>(J, cx);
    }

    uint32_t bv = 0xFFFFFFFFu;
    uint32_t bi = 0xFFFFFFFFu;
    lane_argmin_h<R, 0>(J, w, l, bv, bi);
    block_select(bv, bi, w, l, send + blockIdx.x, cost_out + blk);
}

constexpr size_t kLdsBytes = kLdsDwords * sizeof(float);

template <bool WEIGHTED, int V>
hipError_t launch_h(const Problem &p, int64_t block0, int64_t nb, const float *W,
                    const float *d, const float4 *cb, uint2 *bp, int64_t bp_per_block,
                    uint32_t *send, float *cost, hipStream_t s) {
    using Kern = void (*)(const float *, int64_t, const float *, const float4 *, int, int64_t,
                          int64_t, uint2 *, int64_t, uint32_t *, float *);
    static constexpr Kern kKernels[3] = {acs_l16h_kernel<WEIGHTED, V, 0>,
                                         acs_l16h_kernel<WEIGHTED, V, 1>,
                                         acs_l16h_kernel<WEIGHTED, V, 2>};
    const Kern kern = kKernels[(2 * p.n) % 3];
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kLdsBytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), kLdsBytes, s, W,
                       p.ldw, d, cb, p.n, p.blocks_per_row, block0, bp, bp_per_block, send,
                       cost);
    return hipGetLastError();
}

}  // namespace

bool l16h_supported(const Problem &p) {
    return p.L == 16 && p.kv == 4 && (p.V == 1 || p.V == 2);
}

size_t l16h_fixed_bytes(const Problem &p) { return 3 * p.V * sizeof(float4) * kCopy; }

// two words per lane and half-step, 2n half-steps
size_t l16h_bp_bytes(const Problem &p) {
    return static_cast<size_t>(2 * p.n) * kThreads * sizeof(uint2);
}

hipError_t launch_l16h_prepare(const Problem &p, const float *C, char *ws, hipStream_t s) {
    const int total = 3 * p.V * kCopy;
    if (p.V == 2)
        hipLaunchKernelGGL(l16h_prepare_kernel<2>, dim3((total + 255) / 256), dim3(256), 0, s, C,
                           reinterpret_cast<float4 *>(ws));
    else
        hipLaunchKernelGGL(l16h_prepare_kernel<1>, dim3((total + 255) / 256), dim3(256), 0, s, C,
                           reinterpret_cast<float4 *>(ws));
    return hipGetLastError();
}

hipError_t launch_acs_l16h(const Problem &p, const Plan &pl, const float *W, const float *d,
                           int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s) {
    char *per = ws + pl.fixed;
    uint2 *bp = reinterpret_cast<uint2 *>(per);
    uint32_t *send = reinterpret_cast<uint32_t *>(per + nb * pl.bp_bytes);
    const float4 *cb = reinterpret_cast<const float4 *>(ws);
    const int64_t bpb = static_cast<int64_t>(pl.bp_bytes / sizeof(uint2));
    if (p.V == 2)
        return d ? launch_h<true, 2>(p, block0, nb, W, d, cb, bp, bpb, send, cost, s)
                 : launch_h<false, 2>(p, block0, nb, W, d, cb, bp, bpb, send, cost, s);
    return d ? launch_h<true, 1>(p, block0, nb, W, d, cb, bp, bpb, send, cost, s)
             : launch_h<false, 1>(p, block0, nb, W, d, cb, bp, bpb, send, cost, s);
}

}  // namespace tcq
