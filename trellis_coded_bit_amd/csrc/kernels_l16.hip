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

#include "l16_layout.h"
#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

using namespace l16;

constexpr int kThreads = kWaves * kLanes;  // 512
constexpr int kCopy = kWaves * kGroupsPerLane * kLanes;  // float4 entries per copy
constexpr int kPrefetch = 8;                            // groups of codebook in flight

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

// Shift one bit per lane, taken from a wave-wide compare mask, into acc:
// acc = 2 * acc + mask[lane] in a single VALU op (carry-in from an SGPR pair).
__device__ __forceinline__ uint32_t shift_in(uint32_t acc, uint64_t mask) {
    uint32_t r;
    asm("v_addc_co_u32 %0, vcc, %1, %1, %2" : "=v"(r) : "v"(acc), "s"(mask) : "vcc");
    return r;
}

// Path costs are non-negative floats (sums of d * e * e >= 0 starting from +0, never
// -0), so their bit patterns order exactly like their values: minima and compares run
// on the unsigned bit patterns, which needs no NaN canonicalization.
//
// Codebook copy entry for group g of step P: a raw buffer load whose per-lane offset
// (voff = 16 * lane) is shared by every load and whose group/step offset is a scalar.
template <int P>
__device__ __forceinline__ float4 cb_load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int g) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        rs, voff, ((P - 1) * kCopy + g * kLanes) * static_cast<int>(sizeof(float4)), 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}

// One trellis step at position P (1..3) of the super-step.  `rs` addresses the wave's
// part of the codebook copies.
template <int P, bool WEIGHTED>
__device__ __forceinline__ void acs_step(uint32_t (&J)[kRegs], __amdgpu_buffer_rsrc_t rs,
                                         uint32_t voff, float wt, float dt,
                                         uint2 *__restrict__ bp_out) {
    float4 ring[kPrefetch];
#pragma unroll
    for (int g = 0; g < kPrefetch; ++g) ring[g] = cb_load<P>(rs, voff, g);
    uint32_t acc0 = 0, acc1 = 0;
#pragma unroll
    for (int g = 0; g < kGroupsPerLane; ++g) {
        // keep at most kPrefetch codebook loads in flight: later loads stay below this
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        const float4 c = ring[g % kPrefetch];
        if (g + kPrefetch < kGroupsPerLane) ring[g % kPrefetch] = cb_load<P>(rs, voff, g + kPrefetch);
        const int r0 = group_reg(P, g, 0), r1 = group_reg(P, g, 1);
        const int r2 = group_reg(P, g, 2), r3 = group_reg(P, g, 3);
        const uint32_t u0 = J[r0], u1 = J[r1], u2 = J[r2], u3 = J[r3];
        const uint32_t m01 = u0 < u1 ? u0 : u1;
        const uint32_t m23 = u2 < u3 ? u2 : u3;
        const uint32_t mu = m01 < m23 ? m01 : m23;
        const uint64_t c01 = __ballot(u1 < u0);
        const uint64_t c23 = __ballot(u3 < u2);
        const uint64_t chi = __ballot(m23 < m01);
        const uint64_t b0 = (chi & c23) | (~chi & c01);
        uint32_t &acc = (g < 16) ? acc0 : acc1;
        acc = shift_in(shift_in(acc, chi), b0);
        const float m = __uint_as_float(mu);
        const float e0 = wt - c.x, e1 = wt - c.y, e2 = wt - c.z, e3 = wt - c.w;
        J[r0] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e0 : e0, e0, m));
        J[r1] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e1 : e1, e1, m));
        J[r2] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e2 : e2, e2, m));
        J[r3] = __float_as_uint(__builtin_fmaf(WEIGHTED ? dt * e3 : e3, e3, m));
    }
    *bp_out = make_uint2(acc0, acc1);
}

// Re-lay the costs out for the next super-step (two LDS rounds split on r[6]).
__device__ __forceinline__ void transpose(uint32_t (&J)[kRegs], uint32_t *__restrict__ lds,
                                          uint32_t wlane, uint32_t rlane) {
    uint32_t Jn[kRegs];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 64; ++r) lds[wlane + lds_write_reg(r)] = J[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRegs; r += 2) Jn[r] = lds[rlane + lds_read_reg(r)];
    __syncthreads();
#pragma unroll
    for (int r = 64; r < kRegs; ++r) lds[wlane + lds_write_reg(r)] = J[r];
    __syncthreads();
#pragma unroll
    for (int r = 1; r < kRegs; r += 2) Jn[r] = lds[rlane + lds_read_reg(r)];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) J[r] = Jn[r];
}

template <int P>
__device__ __forceinline__ void lane_argmin(const uint32_t (&J)[kRegs], uint32_t w,
                                            uint32_t l, uint32_t &bv, uint32_t &bi) {
    // the state of slot (w, l, r) is the OR of a lane/wave part and a register part
    const uint32_t lanepart = state_of(P, w, l, 0);
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
        const uint32_t s = lanepart | state_of(P, 0, 0, r);
        const uint32_t v = J[r];
        if (v < bv || (v == bv && s < bi)) {
            bv = v;
            bi = s;
        }
    }
}

template <bool WEIGHTED>
__global__ __launch_bounds__(kThreads, 1) void acs_l16_kernel(
    const float *__restrict__ W, int64_t ldw, const float *__restrict__ d,
    const float4 *__restrict__ cb, int n, int64_t blocks_per_row, int64_t block0,
    uint2 *__restrict__ bp, int64_t bp_per_block, uint32_t *__restrict__ send,
    float *__restrict__ cost_out) {
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t red_v[kWaves];
    __shared__ uint32_t red_i[kWaves];

    const uint32_t tid = threadIdx.x;
    const uint32_t w = tid >> 6;
    const uint32_t l = tid & 63;
    const int64_t blk = block0 + blockIdx.x;
    const int64_t row = blk / blocks_per_row;
    const int64_t col = blk % blocks_per_row;
    const float *wrow = W + row * ldw + col * n;
    const float *drow = WEIGHTED ? d + col * n : nullptr;
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform
    // CDNA buffer descriptor word 3 (raw dword access), as used for gfx9-family parts
    const __amdgpu_buffer_rsrc_t cbw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float4 *>(cb + (wu * kGroupsPerLane) * kLanes), 0,
        3 * kCopy * static_cast<int>(sizeof(float4)), 0x00020000);
    const uint32_t cbvoff = l * static_cast<uint32_t>(sizeof(float4));
    uint2 *bpl = bp + blockIdx.x * bp_per_block + (w * kLanes + l);
    const uint32_t wlane = lds_write_lane(w, l);
    const uint32_t rlane = lds_read_lane(w, l);

    uint32_t J[kRegs];  // fp32 costs held as their bit patterns
#pragma unroll
    for (int r = 0; r < kRegs; ++r) J[r] = 0u;

    const int Q = n / 3;
    const int R = n % 3;
    int t = 0;
    for (int q = 0; q < Q; ++q) {
        acs_step<1, WEIGHTED>(J, cbw, cbvoff, wrow[t], WEIGHTED ? drow[t] : 1.0f, bpl + t * kThreads);
        acs_step<2, WEIGHTED>(J, cbw, cbvoff, wrow[t + 1], WEIGHTED ? drow[t + 1] : 1.0f,
                              bpl + (t + 1) * kThreads);
        acs_step<3, WEIGHTED>(J, cbw, cbvoff, wrow[t + 2], WEIGHTED ? drow[t + 2] : 1.0f,
                              bpl + (t + 2) * kThreads);
        t += 3;
        if (t < n) transpose(J, lds, wlane, rlane);
    }
    if (R >= 1)
        acs_step<1, WEIGHTED>(J, cbw, cbvoff, wrow[t], WEIGHTED ? drow[t] : 1.0f, bpl + t * kThreads);
    if (R >= 2)
        acs_step<2, WEIGHTED>(J, cbw, cbvoff, wrow[t + 1], WEIGHTED ? drow[t + 1] : 1.0f,
                              bpl + (t + 1) * kThreads);

    uint32_t bv = 0xFFFFFFFFu;  // above every finite or infinite cost pattern
    uint32_t bi = 0xFFFFFFFFu;
    if (R == 1)
        lane_argmin<1>(J, w, l, bv, bi);
    else if (R == 2)
        lane_argmin<2>(J, w, l, bv, bi);
    else
        lane_argmin<3>(J, w, l, bv, bi);
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t ov = __shfl_xor(bv, off);
        const uint32_t oi = __shfl_xor(bi, off);
        if (ov < bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (l == 0) {
        red_v[w] = bv;
        red_i[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < kWaves; ++k) {
            if (red_v[k] < bv || (red_v[k] == bv && red_i[k] < bi)) {
                bv = red_v[k];
                bi = red_i[k];
            }
        }
        send[blockIdx.x] = bi;
        cost_out[blk] = __uint_as_float(bv);
    }
}

// One wave per block: follow the remembered predecessors back from the end state and
// pack the 2-bit chunks b_1..b_n, MSB first, into MSB-first words.
__global__ __launch_bounds__(64) void traceback_l16_kernel(
    const uint2 *__restrict__ bp, int64_t bp_per_block, const uint32_t *__restrict__ send,
    int n, int nwords, int64_t block0, uint32_t *__restrict__ bitstream,
    uint32_t *__restrict__ start_state) {
    __shared__ uint8_t chunk[TCQ_MAX_STEPS];
    const int lane = threadIdx.x;
    const uint2 *bpb = bp + blockIdx.x * bp_per_block;
    const int64_t blk = block0 + blockIdx.x;
    if (lane == 0) {
        uint32_t s = send[blockIdx.x];
        for (int t = n; t >= 1; --t) {
            const int p = (t - 1) % 3 + 1;
            const Slot sl = slot_of(p, s);
            const uint32_t g = reg_group(p, sl.r);
            const uint2 word = bpb[(t - 1) * kThreads + sl.w * kLanes + sl.l];
            const uint32_t bits = (g < 16) ? word.x : word.y;
            const uint32_t jb = (bits >> (2 * (15 - (g & 15)))) & 3u;
            chunk[t - 1] = static_cast<uint8_t>(s & 3u);
            s = (jb << 14) | (s >> 2);
        }
        start_state[blk] = s;
    }
    __syncthreads();
    for (int wi = lane; wi < nwords; wi += 64) {
        uint32_t word = 0;
        for (int q = 0; q < 16; ++q) {
            const int ci = wi * 16 + q;
            if (ci < n) word |= static_cast<uint32_t>(chunk[ci]) << (30 - 2 * q);
        }
        bitstream[blk * nwords + wi] = word;
    }
}

constexpr size_t kLdsBytes = kLdsDwords * sizeof(float);

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
    if (d) {
        auto kern = acs_l16_kernel<true>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(kLdsBytes));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), kLdsBytes, s,
                           W, p.ldw, d, cb, p.n, p.blocks_per_row, block0, bp, bp_per_block,
                           send, cost);
    } else {
        auto kern = acs_l16_kernel<false>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(kLdsBytes));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), kLdsBytes, s,
                           W, p.ldw, d, cb, p.n, p.blocks_per_row, block0, bp, bp_per_block,
                           send, cost);
    }
    return hipGetLastError();
}

hipError_t launch_traceback_l16(const Problem &p, const Plan &pl, int64_t block0, int64_t nb,
                                const char *ws, uint32_t *bitstream, uint32_t *start_state,
                                hipStream_t s) {
    const char *per = ws + pl.fixed;
    const uint2 *bp = reinterpret_cast<const uint2 *>(per);
    const uint32_t *send = reinterpret_cast<const uint32_t *>(per + nb * pl.bp_bytes);
    const int nwords = (p.k * p.T + 31) / 32;
    hipLaunchKernelGGL(traceback_l16_kernel, dim3(static_cast<unsigned>(nb)), dim3(64), 0, s, bp,
                       static_cast<int64_t>(pl.bp_bytes / sizeof(uint2)), send, p.n, nwords,
                       block0, bitstream, start_state);
    return hipGetLastError();
}

}  // namespace tcq
