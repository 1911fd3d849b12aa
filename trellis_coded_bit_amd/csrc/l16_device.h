// Device helpers shared by the L = 16 forward kernels (k*V = 2, 3 and 4): the per-block
// context, the carry shift-in of compare masks, the two LDS rounds of the transposition
// (layout in l16_layout.h) and their parts spread over a segment's groups, and the
// lane's lowest (cost, state) at the end.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "l16_layout.h"

namespace tcq {
namespace l16 {

constexpr int kThreads = kWaves * kLanes;                // 512
constexpr int kCopy = kWaves * kGroupsPerLane * kLanes;  // float4 entries per codebook copy

// Shift one bit per lane, taken from a wave-wide compare mask, into acc:
// acc = 2 * acc + mask[lane] in a single VALU op (carry-in from an SGPR pair).
__device__ __forceinline__ uint32_t shift_in(uint32_t acc, uint64_t mask) {
    uint32_t r;
    asm volatile("v_addc_co_u32 %0, vcc, %1, %1, %2" : "=v"(r) : "v"(acc), "s"(mask) : "vcc");
    return r;
}

// Minimum of four cost patterns and the index j of its first occurrence (the lowest j on
// ties), as two wave-wide bit masks: hi = j >> 1, lo = j & 1.  Two VALU minimums and
// three equality compares (into SGPR masks); the index bits are assembled on the SALU:
//   j = 0 if u0 is the minimum, else 1 if u1 is, else 2 if u2 is, else 3.
__device__ __forceinline__ uint32_t argmin4(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3,
                                            uint64_t &hi, uint64_t &lo) {
    const uint32_t m01 = u0 < u1 ? u0 : u1;  // the backend fuses these two into v_min3
    const uint32_t m3 = m01 < u2 ? m01 : u2;
    const uint32_t mu = m3 < u3 ? m3 : u3;
    const uint64_t e0 = __ballot(u0 == mu);
    const uint64_t e1 = __ballot(u1 == mu);
    const uint64_t e2 = __ballot(u2 == mu);
    hi = ~(e0 | e1);
    lo = ~e0 & (e1 | ~e2);
    return mu;
}

// Per-block context shared by the segments and transposition rounds.
struct Ctx {
    __amdgpu_buffer_rsrc_t rs;  // wave's part of the codebook copies
    uint32_t voff;              // 16 * lane
    const float *wcol;          // the block's T weights
    const float *dcol;          // the block's T values of d (weighted only)
    uint32_t *bp;               // lane's backpointer words: + 2 * kThreads * t + half
    int nw;                     // weights in the block
    uint32_t wb[2];             // LDS byte bases for round writes
    uint32_t rb[4];             // LDS byte bases for round reads
};

// Context of one coding block (row, col) for lane l of wave w; n is the block length in
// weights.  The `copies` codebook copies start at cb; each wave addresses its own
// 2048-entry slice of every copy through a raw buffer descriptor, so every load is
// (16 * lane) + scalar offset + immediate.
__device__ __forceinline__ Ctx make_ctx(const float *W, int64_t ldw, const float *d,
                                        const float4 *cb, int n, int64_t row, int64_t col,
                                        uint32_t w, uint32_t l, uint2 *bp_block,
                                        int copies = 3) {
    Ctx cx;
    const uint32_t wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform
    cx.wcol = W + row * ldw + col * n;
    cx.nw = n;
    // the offset, not the pointer, is selected: d keeps its provenance, so its per-step
    // values are read with scalar loads (a vector load's wait would drain the codebook
    // loads in flight)
    cx.dcol = d + (d ? col * n : 0);
    // CDNA buffer descriptor word 3 (raw dword access), as used for gfx9-family parts
    cx.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float4 *>(cb + wu * (kCopy / kWaves)),
                                              0, copies * kCopy * static_cast<int>(sizeof(float4)),
                                              0x00020000);
    cx.voff = l * static_cast<uint32_t>(sizeof(float4));
    cx.bp = reinterpret_cast<uint32_t *>(bp_block + (w * kLanes + l));
    // LDS bases, kept opaque so that every access is base + 16-bit immediate
    const uint32_t wlane = 4u * lds_write_lane(w, l);
    const uint32_t rlane = 4u * lds_read_lane(w, l);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        cx.wb[k] = wlane + k * 4u * 2112u * 8u;
        asm volatile("" : "+v"(cx.wb[k]));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        cx.rb[k] = rlane + k * 4u * 2112u * 4u;
        asm volatile("" : "+v"(cx.rb[k]));
    }
    return cx;
}

// The block's backpointer words through a buffer descriptor: the lane's byte offset in a
// VGPR and the step in the scalar offset, so that a store needs no per-step address
// arithmetic in VGPRs.  store(word, v) has the effect of cx.bp[word] = v, `word`
// (= 2 * kThreads * step + half) being wave-uniform.
struct BpBuf {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off;
    __device__ __forceinline__ void store(int word, uint32_t v) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, rs, static_cast<int>(off),
                                              word * static_cast<int>(sizeof(uint32_t)), 0);
    }
};
__device__ __forceinline__ BpBuf make_bpbuf(uint2 *bp_block, int64_t bp_per_block,
                                            uint32_t w, uint32_t l) {
    BpBuf b;
    b.rs = __builtin_amdgcn_make_buffer_rsrc(
        bp_block, 0, static_cast<int>(bp_per_block * static_cast<int64_t>(sizeof(uint2))),
        0x00020000);
    b.off = (w * kLanes + l) * static_cast<uint32_t>(sizeof(uint2));
    return b;
}

// Weight and d of the three steps of a super-step, held in scalar registers.  They are
// requested one super-step ahead and complete at a workgroup barrier (which waits for
// every LDS and scalar-memory operation), so their use needs no wait: a wait for a
// scalar load is a wait for every LDS operation in flight, which would serialise the
// transposition rounds.
struct StepIn {
    float w[3], d[3];
};
// Steps t0 .. t0 + 2 of a block with one weight per step, each index clamped to the
// block's last weight (past the end the values are never used).
template <bool WEIGHTED>
__device__ __forceinline__ StepIn load_steps(const Ctx &cx, int t0) {
    StepIn s;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int t = t0 + p < cx.nw ? t0 + p : cx.nw - 1;
        s.w[p] = cx.wcol[t];
        s.d[p] = WEIGHTED ? cx.dcol[t] : 1.0f;
    }
    return s;
}

extern __shared__ uint32_t lds_stage[];

__device__ __forceinline__ void lds_put(uint32_t base, uint32_t off, uint32_t v) {
    *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(lds_stage) + base + off) = v;
}
__device__ __forceinline__ uint32_t lds_get(uint32_t base, uint32_t off) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds_stage) + base +
                                               off);
}

// Transposition rounds (l16_layout.h).  Round RHO writes the logical registers with
// r[6] = RHO of naming NM and reads the logical registers with r'[0] = RHO of naming
// 1 - NM; both touch the same physical registers.
template <int NM, int RHO>
__device__ __forceinline__ void round_write(const uint32_t (&J)[kRegs], const Ctx &cx) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const uint32_t r = 64u * RHO + i;
        const uint32_t off = 4u * lds_write_reg(r);
        lds_put(cx.wb[bit(r, 4)], off - bit(r, 4) * 4u * 2112u * 8u, J[phys(NM, r)]);
    }
}
// Registers I0 .. I0 + CNT - 1 of round RHO (the part of round_write a segment issues
// between its groups).
template <int NM, int RHO, int I0, int CNT>
__device__ __forceinline__ void round_write_range(const uint32_t (&J)[kRegs], const Ctx &cx) {
#pragma unroll
    for (int i = I0; i < I0 + CNT; ++i) {
        const uint32_t r = 64u * RHO + i;
        const uint32_t off = 4u * lds_write_reg(r);
        lds_put(cx.wb[bit(r, 4)], off - bit(r, 4) * 4u * 2112u * 8u, J[phys(NM, r)]);
    }
}
// The four registers of group g = 2 i + RHO at step 1 (the registers the next segment
// that needs round RHO consumes together).
template <int NM, int RHO, int I>
__device__ __forceinline__ void round_read_group(uint32_t (&J)[kRegs], const Ctx &cx) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        constexpr uint32_t g = 2u * I + RHO;
        const uint32_t r = group_reg(1, g, b);
        const uint32_t off = 4u * lds_read_reg(r);
        const uint32_t k = off / (4u * 2112u * 4u);
        J[phys(1 - NM, r)] = lds_get(cx.rb[k], off - k * 4u * 2112u * 4u);
    }
}
template <int NM, int RHO, int... I>
__device__ __forceinline__ void round_read_groups(uint32_t (&J)[kRegs], const Ctx &cx,
                                                  std::integer_sequence<int, I...>) {
    (round_read_group<NM, RHO, I>(J, cx), ...);
}
// std::integer_sequence<int, K + I...>
template <int K, int... I>
__device__ __forceinline__ constexpr std::integer_sequence<int, (K + I)...> shifted_seq(
    std::integer_sequence<int, I...>) {
    return {};
}
// All 64 registers r[0] = RHO, group by group.
template <int NM, int RHO>
__device__ __forceinline__ void round_read(uint32_t (&J)[kRegs], const Ctx &cx) {
    round_read_groups<NM, RHO>(J, cx, std::make_integer_sequence<int, 16>{});
}

// LDS work spread over the groups of a segment, so that a transposition round drains
// while the VALU computes instead of in one burst behind a barrier (every wave reaches
// the burst at the same time, and a wave issues nothing else until its LDS queue has
// taken the whole burst).  After group I of the segment, `step<I>` issues its share.
// Round RHO of naming NM written PER registers per group, from register I0 + PER * I of
// the round (pairs of consecutive registers share one ds_write2).
template <int NM, int RHO, int PER, int I0>
struct WriteLds {
    template <int I>
    __device__ __forceinline__ void step(uint32_t (&J)[kRegs], const Ctx &cx) const {
        round_write_range<NM, RHO, I0 + PER * I, PER>(J, cx);
    }
};
// Round 0 of naming NM written behind the segment of the super-step's last step that
// covers the r[6] = 0 half, whose group I holds registers GS * I .. GS * I + GS - 1
// (GS = 4 for 2-bit steps, 8 for 3-bit steps): after group I the registers of group
// I - 1, whose costs are final; the caller writes the last group's after the segment.
template <int NM, int GS>
struct WriteRound0Lagged {
    template <int I>
    __device__ __forceinline__ void step(uint32_t (&J)[kRegs], const Ctx &cx) const {
        if constexpr (I >= 1) round_write_range<NM, 0, GS * (I - 1), GS>(J, cx);
    }
};
// Round RHO read into naming 1 - NM, PER of its 16 register groups per group.
template <int NM, int RHO, int PER>
struct ReadLds {
    template <int I>
    __device__ __forceinline__ void step(uint32_t (&J)[kRegs], const Ctx &cx) const {
        round_read_groups<NM, RHO>(J, cx, shifted_seq<PER * I>(std::make_integer_sequence<int, PER>{}));
    }
};

// The lane's registers in ascending order of Key::of(r), the register part of the state a
// register holds (the lane part is common to all of them and occupies other bits, so this
// is also the order of the full states).
template <class Key>
struct AscendingRegs {
    int r[kRegs];
    constexpr AscendingRegs() : r{} {
        for (int i = 0; i < kRegs; ++i) r[i] = i;
        for (int i = 1; i < kRegs; ++i)
            for (int j = i; j > 0 && Key::of(r[j]) < Key::of(r[j - 1]); --j) {
                const int t = r[j];
                r[j] = r[j - 1];
                r[j - 1] = t;
            }
    }
};
template <class Key, int NM, int... K>
__device__ __forceinline__ void lane_best_impl(const uint32_t (&J)[kRegs], uint32_t &bv,
                                               uint32_t &bs, std::integer_sequence<int, K...>) {
    constexpr AscendingRegs<Key> ord{};
    // strict '<' in ascending state order keeps the lowest state among equal costs; every
    // cost pattern is below 0xFFFFFFFF (costs are never negative), so the first register
    // always replaces the start value
    ((bs = J[phys(NM, ord.r[K])] < bv ? Key::of(ord.r[K]) : bs,
      bv = J[phys(NM, ord.r[K])] < bv ? J[phys(NM, ord.r[K])] : bv),
     ...);
}
// The lane's smallest cost pattern bv and, among its registers of that cost, the lowest
// state lanepart | Key::of(r), in branch-free selects (the branchy form of this loop left
// the compiler short of registers and spilling in the kernels' last lines).
template <class Key, int NM>
__device__ __forceinline__ void lane_best(const uint32_t (&J)[kRegs], uint32_t lanepart,
                                          uint32_t &bv, uint32_t &bi) {
    uint32_t v = 0xFFFFFFFFu, s = 0u;
    lane_best_impl<Key, NM>(J, v, s, std::make_integer_sequence<int, kRegs>{});
    bv = v;
    bi = lanepart | s;
}

// Lowest-index minimum over the workgroup: (bv, bi) are each lane's best cost pattern
// and state; lane 0 of wave 0 writes the chosen end state and its cost.
__device__ __forceinline__ void block_select(uint32_t bv, uint32_t bi, uint32_t w, uint32_t l,
                                             uint32_t *send_slot, float *cost_slot) {
    __shared__ uint32_t red_v[kWaves];
    __shared__ uint32_t red_i[kWaves];
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
    if (w == 0 && l == 0) {
        for (int k = 1; k < kWaves; ++k) {
            if (red_v[k] < bv || (red_v[k] == bv && red_i[k] < bi)) {
                bv = red_v[k];
                bi = red_i[k];
            }
        }
        *send_slot = bi;
        *cost_slot = __uint_as_float(bv);
    }
}

}  // namespace l16
}  // namespace tcq
