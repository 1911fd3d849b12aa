// Generic Viterbi path: any supported (L, k, V, T).  One workgroup per coding block,
// groups of states across threads, cost vectors double-buffered in LDS (L <= 13) or in
// the workspace (larger L, L2-resident per block), backpointers as bit-planes.
//
// The step (Pingala-8 post, Viterbi paragraph: each state retains its lowest-cost
// incoming path; bitshift structure from the QTIP abstract; weighted metric from the CurveTQ
// abstract): the predecessors of s' = (x << kv) | b are (j << (L-kv)) | x, so one
// min/argmin per group x serves its 2^kv successors.  Starting every state at cost +0
// before step 1 is the free start: step 1 then extends +0 by the branch metric, and
// the remembered predecessor of group x is j = 0, i.e. s_0 = x = s_1 >> kv.
#include <hip/hip_runtime.h>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float branch_chain(float acc, const float *wv, const float *dv,
                                              const float *__restrict__ c, int V,
                                              bool weighted) {
    for (int v = 0; v < V; ++v) {
        const float e = wv[v] - c[v];
        const float de = weighted ? dv[v] * e : e;
        acc = __builtin_fmaf(de, e, acc);
    }
    return acc;
}

// bp layout per block: [step t-1][plane p][ceil(ngroups/64)] uint64; bit (x mod 64) of
// word x/64 of plane p is bit p of the predecessor index kept for group x at step t.
template <bool WEIGHTED, bool IN_LDS>
__global__ __launch_bounds__(kThreads) void acs_generic_kernel(
    const float *__restrict__ W, int64_t ldw, const float *__restrict__ d,
    const float *__restrict__ C, int L, int kv, int V, int n, int64_t blocks_per_row,
    int64_t block0, uint64_t *__restrict__ bp, int64_t bp_words_per_block,
    float *__restrict__ gcost, int64_t gcost_per_block, uint32_t *__restrict__ send,
    float *__restrict__ cost_out) {
    extern __shared__ float lds[];
    __shared__ float red_v[kThreads / 64];
    __shared__ uint32_t red_i[kThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t blk = block0 + blockIdx.x;
    const int64_t row = blk / blocks_per_row;
    const int64_t col = blk % blocks_per_row;
    const int T = n * V;
    const float *w = W + row * ldw + col * T;
    const float *dd = WEIGHTED ? d + col * T : nullptr;

    const int64_t nstates = int64_t{1} << L;
    const int64_t ngroups = int64_t{1} << (L - kv);
    const int G = 1 << kv;
    const int sh = L - kv;
    const int64_t nw64 = (ngroups + 63) / 64;

    float *J = IN_LDS ? lds : gcost + blockIdx.x * gcost_per_block;
    float *Jn = J + nstates;
    uint64_t *bpb = bp + blockIdx.x * bp_words_per_block;

    for (int64_t s = tid; s < nstates; s += kThreads) J[s] = 0.0f;
    __syncthreads();

    float wv[TCQ_MAX_V], dv[TCQ_MAX_V];
    for (int t = 1; t <= n; ++t) {
        for (int v = 0; v < V; ++v) {
            wv[v] = w[(t - 1) * V + v];
            dv[v] = WEIGHTED ? dd[(t - 1) * V + v] : 1.0f;
        }
        for (int64_t base = 0; base < ngroups; base += kThreads) {
            const int64_t x = base + tid;
            const bool act = x < ngroups;
            int jb = 0;
            if (act) {
                float m = J[x];
                for (int j = 1; j < G; ++j) {
                    const float c = J[(static_cast<int64_t>(j) << sh) | x];
                    if (c < m) {
                        m = c;
                        jb = j;
                    }
                }
                for (int b = 0; b < G; ++b) {
                    const int64_t sn = (x << kv) | b;
                    Jn[sn] = branch_chain(m, wv, dv, C + sn * V, V, WEIGHTED);
                }
            }
            const int64_t x0 = base + (tid & ~63);  // group of this wave's lane 0
            for (int p = 0; p < kv; ++p) {
                const uint64_t mask = __ballot(act && ((jb >> p) & 1));
                if (lane == 0 && x0 < ngroups)
                    bpb[(static_cast<int64_t>(t - 1) * kv + p) * nw64 + (x0 >> 6)] = mask;
            }
        }
        __syncthreads();
        float *tmp = J;
        J = Jn;
        Jn = tmp;
    }

    // lowest-index minimum over the final cost vector.  A thread's first state is taken
    // unconditionally, so a vector of +inf costs (squares that overflowed) still selects
    // a real state -- the lowest one, as the reduction below breaks ties by index --
    // and never leaves the 0xFFFFFFFF marker of threads that own no state.
    float bv = __builtin_inff();
    uint32_t bi = 0xFFFFFFFFu;
    for (int64_t s = tid; s < nstates; s += kThreads) {
        const float v = J[s];
        if (bi == 0xFFFFFFFFu || v < bv) {
            bv = v;
            bi = static_cast<uint32_t>(s);
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const uint32_t oi = __shfl_xor(bi, off);
        if (ov < bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        red_v[tid >> 6] = bv;
        red_i[tid >> 6] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int wv_ = 1; wv_ < kThreads / 64; ++wv_) {
            if (red_v[wv_] < bv || (red_v[wv_] == bv && red_i[wv_] < bi)) {
                bv = red_v[wv_];
                bi = red_i[wv_];
            }
        }
        send[blockIdx.x] = bi;
        cost_out[blk] = bv;
    }
}

// One wave per block: chase the remembered predecessors from the chosen end state,
// then pack the chunks b_1..b_n (kv bits each, MSB first) into MSB-first words.
__global__ __launch_bounds__(64) void traceback_planes_kernel(
    const uint64_t *__restrict__ bp, int64_t bp_words_per_block,
    const uint32_t *__restrict__ send, int L, int kv, int n, int nwords, int64_t block0,
    uint32_t *__restrict__ bitstream, uint32_t *__restrict__ start_state) {
    __shared__ uint8_t chunk[TCQ_MAX_STEPS];
    const int lane = threadIdx.x;
    const uint64_t *bpb = bp + blockIdx.x * bp_words_per_block;
    const int64_t blk = block0 + blockIdx.x;
    const int sh = L - kv;
    const int64_t nw64 = ((int64_t{1} << sh) + 63) / 64;
    if (lane == 0) {
        uint32_t s = send[blockIdx.x];
        const uint32_t gmask = (1u << kv) - 1u;
        for (int t = n; t >= 1; --t) {
            const uint32_t x = s >> kv;
            chunk[t - 1] = static_cast<uint8_t>(s & gmask);
            uint32_t jb = 0;
            for (int p = 0; p < kv; ++p) {
                const uint64_t word = bpb[(static_cast<int64_t>(t - 1) * kv + p) * nw64 + (x >> 6)];
                jb |= static_cast<uint32_t>((word >> (x & 63)) & 1u) << p;
            }
            s = (jb << sh) | x;
        }
        start_state[blk] = s;
    }
    __syncthreads();
    const int total = n * kv;
    for (int wi = lane; wi < nwords; wi += 64) {
        uint32_t word = 0;
        for (int q = 0; q < 32; ++q) {
            const int pos = wi * 32 + q;
            if (pos < total) {
                const int ci = pos / kv;
                const int within = kv - 1 - pos % kv;
                word |= ((static_cast<uint32_t>(chunk[ci]) >> within) & 1u) << (31 - q);
            }
        }
        bitstream[blk * nwords + wi] = word;
    }
}

template <bool W, bool LDS>
hipError_t launch_one(const Problem &p, const Plan &pl, const float *Wm, const float *d,
                      const float *C, int64_t block0, int64_t nb, char *ws, float *cost,
                      hipStream_t s) {
    const size_t shmem = LDS ? 2 * static_cast<size_t>(p.nstates) * sizeof(float) : 0;
    auto kern = acs_generic_kernel<W, LDS>;
    if (shmem > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(shmem));
        if (e != hipSuccess) return e;
    }
    char *per = ws + pl.fixed;
    uint64_t *bp = reinterpret_cast<uint64_t *>(per);
    float *gcost = reinterpret_cast<float *>(per + nb * pl.bp_bytes);
    uint32_t *send = reinterpret_cast<uint32_t *>(per + nb * (pl.bp_bytes + pl.cost_bytes));
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(kThreads), shmem, s, Wm,
                       p.ldw, d, C, p.L, p.kv, p.V, p.n, p.blocks_per_row, block0, bp,
                       static_cast<int64_t>(pl.bp_bytes / 8), gcost,
                       static_cast<int64_t>(pl.cost_bytes / 4), send, cost);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_acs_generic(const Problem &p, const Plan &pl, const float *W,
                              const float *d, const float *C, int64_t block0, int64_t nb,
                              char *ws, float *cost, hipStream_t s) {
    const bool lds = pl.variant == kGenericLds;
    if (d) {
        return lds ? launch_one<true, true>(p, pl, W, d, C, block0, nb, ws, cost, s)
                   : launch_one<true, false>(p, pl, W, d, C, block0, nb, ws, cost, s);
    }
    return lds ? launch_one<false, true>(p, pl, W, d, C, block0, nb, ws, cost, s)
               : launch_one<false, false>(p, pl, W, d, C, block0, nb, ws, cost, s);
}

hipError_t launch_traceback_planes(const Problem &p, const Plan &pl, int64_t block0,
                                   int64_t nb, const char *ws, uint32_t *bitstream,
                                   uint32_t *start_state, hipStream_t s) {
    const char *per = ws + pl.fixed;
    const uint64_t *bp = reinterpret_cast<const uint64_t *>(per);
    const uint32_t *send =
        reinterpret_cast<const uint32_t *>(per + nb * (pl.bp_bytes + pl.cost_bytes));
    const int nwords = (p.k * p.T + 31) / 32;
    hipLaunchKernelGGL(traceback_planes_kernel, dim3(static_cast<unsigned>(nb)), dim3(64), 0,
                       s, bp, static_cast<int64_t>(pl.bp_bytes / 8), send, p.L, p.kv, p.n,
                       nwords, block0, bitstream, start_state);
    return hipGetLastError();
}

}  // namespace tcq
