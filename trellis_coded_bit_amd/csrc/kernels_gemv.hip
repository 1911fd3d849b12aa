// y = W_hat x with the weights decoded inside the product (Pingala-8 post, decoding
// paragraph: decoding reads bits, updates the state and looks values up, inside the
// matrix-vector product).
//
// The state of step t is the L-bit window of s_0 || b_1 || ... || b_n that ends with
// chunk b_t, so it can be read straight from two neighbouring 32-bit words of the stream
// (the word before the first one being s_0).  A lane owns one stream word and decodes
// every step whose chunk ends inside it.
//
// The codebook (2^L x V floats; 256 KiB at L=16, V=1) is read at random, one entry per
// step.  From L2 every such read pulls a whole cache line into L1, so the table is staged
// through LDS instead, up to 128 KiB at a time: P = table / part passes over the stream,
// each adding the products whose state falls in the part held in LDS.  Each wave keeps
// the same rows in every pass and adds its part sums to y in pass order, so results are
// deterministic.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

constexpr int kGemvThreads = 1024;
constexpr int kGemvWaves = kGemvThreads / 64;  // rows in flight per workgroup
constexpr int64_t kGemvPartBytes = 128 << 10;     // largest codebook part in LDS
constexpr int64_t kGemvMinPartBytes = 32 << 10;   // smallest part worth staging x for
constexpr int64_t kGemvLdsBytes = 152 << 10;      // dynamic LDS used at most

struct GemvArgs {
    const uint32_t *bits;
    const uint32_t *s0;
    const float *C;
    const float *x;
    float *y;
    int64_t M;
    int64_t bpr;        // blocks per row
    int nwords;         // stream words per block
    int64_t wpr;        // stream words per row = bpr * nwords
    int L, kv, V, n, T;
    int part_log2;      // log2(states per part)
    int parts;
    int64_t step_c;     // 64 / nwords: blocks advanced per 64 words
    int step_j;         // 64 % nwords
    int64_t xt_len;     // floats of x staged in LDS (tiled kernel)
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Tiled kernel.  A unit is U = KV / gcd(KV, 32) stream words holding exactly S = 32 U / KV
// whole steps; every block's stream is a whole number of units, so step q of row unit u
// is step g = u S + q of the row and multiplies x[g V + v].  x is staged once per
// workgroup in LDS in the order [tile of 64 units][q][lane][v], which makes the reads of
// a wave for one q contiguous.  R waves share a row (R = 1 unless the rows are too few
// to give every CU a workgroup): wave r of the group takes the row's tiles of 64 units
// r, r + R, ..., lane l owning the l-th unit of each; the 64 lane sums meet in a shuffle
// tree, and the R wave sums are added in order through LDS.  A step whose state is in
// another codebook part multiplies an exact 0 (its table read is masked off), which
// leaves the sum unchanged.
template <int KV, int V, int R>
__global__ __launch_bounds__(kGemvThreads) void gemv_tiled_kernel(GemvArgs a) {
    static_assert(R == 1 || R == 2 || R == 4, "waves per row");
    extern __shared__ float lds[];
    constexpr int U = KV / gcd_c(KV, 32);
    constexpr int S = 32 * U / KV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t per_part = int64_t{1} << a.part_log2;
    float *tab = lds;
    float *xt = lds + per_part * V;
    const int64_t upr = a.wpr / U;          // units per row
    const int upb = a.nwords / U;           // units per block
    for (int64_t j = tid; j < a.xt_len; j += kGemvThreads) {
        const int v = static_cast<int>(j % V);
        const int64_t r = j / V;
        const int l = static_cast<int>(r & 63);
        const int64_t tq = r >> 6;
        const int q = static_cast<int>(tq % S);
        const int64_t u = (tq / S) * 64 + l;
        xt[j] = (u < upr) ? a.x[(u * S + q) * V + v] : 0.0f;
    }
    const int wv = tid >> 6;
    const int rsub = wv & (R - 1);            // this wave's share of its row's tiles
    constexpr int kRowsPerWg = kGemvWaves / R;
    const uint32_t mask = (1u << a.L) - 1u;
    const uint32_t pmask = static_cast<uint32_t>(per_part - 1);
    const int plog = a.part_log2;
    const int64_t step_c = 64 / upb;
    const int step_j = 64 % upb;
    for (int p = 0; p < a.parts; ++p) {
        __syncthreads();  // previous pass finished with the table
        if ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0 && per_part * V >= 4) {
            const float4 *src = reinterpret_cast<const float4 *>(a.C + p * per_part * V);
            float4 *dst = reinterpret_cast<float4 *>(tab);
            for (int64_t i = tid; i < per_part * V / 4; i += kGemvThreads) dst[i] = src[i];
        } else {
            const float *srcf = a.C + p * per_part * V;
            for (int64_t i = tid; i < per_part * V; i += kGemvThreads) tab[i] = srcf[i];
        }
        __syncthreads();
        // the same number of row iterations in every wave of the workgroup (with R > 1
        // there are barriers at the end of each)
        for (int64_t base = static_cast<int64_t>(blockIdx.x) * kRowsPerWg; base < a.M;
             base += static_cast<int64_t>(gridDim.x) * kRowsPerWg) {
            const int64_t row = base + wv / R;
            float acc = 0.0f;
            const int u1 = rsub * 64 + lane;             // this lane's unit in its first tile
            int64_t c = u1 / upb;                        // block of this lane's unit
            int ju = u1 - static_cast<int>(c) * upb;     // unit within the block
            for (int64_t u0 = rsub * 64; row < a.M && u0 < upr; u0 += 64 * R) {
                if (u0 + lane < upr) {
                    const int64_t blk = row * a.bpr + c;
                    const uint32_t *wb = a.bits + blk * a.nwords + ju * U;
                    uint32_t wd[U + 1];
                    wd[0] = ju ? wb[-1] : a.s0[blk];
#pragma unroll
                    for (int i = 0; i < U; ++i) wd[i + 1] = wb[i];
                    const float *xq = xt + (static_cast<int>(u0 >> 6) * S * 64 + lane) * V;
                    // gather this unit's table entries (masked to the part in LDS), then
                    // the products in step order
                    float cv[S][V];
#pragma unroll
                    for (int q = 0; q < S; ++q) {
                        const int e = (q + 1) * KV;          // window end, bits into the unit
                        const int jj = (e - 1) >> 5;         // word holding bit e - 1
                        const uint32_t st =
                            __builtin_amdgcn_alignbit(wd[jj], wd[jj + 1], 32 * (jj + 1) - e) & mask;
#pragma unroll
                        for (int v = 0; v < V; ++v) cv[q][v] = 0.0f;
                        if ((st >> plog) == static_cast<uint32_t>(p)) {
                            const float *cs = tab + (st & pmask) * V;
#pragma unroll
                            for (int v = 0; v < V; ++v) cv[q][v] = cs[v];
                        }
                    }
#pragma unroll
                    for (int q = 0; q < S; ++q) {
#pragma unroll
                        for (int v = 0; v < V; ++v)
                            acc = __builtin_fmaf(cv[q][v], xq[q * 64 * V + v], acc);
                    }
                }
#pragma unroll
                for (int t = 0; t < R; ++t) {  // R tiles on
                    c += step_c;
                    ju += step_j;
                    if (ju >= upb) {
                        ju -= upb;
                        ++c;
                    }
                }
            }
            for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
            if constexpr (R == 1) {
                if (row < a.M && lane == 0) a.y[row] = (p == 0) ? acc : a.y[row] + acc;
            } else {
                // the R wave sums of the row, added in order
                __shared__ float rpart[kGemvWaves];
                if (lane == 0) rpart[wv] = acc;
                __syncthreads();
                if (rsub == 0 && row < a.M && lane == 0) {
                    float t = rpart[wv];
                    for (int q = 1; q < R; ++q) t += rpart[wv + q];
                    a.y[row] = (p == 0) ? t : a.y[row] + t;
                }
                __syncthreads();  // rpart is written again next iteration
            }
        }
    }
}

// Any shape: lane l owns words l, l + 64, ... of the row and decodes every step whose
// chunk ends inside its word (a chunk may straddle two words); x is read from global
// memory.  Codebook parts in LDS as above.
__global__ __launch_bounds__(kGemvThreads) void gemv_generic_kernel(GemvArgs a) {
    extern __shared__ float tab[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int V = a.V;
    const int kv = a.kv;
    const int64_t gwave = static_cast<int64_t>(blockIdx.x) * kGemvWaves + (tid >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kGemvWaves;
    const int64_t per_part = int64_t{1} << a.part_log2;
    const uint32_t mask = (1u << a.L) - 1u;
    const uint32_t pmask = static_cast<uint32_t>(per_part - 1);
    for (int p = 0; p < a.parts; ++p) {
        __syncthreads();
        const float *src = a.C + p * per_part * V;
        for (int64_t i = tid; i < per_part * V; i += kGemvThreads) tab[i] = src[i];
        __syncthreads();
        for (int64_t row = gwave; row < a.M; row += nwaves) {
            float acc = 0.0f;
            int64_t c = lane / a.nwords;
            int jw = lane - static_cast<int>(c) * a.nwords;
            for (int64_t w = lane; w < a.wpr; w += 64) {
                const int64_t blk = row * a.bpr + c;
                const uint32_t *wb = a.bits + blk * a.nwords;
                const uint32_t hi = jw ? wb[jw - 1] : a.s0[blk];
                const uint32_t lo = wb[jw];
                // steps whose chunk ends in bits (32 jw, 32 jw + 32] of the block's stream
                const int t0 = (32 * jw) / kv + 1;
                int t1 = (32 * jw + 32) / kv;
                if (t1 > a.n) t1 = a.n;
                const float *xc = a.x + c * a.T;
                for (int t = t0; t <= t1; ++t) {
                    const uint32_t st =
                        __builtin_amdgcn_alignbit(hi, lo, 32 * jw + 32 - t * kv) & mask;
                    if ((st >> a.part_log2) == static_cast<uint32_t>(p)) {
                        const float *cs = tab + (st & pmask) * V;
                        const float *xv = xc + (t - 1) * V;
                        for (int v = 0; v < V; ++v) acc = __builtin_fmaf(cs[v], xv[v], acc);
                    }
                }
                c += a.step_c;
                jw += a.step_j;
                if (jw >= a.nwords) {
                    jw -= a.nwords;
                    ++c;
                }
            }
            for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) a.y[row] = (p == 0) ? acc : a.y[row] + acc;
        }
    }
}

// Raise a kernel's dynamic LDS limit to the most this file uses, once per kernel (the
// attribute is process-wide, so later launches skip the runtime call).  Calls may come
// from several host threads at once.
hipError_t allow_lds(const void *kern) {
    static std::mutex mu;
    static const void *done[48] = {};  // every kernel of this file
    std::lock_guard<std::mutex> lock(mu);
    for (const void *k : done)
        if (k == kern) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kGemvLdsBytes));
    if (e != hipSuccess) return e;
    for (const void *&k : done)
        if (!k) {
            k = kern;
            break;
        }
    return hipSuccess;
}

// Compute units of the current device (asked on every call: devices of one process, such
// as partitions of one GPU, need not have the same count).
int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return 256;
}

}  // namespace

hipError_t launch_decode_gemv(const uint32_t *bitstream, const uint32_t *start_state,
                              const float *C, const float *x, float *y, int64_t M, int64_t N,
                              int L, int k, int V, int T, hipStream_t s) {
    GemvArgs a{};
    a.bits = bitstream;
    a.s0 = start_state;
    a.C = C;
    a.x = x;
    a.y = y;
    a.M = M;
    a.bpr = N / T;
    a.nwords = (k * T + 31) / 32;
    a.wpr = a.bpr * a.nwords;
    a.L = L;
    a.kv = k * V;
    a.V = V;
    a.n = T / V;
    a.T = T;
    a.step_c = 64 / a.nwords;
    a.step_j = 64 % a.nwords;
    // Tiled kernel when every block is a whole number of units (U words, S steps) and x
    // fits beside a table part.
    const int U = a.kv / gcd_c(a.kv, 32);
    const int64_t S = 32 * U / a.kv;
    const bool whole = a.wpr > 0 && (a.nwords % U == 0) &&
                       (static_cast<int64_t>(a.kv) * a.n == static_cast<int64_t>(a.nwords) * 32);
    const int64_t tiles = (a.wpr / U + 63) / 64;
    a.xt_len = whole ? tiles * 64 * S * V : 0;
    const int64_t xt_bytes = a.xt_len * 4;
    const bool tiled = whole && xt_bytes + kGemvMinPartBytes <= kGemvLdsBytes;
    const int64_t budget = tiled ? kGemvLdsBytes - xt_bytes : kGemvPartBytes;
    // states per part: the largest power of two whose V floats fit in the budget
    int plog = 0;
    while (plog < L && (int64_t{2} << plog) * V * 4 <= budget &&
           (int64_t{2} << plog) * V * 4 <= kGemvPartBytes)
        ++plog;
    a.part_log2 = plog;
    a.parts = 1 << (L - plog);
    const int64_t cus = cu_count();
    // tiled kernel with rows too few to give every CU a workgroup of one-row waves: R
    // waves share a row (at most 4, and no more than a row has tiles of 64 units)
    int rsplit = 1;
    while (rsplit < 4 && (M * rsplit * 2 + kGemvWaves - 1) / kGemvWaves <= cus &&
           rsplit * 2 <= tiles)
        rsplit *= 2;
    const void *kern = reinterpret_cast<const void *>(gemv_generic_kernel);
    if (tiled && (V == 1 || V == 2 || V == 4)) {
#define TCQ_GEMV_CASE(KV_, V_)                                                            \
    if (a.kv == KV_ && V == V_)                                                          \
        kern = rsplit == 4   ? reinterpret_cast<const void *>(gemv_tiled_kernel<KV_, V_, 4>) \
               : rsplit == 2 ? reinterpret_cast<const void *>(gemv_tiled_kernel<KV_, V_, 2>) \
                             : reinterpret_cast<const void *>(gemv_tiled_kernel<KV_, V_, 1>);
        TCQ_GEMV_CASE(1, 1)
        TCQ_GEMV_CASE(2, 1)
        TCQ_GEMV_CASE(2, 2)
        TCQ_GEMV_CASE(3, 1)
        TCQ_GEMV_CASE(4, 1)
        TCQ_GEMV_CASE(4, 2)
        TCQ_GEMV_CASE(4, 4)
        TCQ_GEMV_CASE(6, 2)
        TCQ_GEMV_CASE(8, 1)
        TCQ_GEMV_CASE(8, 2)
        TCQ_GEMV_CASE(8, 4)
#undef TCQ_GEMV_CASE
    }
    if (kern == reinterpret_cast<const void *>(gemv_generic_kernel)) {
        // the generic kernel keeps x in global memory: give the table the whole budget
        plog = 0;
        while (plog < L && (int64_t{2} << plog) * V * 4 <= kGemvPartBytes) ++plog;
        a.part_log2 = plog;
        a.parts = 1 << (L - plog);
    }
    const bool use_xt = kern != reinterpret_cast<const void *>(gemv_generic_kernel);
    if (!use_xt) rsplit = 1;  // the generic kernel has one wave per row
    int64_t grid = cus;
    const int64_t need = (M * rsplit + kGemvWaves - 1) / kGemvWaves;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    const size_t shmem = (size_t{1} << plog) * V * sizeof(float) +
                         (use_xt ? static_cast<size_t>(xt_bytes) : 0);
    hipError_t e = allow_lds(kern);
    if (e != hipSuccess) return e;
    void *args[] = {&a};
    e = hipLaunchKernel(kern, dim3(static_cast<unsigned>(grid)), dim3(kGemvThreads), args,
                        shmem, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace tcq
