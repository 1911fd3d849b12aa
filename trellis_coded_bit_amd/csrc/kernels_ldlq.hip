// Error feedback over coding blocks (LDLQ).  Pingala-8 post, error-feedback toy and LDLQ
// paragraph: columns are quantized in order and each one's error moves onto the columns
// not yet quantized, weighted through H.  With H = U D U^T (U unit upper
// block-triangular over blocks of T columns, D block diagonal), column c of block j is
// coded against
//     t_c = w_c + sum_{i < jT} fl(w_i - what_i) * U[i][c],
// accumulated in fp32 as acc = w_c, then acc = fmaf(fl(w_i - what_i), U[i][c], acc) for
// i = 0, 1, ..., jT - 1 in ascending order.  The driver applies the terms of block j to
// every later column right after block j is coded, in that same order, so each target
// sees exactly that chain of fmaf.
#include <hip/hip_runtime.h>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

constexpr int kTile = 64;   // rows and columns of targets per workgroup
constexpr int kChunk = 16;  // feedback terms staged in LDS at a time

// tgt[r][c] += sum over i of E[r][i] * U[i][c] for rows [0, M), columns
// [c_begin, c_end), and i over the T columns [i0, i0 + T) of the block just coded.
// 256 threads; thread (ty, tx) owns rows ty + 16a and columns tx + 16b (a, b < 4), so
// every target's fmaf chain runs over i in ascending order inside one thread.
__global__ __launch_bounds__(256) void ldlq_update_kernel(
    float *__restrict__ tgt, int64_t ldt, const float *__restrict__ W, int64_t ldw,
    const float *__restrict__ what, int64_t ldh, const float *__restrict__ U, int64_t ldu,
    int64_t M, int64_t c_begin, int64_t c_end, int64_t i0, int T) {
    __shared__ float Es[kChunk][kTile + 1];
    __shared__ float Us[kChunk][kTile];
    const int tid = threadIdx.x;
    const int tx = tid & 15;
    const int ty = tid >> 4;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTile;
    const int64_t c0 = c_begin + static_cast<int64_t>(blockIdx.x) * kTile;

    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t r = r0 + ty + 16 * a;
            const int64_t c = c0 + tx + 16 * b;
            acc[a][b] = (r < M && c < c_end) ? tgt[r * ldt + c] : 0.0f;
        }
    }
    // The next chunk's W, what and U values are requested into registers before the
    // current chunk is computed, so the global-memory latency overlaps the fmaf work.
    float pw[4], ph[4], pu[4];
    auto fetch = [&](int ib) {
        const int nk = (T - ib < kChunk) ? T - ib : kChunk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // E tile: 64 rows x 16 terms, read along a row (contiguous in i)
            const int idx = tid + 256 * q;
            const int rr = idx >> 4;
            const int ii = idx & 15;
            const int64_t r = r0 + rr;
            pw[q] = 0.0f;
            ph[q] = 0.0f;
            if (r < M && ii < nk) {
                pw[q] = W[r * ldw + i0 + ib + ii];
                ph[q] = what[r * ldh + (ib + ii)];
            }
            // U tile: 16 terms x 64 columns, read along a row of U (contiguous in c)
            const int ui = idx >> 6;
            const int cc = idx & 63;
            const int64_t c = c0 + cc;
            pu[q] = (ui < nk && c < c_end) ? U[(i0 + ib + ui) * ldu + c] : 0.0f;
        }
    };
    fetch(0);
    for (int ib = 0; ib < T; ib += kChunk) {
        const int nk = (T - ib < kChunk) ? T - ib : kChunk;
        __syncthreads();  // every thread is done with the previous chunk
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = tid + 256 * q;
            Es[idx & 15][idx >> 4] = pw[q] - ph[q];  // zero outside the tile (0 - 0)
            Us[idx >> 6][idx & 63] = pu[q];
        }
        __syncthreads();
        if (ib + kChunk < T) fetch(ib + kChunk);
        for (int ii = 0; ii < nk; ++ii) {
            float e[4], u[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) e[a] = Es[ii][ty + 16 * a];
#pragma unroll
            for (int b = 0; b < 4; ++b) u[b] = Us[ii][tx + 16 * b];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(e[a], u[b], acc[a][b]);
            }
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t r = r0 + ty + 16 * a;
            const int64_t c = c0 + tx + 16 * b;
            if (r < M && c < c_end) tgt[r * ldt + c] = acc[a][b];
        }
    }
}

// Slice outputs (one block per row, block r) -> the matrix layout (block r*nbpr + j).
__global__ __launch_bounds__(64) void ldlq_scatter_kernel(
    const uint32_t *__restrict__ sbits, const uint32_t *__restrict__ sstart,
    const float *__restrict__ scost, int64_t M, int nwords, int64_t nbpr, int64_t j,
    uint32_t *__restrict__ bitstream, uint32_t *__restrict__ start_state,
    float *__restrict__ cost) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
    if (r >= M) return;
    const int64_t b = r * nbpr + j;
    for (int w = 0; w < nwords; ++w) bitstream[b * nwords + w] = sbits[r * nwords + w];
    start_state[b] = sstart[r];
    cost[b] = scost[r];
}

}  // namespace

hipError_t launch_ldlq_update(float *tgt, int64_t ldt, const float *W, int64_t ldw,
                              const float *what, int64_t ldh, const float *U, int64_t ldu,
                              int64_t M, int64_t c_begin, int64_t c_end, int64_t i0, int T,
                              hipStream_t s) {
    const int64_t ct = (c_end - c_begin + kTile - 1) / kTile;
    const int64_t rt = (M + kTile - 1) / kTile;
    if (ct <= 0 || rt <= 0) return hipSuccess;
    hipLaunchKernelGGL(ldlq_update_kernel, dim3(static_cast<unsigned>(ct),
                       static_cast<unsigned>(rt)), dim3(256), 0, s, tgt, ldt, W, ldw, what,
                       ldh, U, ldu, M, c_begin, c_end, i0, T);
    return hipGetLastError();
}

hipError_t launch_ldlq_scatter(const uint32_t *sbits, const uint32_t *sstart,
                               const float *scost, int64_t M, int nwords, int64_t nbpr,
                               int64_t j, uint32_t *bitstream, uint32_t *start_state,
                               float *cost, hipStream_t s) {
    const int64_t g = (M + 63) / 64;
    hipLaunchKernelGGL(ldlq_scatter_kernel, dim3(static_cast<unsigned>(g)), dim3(64), 0, s,
                       sbits, sstart, scost, M, nwords, nbpr, j, bitstream, start_state, cost);
    return hipGetLastError();
}

}  // namespace tcq
