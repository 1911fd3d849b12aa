// Pre-processing before coding.
//
// Randomized Hadamard rotation (Pingala-8 post, rotation paragraph and its 4x4 example):
// W x = (W R^T)(R x) for orthogonal R, with R = H_n diag(sigma) / sqrt(n) and H_n the
// Sylvester-ordered Hadamard matrix, H_n[k][i] = (-1)^popcount(k & i).  Rows longer than
// n are rotated in consecutive chunks of n.  Applied to a row x (forward, y = R x):
// sign flip, then the fast Walsh-Hadamard butterflies (a, b) -> (a + b, a - b) over each
// index bit, then the 1/sqrt(n) scale.  Inverse (x = R^T y): butterflies, scale, sign.
//
// Factored row x column scale field (CurveTQ abstract: amplitude carried by a factored
// scale field instead of a rotation): a_r = sqrt(mean_c W_rc^2),
// b_c = sqrt(mean_r (W_rc / a_r)^2), Wn_rc = W_rc / (a_r b_c); an all-zero row or column
// gets scale 1.
#include <hip/hip_runtime.h>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

// One wave per chunk of n = 64 * E values.  Element i = j * 64 + lane sits in register
// j of lane `lane`: index bits 0..5 are lanes (butterflies through cross-lane shuffles),
// bits 6.. are registers (butterflies inside the lane).  Loads and stores are 256-byte
// rows per instruction.
template <int E>
__global__ __launch_bounds__(256) void fwht_wave_kernel(
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
    int64_t rows, int64_t chunks_per_row, const float *__restrict__ sigma, int inverse,
    float scale) {
    constexpr int n = 64 * E;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (chunk >= rows * chunks_per_row) return;
    const int64_t r = chunk / chunks_per_row;
    const int64_t c0 = (chunk % chunks_per_row) * n;
    const float *x = X + r * ldx + c0;
    const float *sg = sigma ? sigma + c0 : nullptr;
    float v[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        v[j] = x[j * 64 + lane];
        if (sg && !inverse) v[j] *= sg[j * 64 + lane];
    }
    // register bits (h = 64, 128, ...)
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if ((j & h) == 0) {
                const float a = v[j];
                const float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    // lane bits (h = 1, ..., 32)
#pragma unroll
    for (int p = 1; p < 64; p <<= 1) {
        const bool upper = (lane & p) != 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float o = __shfl_xor(v[j], p);
            v[j] = upper ? o - v[j] : v[j] + o;
        }
    }
    float *y = Y + r * ldy + c0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        float t = v[j] * scale;
        if (sg && inverse) t *= sg[j * 64 + lane];
        y[j * 64 + lane] = t;
    }
}

// Chunks of n = 256 F values with 16-byte aligned rows: one wave per chunk, element
// i = q + 4 lane + 256 j in component q of float4 register j.  Index bits 0, 1 are
// butterflies inside a float4, bits 2..7 go through cross-lane shuffles, bits 8.. are
// butterflies between registers; each load or store moves 1 KiB per wave.  The levels
// commute, so the order differs from fwht_wave_kernel only in rounding.
template <int F>
__global__ __launch_bounds__(256) void fwht_wave4_kernel(
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
    int64_t rows, int64_t chunks_per_row, const float *__restrict__ sigma, int inverse,
    float scale) {
    constexpr int n = 256 * F;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (chunk >= rows * chunks_per_row) return;
    const int64_t r = chunk / chunks_per_row;
    const int64_t c0 = (chunk % chunks_per_row) * n;
    const float4 *x = reinterpret_cast<const float4 *>(X + r * ldx + c0);
    const float4 *sg = sigma ? reinterpret_cast<const float4 *>(sigma + c0) : nullptr;
    float v[F][4];
#pragma unroll
    for (int j = 0; j < F; ++j) {
        float4 t = x[j * 64 + lane];
        if (sg && !inverse) {
            const float4 g = sg[j * 64 + lane];
            t.x *= g.x;
            t.y *= g.y;
            t.z *= g.z;
            t.w *= g.w;
        }
        v[j][0] = t.x;
        v[j][1] = t.y;
        v[j][2] = t.z;
        v[j][3] = t.w;
    }
    // index bits 0 and 1 (inside the float4)
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const float a0 = v[j][0] + v[j][1], a1 = v[j][0] - v[j][1];
        const float a2 = v[j][2] + v[j][3], a3 = v[j][2] - v[j][3];
        v[j][0] = a0 + a2;
        v[j][2] = a0 - a2;
        v[j][1] = a1 + a3;
        v[j][3] = a1 - a3;
    }
    // index bits 2..7 (lanes)
#pragma unroll
    for (int p = 1; p < 64; p <<= 1) {
        const bool upper = (lane & p) != 0;
#pragma unroll
        for (int j = 0; j < F; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float o = __shfl_xor(v[j][q], p);
                v[j][q] = upper ? o - v[j][q] : v[j][q] + o;
            }
    }
    // index bits 8.. (registers)
#pragma unroll
    for (int h = 1; h < F; h <<= 1)
#pragma unroll
        for (int j = 0; j < F; ++j)
            if ((j & h) == 0)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = v[j][q], b = v[j + h][q];
                    v[j][q] = a + b;
                    v[j + h][q] = a - b;
                }
    float4 *y = reinterpret_cast<float4 *>(Y + r * ldy + c0);
#pragma unroll
    for (int j = 0; j < F; ++j) {
        float4 t = make_float4(v[j][0] * scale, v[j][1] * scale, v[j][2] * scale,
                               v[j][3] * scale);
        if (sg && inverse) {
            const float4 g = sg[j * 64 + lane];
            t.x *= g.x;
            t.y *= g.y;
            t.z *= g.z;
            t.w *= g.w;
        }
        y[j * 64 + lane] = t;
    }
}

// Small chunks (n < 64): one workgroup of 64 threads per row, the row staged in LDS and
// one barrier per butterfly level.
__global__ __launch_bounds__(64) void fwht_small_kernel(
    const float *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy, int64_t len,
    int n, const float *__restrict__ sigma, int inverse, float scale) {
    extern __shared__ float buf[];
    const int64_t r = blockIdx.x;
    const float *x = X + r * ldx;
    for (int64_t i = threadIdx.x; i < len; i += 64) {
        float t = x[i];
        if (sigma && !inverse) t *= sigma[i];
        buf[i] = t;
    }
    __syncthreads();
    for (int h = 1; h < n; h <<= 1) {
        for (int64_t q = threadIdx.x; q < len / 2; q += 64) {
            // q-th pair of this level: low index has bit h clear
            const int64_t lo = (q / h) * 2 * h + (q % h);
            const float a = buf[lo];
            const float b = buf[lo + h];
            buf[lo] = a + b;
            buf[lo + h] = a - b;
        }
        __syncthreads();
    }
    float *y = Y + r * ldy;
    for (int64_t i = threadIdx.x; i < len; i += 64) {
        float t = buf[i] * scale;
        if (sigma && inverse) t *= sigma[i];
        y[i] = t;
    }
}

__global__ __launch_bounds__(256) void row_rms_kernel(const float *__restrict__ W, int64_t ldw,
                                                      int64_t N, float *__restrict__ a) {
    __shared__ float part[4];
    const int64_t r = blockIdx.x;
    const float *w = W + r * ldw;
    float s = 0.0f;
    for (int64_t c = threadIdx.x; c < N; c += 256) s = __builtin_fmaf(w[c], w[c], s);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float tot = ((part[0] + part[1]) + part[2]) + part[3];
        a[r] = tot > 0.0f ? __builtin_sqrtf(tot / static_cast<float>(N)) : 1.0f;
    }
}

// The same with 16-byte loads (N % 4 == 0, 16-byte aligned rows): a lane keeps four
// partial sums, one per component (N/1024 terms each), added pairwise before the tree.
__global__ __launch_bounds__(256) void row_rms4_kernel(const float *__restrict__ W,
                                                       int64_t ldw, int64_t N,
                                                       float *__restrict__ a) {
    __shared__ float part[4];
    const int64_t r = blockIdx.x;
    const float4 *w = reinterpret_cast<const float4 *>(W + r * ldw);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    for (int64_t q = threadIdx.x; q < N / 4; q += 256) {
        const float4 v = w[q];
        s0 = __builtin_fmaf(v.x, v.x, s0);
        s1 = __builtin_fmaf(v.y, v.y, s1);
        s2 = __builtin_fmaf(v.z, v.z, s2);
        s3 = __builtin_fmaf(v.w, v.w, s3);
    }
    float s = (s0 + s1) + (s2 + s3);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float tot = ((part[0] + part[1]) + part[2]) + part[3];
        a[r] = tot > 0.0f ? __builtin_sqrtf(tot / static_cast<float>(N)) : 1.0f;
    }
}

// Column sums of (W_rc / a_r)^2 over row slab blockIdx.y, rows in ascending order.
__global__ __launch_bounds__(256) void col_partial_kernel(
    const float *__restrict__ W, int64_t ldw, int64_t M, int64_t N, int64_t slab_rows,
    const float *__restrict__ a, float *__restrict__ part) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= N) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * slab_rows;
    const int64_t r1 = (r0 + slab_rows < M) ? r0 + slab_rows : M;
    // rows in ascending order; loads of 32 rows are issued before their sums (the walk
    // is a chain of dependent sums, so the loads are what it waits for)
    float s = 0.0f;
    int64_t r = r0;
    for (; r + 32 <= r1; r += 32) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = W[(r + i) * ldw + c] / a[r + i];
#pragma unroll
        for (int i = 0; i < 32; ++i) s = __builtin_fmaf(v[i], v[i], s);
    }
    for (; r < r1; ++r) {
        const float v = W[r * ldw + c] / a[r];
        s = __builtin_fmaf(v, v, s);
    }
    part[static_cast<int64_t>(blockIdx.y) * N + c] = s;
}

__global__ __launch_bounds__(256) void col_finalize_kernel(const float *__restrict__ part,
                                                           int nslabs, int64_t M, int64_t N,
                                                           float *__restrict__ b) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= N) return;
    // slab sums in ascending order; the loads of all (up to 64) slabs are issued before
    // their sums
    float s = 0.0f;
    int i = 0;
    for (; i + 64 <= nslabs; i += 64) {
        float v[64];
#pragma unroll
        for (int q = 0; q < 64; ++q) v[q] = part[static_cast<int64_t>(i + q) * N + c];
#pragma unroll
        for (int q = 0; q < 64; ++q) s += v[q];
    }
    for (; i < nslabs; ++i) s += part[static_cast<int64_t>(i) * N + c];
    b[c] = s > 0.0f ? __builtin_sqrtf(s / static_cast<float>(M)) : 1.0f;
}

__global__ __launch_bounds__(256) void scale_apply_kernel(
    const float *__restrict__ W, int64_t ldw, int64_t N, const float *__restrict__ a,
    const float *__restrict__ b, float *__restrict__ Wn, int64_t ldn) {
    const int64_t r = blockIdx.x;
    const float ar = a[r];
    for (int64_t c = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x; c < N;
         c += static_cast<int64_t>(gridDim.y) * 256)
        Wn[r * ldn + c] = W[r * ldw + c] / (ar * b[c]);
}

// The same with 16-byte accesses (N % 4 == 0, 16-byte aligned rows and b); the
// arithmetic per element is unchanged.
__global__ __launch_bounds__(256) void scale_apply4_kernel(
    const float *__restrict__ W, int64_t ldw, int64_t N, const float *__restrict__ a,
    const float *__restrict__ b, float *__restrict__ Wn, int64_t ldn) {
    const int64_t r = blockIdx.x;
    const float ar = a[r];
    const float4 *w = reinterpret_cast<const float4 *>(W + r * ldw);
    const float4 *b4 = reinterpret_cast<const float4 *>(b);
    float4 *o = reinterpret_cast<float4 *>(Wn + r * ldn);
    for (int64_t q = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x; q < N / 4;
         q += static_cast<int64_t>(gridDim.y) * 256) {
        const float4 v = w[q];
        const float4 bc = b4[q];
        o[q] = make_float4(v.x / (ar * bc.x), v.y / (ar * bc.y), v.z / (ar * bc.z),
                           v.w / (ar * bc.w));
    }
}

template <int F>
hipError_t launch_wave4(const float *X, int64_t ldx, float *Y, int64_t ldy, int64_t rows,
                        int64_t cpr, const float *sigma, int inverse, float scale,
                        hipStream_t s) {
    const int64_t chunks = rows * cpr;
    const int64_t grid = (chunks + 3) / 4;
    hipLaunchKernelGGL(fwht_wave4_kernel<F>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       s, X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale);
    return hipGetLastError();
}

template <int E>
hipError_t launch_wave(const float *X, int64_t ldx, float *Y, int64_t ldy, int64_t rows,
                       int64_t cpr, const float *sigma, int inverse, float scale,
                       hipStream_t s) {
    const int64_t chunks = rows * cpr;
    const int64_t grid = (chunks + 3) / 4;
    hipLaunchKernelGGL(fwht_wave_kernel<E>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                       X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale);
    return hipGetLastError();
}

}  // namespace

size_t scale_field_slabs(int64_t M) { return static_cast<size_t>(M < 64 ? (M > 0 ? M : 1) : 64); }

hipError_t launch_hadamard(const float *X, int64_t ldx, float *Y, int64_t ldy, int64_t rows,
                           int64_t len, int64_t n, const float *sigma, int inverse,
                           hipStream_t s) {
    const float scale = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(n)));
    const int64_t cpr = len / n;
    // 16-byte rows (and signs): float4 loads and stores
    const bool a16 = ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y) |
                       reinterpret_cast<uintptr_t>(sigma)) & 15u) == 0 &&
                     ldx % 4 == 0 && ldy % 4 == 0;
    if (a16) {
        switch (n) {
            case 256: return launch_wave4<1>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
            case 512: return launch_wave4<2>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
            case 1024: return launch_wave4<4>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
            case 2048: return launch_wave4<8>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
            case 4096: return launch_wave4<16>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
            default: break;
        }
    }
    switch (n) {
        case 64: return launch_wave<1>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 128: return launch_wave<2>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 256: return launch_wave<4>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 512: return launch_wave<8>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 1024: return launch_wave<16>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 2048: return launch_wave<32>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        case 4096: return launch_wave<64>(X, ldx, Y, ldy, rows, cpr, sigma, inverse, scale, s);
        default: break;
    }
    // n < 64: whole row in LDS (len <= kHadamardSmallMaxLen)
    const size_t shmem = static_cast<size_t>(len) * sizeof(float);
    hipLaunchKernelGGL(fwht_small_kernel, dim3(static_cast<unsigned>(rows)), dim3(64), shmem, s,
                       X, ldx, Y, ldy, len, static_cast<int>(n), sigma, inverse, scale);
    return hipGetLastError();
}

hipError_t launch_scale_field(const float *W, int64_t ldw, int64_t M, int64_t N, float *a,
                              float *b, float *Wn, int64_t ldn, float *part, hipStream_t s) {
    // 16-byte accesses where every row (and b) is 16-byte aligned
    const bool v4 = N % 4 == 0 && ldw % 4 == 0 &&
                    (reinterpret_cast<uintptr_t>(W) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(b) & 15u) == 0 &&
                    (!Wn || (ldn % 4 == 0 && (reinterpret_cast<uintptr_t>(Wn) & 15u) == 0));
    if (v4)
        hipLaunchKernelGGL(row_rms4_kernel, dim3(static_cast<unsigned>(M)), dim3(256), 0, s, W,
                           ldw, N, a);
    else
        hipLaunchKernelGGL(row_rms_kernel, dim3(static_cast<unsigned>(M)), dim3(256), 0, s, W,
                           ldw, N, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nslabs = static_cast<int64_t>(scale_field_slabs(M));
    const int64_t slab_rows = (M + nslabs - 1) / nslabs;
    const int64_t cb = (N + 255) / 256;
    hipLaunchKernelGGL(col_partial_kernel, dim3(static_cast<unsigned>(cb),
                       static_cast<unsigned>(nslabs)), dim3(256), 0, s, W, ldw, M, N, slab_rows,
                       a, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(col_finalize_kernel, dim3(static_cast<unsigned>(cb)), dim3(256), 0, s,
                       part, static_cast<int>(nslabs), M, N, b);
    e = hipGetLastError();
    if (e != hipSuccess || !Wn) return e;
    if (v4) {
        const int64_t cb4 = (N / 4 + 255) / 256;
        const int64_t gy4 = cb4 < 16 ? cb4 : 16;
        hipLaunchKernelGGL(scale_apply4_kernel, dim3(static_cast<unsigned>(M),
                           static_cast<unsigned>(gy4)), dim3(256), 0, s, W, ldw, N, a, b, Wn,
                           ldn);
        return hipGetLastError();
    }
    const int64_t gy = cb < 16 ? cb : 16;
    hipLaunchKernelGGL(scale_apply_kernel, dim3(static_cast<unsigned>(M),
                       static_cast<unsigned>(gy)), dim3(256), 0, s, W, ldw, N, a, b, Wn, ldn);
    return hipGetLastError();
}

}  // namespace tcq
