// Soft trellis (BCJR) at temperature tau.  BCJR-QAT abstract (aqora listing): a tempered
// forward-backward pass stands in for the hard minimum of the Viterbi search; each output
// is the mean emitted value when paths are weighted by exp(-J/tau), and as tau falls to 0
// the output returns to the Viterbi reconstruction.
//
// Energy of a path = the weighted squared error the Viterbi search minimises; probability
// of a path = exp(-J/tau) / Z.  Work is in base-2 logs: the log-weight of state s at a
// step is g(s) = sum_v d_v * e_v^2 * ns with e_v = w_v - C[s][v] and ns = -log2(e)/tau,
// added to the incoming vector value in fp32 as one fma per coordinate.
//
// Group form used here (x = a group of 2^kv states that share predecessors):
//  - forward:  F_t(x) = LSE_j [g_t(s_j) + F_{t-1}(s_j >> kv)], s_j = (j << (L-kv)) | x,
//              F_0 = 0; then alpha_t(s') = g_t(s') + F_{t-1}(s' >> kv), and
//              log2 Z = LSE_x F_n(x).
//  - backward: the successors of s depend only on x = s mod 2^(L-kv), so
//              beta_t(s) = B_t(s mod 2^(L-kv)) with B_n = 0 and
//              B_{t-1}(x) = LSE_b [g_t(s'_b) + B_t(s'_b mod 2^(L-kv))], s'_b = (x << kv) | b.
//  - marginal: P(s_t = s'_b) is proportional to 2^(g_t(s'_b) + B_t(..) + F_{t-1}(x)),
//              i.e. a softmax over b inside the group times a group weight.
// Only vectors of 2^(L-kv) values are carried (in LDS when they fit).  F_{t-1} is kept
// in the workspace for the backward pass.  Each step's vector is shifted by the previous
// step's maximum so values stay near 0; a per-step constant cancels in the marginals,
// and the forward shifts are summed (in double) for log Z.
#include <hip/hip_runtime.h>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / 64;
constexpr float kNegInf = -__builtin_inff();

struct BcjrArgs {
    const float *W;
    int64_t ldw;
    const float *d;
    const float *C;
    int L, kv, V, n;
    int64_t blocks_per_row, block0;
    float ns;              // -log2(e) / tau
    float *fstore;         // [block][t][x], t < n
    int64_t fstore_per_block;
    float *gbuf;           // 2 * 2^(L-kv) floats per block when the vectors are not in LDS
    int64_t gbuf_per_block;
    float *soft;
    int64_t ldo;
    float *logz;
};

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

// base + g(s) in base-2 log units: g(s) = sum_v d_v * (w_v - c_v)^2 * ns, evaluated as
// the chain acc = base, acc = fmaf(fl(e_v * e_v), dn_v, acc) over v, dn_v = fl(d_v * ns).
__device__ __forceinline__ float add_log_weight(float base, const float *wv, const float *dn,
                                                const float *c, int V) {
    float acc = base;
    for (int v = 0; v < V; ++v) {
        const float e = wv[v] - c[v];
        acc = __builtin_fmaf(e * e, dn[v], acc);
    }
    return acc;
}

// (m, s) stands for m + log2(s); merge two such pairs.
__device__ __forceinline__ void lse_merge(float &m, float &s, float om, float os) {
    const float nm = fmaxf(m, om);
    if (nm == kNegInf) return;
    s = s * exp2_(m - nm) + os * exp2_(om - nm);
    m = nm;
}

// Weighted expectation accumulator: (u, num[], den) stands for the pair
// (2^u * num, 2^u * den).
struct Expect {
    float u;
    float num[TCQ_MAX_V];
    float den;
};

__device__ __forceinline__ void expect_merge(Expect &a, float ou, const float *onum, float oden,
                                             int V) {
    const float nm = fmaxf(a.u, ou);
    if (nm == kNegInf) return;
    const float sa = (a.u == kNegInf) ? 0.0f : exp2_(a.u - nm);
    const float sb = (ou == kNegInf) ? 0.0f : exp2_(ou - nm);
    for (int v = 0; v < V; ++v) a.num[v] = a.num[v] * sa + onum[v] * sb;
    a.den = a.den * sa + oden * sb;
    a.u = nm;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Threads per workgroup: 1024 for up to 4 terms per group, 512 above (more registers).
constexpr int max_threads(int kv) { return kv <= 2 ? kMaxThreads : kMaxThreads / 2; }

// G = 2^KV predecessors/successors per group, held in registers (KV <= 4).
template <int KV, bool IN_LDS>
__global__ __launch_bounds__(max_threads(KV)) void bcjr_kernel(BcjrArgs a) {
    extern __shared__ float lds[];
    __shared__ float part_max[2][kMaxWaves];
    __shared__ float part_m[kMaxWaves], part_s[kMaxWaves];
    __shared__ float part_u[2][kMaxWaves];
    __shared__ float part_num[2][kMaxWaves][TCQ_MAX_V];
    __shared__ float part_den[2][kMaxWaves];

    constexpr int G = 1 << KV;
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = nt >> 6;
    const int L = a.L;
    const int V = a.V;
    const int n = a.n;
    const int64_t X = int64_t{1} << (L - KV);
    const int sh = L - KV;
    const int64_t blk = a.block0 + blockIdx.x;
    const int64_t row = blk / a.blocks_per_row;
    const int64_t col = blk % a.blocks_per_row;
    const int T = n * V;
    const float *w = a.W + row * a.ldw + col * T;
    const float *dd = a.d ? a.d + col * T : nullptr;
    const bool weighted = a.d != nullptr;
    float *fst = a.fstore + static_cast<int64_t>(blockIdx.x) * a.fstore_per_block;
    float *bufA = IN_LDS ? lds : a.gbuf + static_cast<int64_t>(blockIdx.x) * a.gbuf_per_block;
    float *bufB = bufA + X;
    const float ns = a.ns;

    for (int64_t x = tid; x < X; x += nt) {
        bufA[x] = 0.0f;
        fst[x] = 0.0f;  // F_0
    }
    __syncthreads();

    // ---------------- forward ----------------
    float *Fc = bufA;
    float *Fn = bufB;
    double offset = 0.0;  // sum of the shifts, base-2 log
    float wv[TCQ_MAX_V], dn[TCQ_MAX_V];
    for (int t = 1; t <= n; ++t) {
        float c = 0.0f;
        if (t >= 2) {
            c = part_max[(t - 1) & 1][0];
            for (int i = 1; i < nwaves; ++i) c = fmaxf(c, part_max[(t - 1) & 1][i]);
            offset += static_cast<double>(c);
        }
        for (int v = 0; v < V; ++v) {
            wv[v] = w[(t - 1) * V + v];
            dn[v] = (weighted ? dd[(t - 1) * V + v] : 1.0f) * ns;
        }
        float lmax = kNegInf;
        for (int64_t x = tid; x < X; x += nt) {
            float val[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int64_t s = (static_cast<int64_t>(j) << sh) | x;
                val[j] = add_log_weight(Fc[s >> KV], wv, dn, a.C + s * V, V);
            }
            float mx = val[0];
#pragma unroll
            for (int j = 1; j < G; ++j) mx = fmaxf(mx, val[j]);
            float sum = exp2_(val[0] - mx);
#pragma unroll
            for (int j = 1; j < G; ++j) sum += exp2_(val[j] - mx);
            const float f = mx + log2_(sum) - c;
            Fn[x] = f;
            if (t < n) fst[static_cast<int64_t>(t) * X + x] = f;
            lmax = fmaxf(lmax, f);
        }
        lmax = wave_max(lmax);
        if (lane == 0) part_max[t & 1][wave] = lmax;
        __syncthreads();
        float *tmp = Fc;
        Fc = Fn;
        Fn = tmp;
    }
    // log2 Z = LSE_x F_n(x) + offset
    {
        float m = kNegInf, s = 0.0f;
        for (int64_t x = tid; x < X; x += nt) lse_merge(m, s, Fc[x], 1.0f);
        for (int off = 32; off >= 1; off >>= 1) {
            const float om = __shfl_xor(m, off);
            const float os = __shfl_xor(s, off);
            lse_merge(m, s, om, os);
        }
        if (lane == 0) {
            part_m[wave] = m;
            part_s[wave] = s;
        }
        __syncthreads();
        if (tid == 0 && a.logz) {
            float fm = part_m[0], fs = part_s[0];
            for (int i = 1; i < nwaves; ++i) lse_merge(fm, fs, part_m[i], part_s[i]);
            const double l2 = static_cast<double>(fm) + static_cast<double>(log2_(fs)) + offset;
            a.logz[blk] = static_cast<float>(l2 * 0.69314718055994530942);
        }
    }
    __threadfence();
    __syncthreads();

    // ---------------- backward ----------------
    float *Bc = bufA;
    float *Bn = bufB;
    for (int64_t x = tid; x < X; x += nt) Bc[x] = 0.0f;
    __syncthreads();
    const int64_t lowmask = X - 1;
    float *out = a.soft + row * a.ldo + col * T;
    for (int t = n; t >= 1; --t) {
        float c = 0.0f;
        if (t < n) {
            c = part_max[(t + 1) & 1][0];
            for (int i = 1; i < nwaves; ++i) c = fmaxf(c, part_max[(t + 1) & 1][i]);
        }
        for (int v = 0; v < V; ++v) {
            wv[v] = w[(t - 1) * V + v];
            dn[v] = (weighted ? dd[(t - 1) * V + v] : 1.0f) * ns;
        }
        Expect ex;
        ex.u = kNegInf;
        for (int v = 0; v < TCQ_MAX_V; ++v) ex.num[v] = 0.0f;
        ex.den = 0.0f;
        float lmax = kNegInf;
        for (int64_t x = tid; x < X; x += nt) {
            const float fx = fst[static_cast<int64_t>(t - 1) * X + x];
            float val[G];
#pragma unroll
            for (int b = 0; b < G; ++b) {
                const int64_t s2 = (x << KV) | b;
                val[b] = add_log_weight(Bc[s2 & lowmask], wv, dn, a.C + s2 * V, V);
            }
            float mx = val[0];
#pragma unroll
            for (int b = 1; b < G; ++b) mx = fmaxf(mx, val[b]);
            float sum = 0.0f;
            float gnum[TCQ_MAX_V];
            for (int v = 0; v < V; ++v) gnum[v] = 0.0f;
#pragma unroll
            for (int b = 0; b < G; ++b) {
                const float e = exp2_(val[b] - mx);
                sum += e;
                const float *cs = a.C + ((x << KV) | b) * V;
                for (int v = 0; v < V; ++v) gnum[v] = __builtin_fmaf(e, cs[v], gnum[v]);
            }
            if (t > 1) {
                const float bnew = mx + log2_(sum) - c;
                Bn[x] = bnew;
                lmax = fmaxf(lmax, bnew);
            }
            expect_merge(ex, mx + fx, gnum, sum, V);
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const float ou = __shfl_xor(ex.u, off);
            float onum[TCQ_MAX_V];
            for (int v = 0; v < V; ++v) onum[v] = __shfl_xor(ex.num[v], off);
            const float oden = __shfl_xor(ex.den, off);
            expect_merge(ex, ou, onum, oden, V);
        }
        lmax = wave_max(lmax);
        if (lane == 0) {
            part_max[t & 1][wave] = lmax;
            part_u[t & 1][wave] = ex.u;
            for (int v = 0; v < V; ++v) part_num[t & 1][wave][v] = ex.num[v];
            part_den[t & 1][wave] = ex.den;
        }
        __syncthreads();
        if (tid == 0) {
            Expect tot;
            tot.u = part_u[t & 1][0];
            for (int v = 0; v < V; ++v) tot.num[v] = part_num[t & 1][0][v];
            tot.den = part_den[t & 1][0];
            for (int i = 1; i < nwaves; ++i)
                expect_merge(tot, part_u[t & 1][i], part_num[t & 1][i], part_den[t & 1][i], V);
            for (int v = 0; v < V; ++v) out[(t - 1) * V + v] = tot.num[v] / tot.den;
        }
        float *tmp = Bc;
        Bc = Bn;
        Bn = tmp;
    }
}

// Register-codebook variant for L = 16, V = 1, kv = 2 or 3.  Thread tid owns the y values
// y_i = tid + NT i (i < NY), and with them the states
//     s = (j << (L - kv)) | (y << kv) | b,   j, b < 2^kv.
// In the forward pass these are the predecessors of its groups x = (y << kv) | b; in the
// backward pass they are the successors of its groups x' = (j << (L - 2 kv)) | y.  So the
// thread's codebook values never change and stay in registers for the whole block, and
// the G forward values F(s >> kv) (or backward values B(s mod 2^(L-kv))) that a y needs
// are read from LDS once and shared by its G groups.  LDS vectors are padded by one
// float every 32 to spread the strided accesses over the banks.  With L fixed, every LDS
// and workspace index is a per-lane base plus a compile-time offset.
__host__ __device__ constexpr int pad(int i) { return i + (i >> 5); }
// y values per thread that fit in registers (NY G^2 codebook floats)
constexpr int reg_max_ny(int kv) { return kv == 2 ? 8 : 2; }

template <int KV, int NT>
__global__ __launch_bounds__(NT) void bcjr_reg_kernel(BcjrArgs a) {
    extern __shared__ float lds[];
    // the block's weights and d, read through LDS so that no per-step vector-memory
    // wait drains the workspace loads in flight
    __shared__ float wsh[TCQ_MAX_STEPS], dsh[TCQ_MAX_STEPS];
    __shared__ float part_max[2][kMaxWaves];
    __shared__ float part_m[kMaxWaves], part_s[kMaxWaves];
    __shared__ float part_u[2][kMaxWaves];
    __shared__ float part_num[2][kMaxWaves];
    __shared__ float part_den[2][kMaxWaves];

    constexpr int L = 16;
    constexpr int G = 1 << KV;
    constexpr int nwaves = NT / 64;
    constexpr int X = 1 << (L - KV);  // groups per step
    constexpr int shF = L - KV;       // j position in a state
    constexpr int shY = L - 2 * KV;   // j position in a backward group
    constexpr int NY = (1 << shY) / NT;
    constexpr int PX = pad(X);        // padded vector length
    static_assert(NY >= 1 && NY * NT == (1 << shY) && NY <= reg_max_ny(KV), "y split");
    static_assert(NT % 32 == 0 && shY >= 5, "padding splits into base + offset");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = a.n;
    const int64_t blk = a.block0 + blockIdx.x;
    const int64_t row = blk / a.blocks_per_row;
    const int64_t col = blk % a.blocks_per_row;
    const float *w = a.W + row * a.ldw + col * n;
    const float *dd = a.d ? a.d + col * n : nullptr;
    const bool weighted = a.d != nullptr;
    float *fst = a.fstore + static_cast<int64_t>(blockIdx.x) * a.fstore_per_block;
    float *bufA = lds;
    float *bufB = lds + PX;
    const float ns = a.ns;
    // per-lane parts of the padded indices: pad(A + B) = pad(A) + pad(B) when A is a
    // multiple of 32
    const int pT = pad(tid);       // y_i = tid + NT i, groups (j << shY) | y_i
    const int pG = pad(tid << KV); // groups (y_i << KV) | b: pad(.) = pG + b + const

    float creg[NY][G][G];
#pragma unroll
    for (int i = 0; i < NY; ++i) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float *src = a.C + ((j << shF) | ((tid + NT * i) << KV));
#pragma unroll
            for (int b = 0; b < G; ++b) creg[i][j][b] = src[b];
        }
    }
    for (int x = tid; x < X; x += NT) {
        bufA[pad(x)] = 0.0f;
        fst[x] = 0.0f;  // F_0
    }
    for (int t = tid; t < n; t += NT) {
        wsh[t] = w[t];
        dsh[t] = (weighted ? dd[t] : 1.0f) * ns;
    }
    __syncthreads();

    // ---------------- forward ----------------
    float *Fc = bufA;
    float *Fn = bufB;
    double offset = 0.0;
    for (int t = 1; t <= n; ++t) {
        float c = 0.0f;
        if (t >= 2) {
            c = part_max[(t - 1) & 1][0];
            for (int i = 1; i < nwaves; ++i) c = fmaxf(c, part_max[(t - 1) & 1][i]);
            offset += static_cast<double>(c);
        }
        const float wt = wsh[t - 1];
        const float dn = dsh[t - 1];
        float4 *frow = reinterpret_cast<float4 *>(fst + static_cast<int64_t>(t) * X);
        float lmax = kNegInf;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            float fj[G];
#pragma unroll
            for (int j = 0; j < G; ++j) fj[j] = Fc[pT + pad(NT * i) + pad(j << shY)];
            float fo[G];
#pragma unroll
            for (int b = 0; b < G; ++b) {
                float val[G];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const float e = wt - creg[i][j][b];
                    val[j] = __builtin_fmaf(e * e, dn, fj[j]);
                }
                float mx = val[0];
#pragma unroll
                for (int j = 1; j < G; ++j) mx = fmaxf(mx, val[j]);
                float sum = exp2_(val[0] - mx);
#pragma unroll
                for (int j = 1; j < G; ++j) sum += exp2_(val[j] - mx);
                fo[b] = mx + log2_(sum) - c;
                lmax = fmaxf(lmax, fo[b]);
            }
#pragma unroll
            for (int b = 0; b < G; ++b) Fn[pG + b + pad((NT * i) << KV)] = fo[b];
            if (t < n) {
                // groups ((tid + NT i) << KV) + b, b < G: G / 4 float4 per thread
#pragma unroll
                for (int q = 0; q < G / 4; ++q)
                    frow[((NT * i) << KV) / 4 + tid * (G / 4) + q] =
                        make_float4(fo[4 * q], fo[4 * q + 1], fo[4 * q + 2], fo[4 * q + 3]);
            }
        }
        lmax = wave_max(lmax);
        if (lane == 0) part_max[t & 1][wave] = lmax;
        __syncthreads();
        float *tmp = Fc;
        Fc = Fn;
        Fn = tmp;
    }
    {
        float m = kNegInf, s2 = 0.0f;
        for (int x = tid; x < X; x += NT) lse_merge(m, s2, Fc[pad(x)], 1.0f);
        for (int off = 32; off >= 1; off >>= 1) {
            const float om = __shfl_xor(m, off);
            const float os = __shfl_xor(s2, off);
            lse_merge(m, s2, om, os);
        }
        if (lane == 0) {
            part_m[wave] = m;
            part_s[wave] = s2;
        }
        __syncthreads();
        if (tid == 0 && a.logz) {
            float fm = part_m[0], fs = part_s[0];
            for (int i = 1; i < nwaves; ++i) lse_merge(fm, fs, part_m[i], part_s[i]);
            const double l2 = static_cast<double>(fm) + static_cast<double>(log2_(fs)) + offset;
            a.logz[blk] = static_cast<float>(l2 * 0.69314718055994530942);
        }
    }
    __threadfence();
    __syncthreads();

    // ---------------- backward ----------------
    float *Bc = bufA;
    float *Bn = bufB;
    for (int x = tid; x < X; x += NT) Bc[pad(x)] = 0.0f;
    // F_{t-1} at the thread's backward groups (j << shY) | y_i, consumed in the order
    // p = G i + j (NP per step) and requested kRing positions ahead of use, across the
    // step boundary (the last step requests row 0 again; those values go unused)
    constexpr int NP = NY * G;
    constexpr int kRing = NP / 2;
    // raw buffer loads over the block's n rows: one per-lane offset (4 * tid) for every
    // load, the row and position in the scalar offset
    const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(
        fst, 0, n * X * static_cast<int>(sizeof(float)), 0x00020000);
    const int voff = tid * static_cast<int>(sizeof(float));
    auto fload = [&](int r, int q) {
        const int soff = (r * X + ((q % G) << shY) + NT * (q / G)) * static_cast<int>(sizeof(float));
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(frs, voff, soff, 0));
    };
    float ring[kRing];
#pragma unroll
    for (int p = 0; p < kRing; ++p) ring[p] = fload(n - 1, p);
    __syncthreads();
    float *out = a.soft + row * a.ldo + col * n;
    for (int t = n; t >= 1; --t) {
        float c = 0.0f;
        if (t < n) {
            c = part_max[(t + 1) & 1][0];
            for (int i = 1; i < nwaves; ++i) c = fmaxf(c, part_max[(t + 1) & 1][i]);
        }
        const float wt = wsh[t - 1];
        const float dn = dsh[t - 1];
        const int nrow = t >= 2 ? t - 2 : 0;
        // (eu, enum_, eden) stands for (2^eu enum_, 2^eu eden); every term is finite, so
        // the first y initialises it and later ones merge into it
        float eu = 0.0f, enum_ = 0.0f, eden = 0.0f;
        float lmax = kNegInf;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            float bb[G];
#pragma unroll
            for (int b = 0; b < G; ++b) bb[b] = Bc[pG + b + pad((NT * i) << KV)];
            float gu[G], gs[G], gn[G];  // per group: log2 weight, softmax sum, numerator
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float val[G];
#pragma unroll
                for (int b = 0; b < G; ++b) {
                    const float e = wt - creg[i][j][b];
                    val[b] = __builtin_fmaf(e * e, dn, bb[b]);
                }
                float mx = val[0];
#pragma unroll
                for (int b = 1; b < G; ++b) mx = fmaxf(mx, val[b]);
                float sum = exp2_(val[0] - mx);
                float gnum = sum * creg[i][j][0];
#pragma unroll
                for (int b = 1; b < G; ++b) {
                    const float e = exp2_(val[b] - mx);
                    sum += e;
                    gnum = __builtin_fmaf(e, creg[i][j][b], gnum);
                }
                // B_{t-1}; on the last step (t = 1) it lands in the unused buffer
                const float bnew = mx + log2_(sum) - c;
                Bn[pT + pad(NT * i) + pad(j << shY)] = bnew;
                lmax = fmaxf(lmax, bnew);
                const int pos = G * i + j;
                gu[j] = mx + ring[pos % kRing];
                {
                    const int q = pos + kRing;  // position requested now
                    // keep the request here: the scheduler would otherwise sink it towards
                    // its use and shorten the distance the ring is meant to cover
                    __builtin_amdgcn_sched_barrier(0);
                    ring[pos % kRing] = q < NP ? fload(t - 1, q) : fload(nrow, q - NP);
                }
                gs[j] = sum;
                gn[j] = gnum;
            }
            // the G groups of this y against their own maximum, then into the running sum
            float lu = gu[0];
#pragma unroll
            for (int j = 1; j < G; ++j) lu = fmaxf(lu, gu[j]);
            float sc = exp2_(gu[0] - lu);
            float ln = gn[0] * sc, ld = gs[0] * sc;
#pragma unroll
            for (int j = 1; j < G; ++j) {
                sc = exp2_(gu[j] - lu);
                ln = __builtin_fmaf(gn[j], sc, ln);
                ld = __builtin_fmaf(gs[j], sc, ld);
            }
            if (i == 0) {
                eu = lu;
                enum_ = ln;
                eden = ld;
            } else {
                const float nm = fmaxf(eu, lu);
                const float sa = exp2_(eu - nm);
                const float sb = exp2_(lu - nm);
                enum_ = __builtin_fmaf(enum_, sa, ln * sb);
                eden = __builtin_fmaf(eden, sa, ld * sb);
                eu = nm;
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const float ou = __shfl_xor(eu, off);
            const float onum = __shfl_xor(enum_, off);
            const float oden = __shfl_xor(eden, off);
            const float nm = fmaxf(eu, ou);
            if (nm != kNegInf) {
                const float sa = (eu == kNegInf) ? 0.0f : exp2_(eu - nm);
                const float sb = (ou == kNegInf) ? 0.0f : exp2_(ou - nm);
                enum_ = enum_ * sa + onum * sb;
                eden = eden * sa + oden * sb;
                eu = nm;
            }
        }
        lmax = wave_max(lmax);
        if (lane == 0) {
            part_max[t & 1][wave] = lmax;
            part_u[t & 1][wave] = eu;
            part_num[t & 1][wave] = enum_;
            part_den[t & 1][wave] = eden;
        }
        __syncthreads();
        if (tid == 0) {
            float tu = part_u[t & 1][0], tn = part_num[t & 1][0], td = part_den[t & 1][0];
            for (int i = 1; i < nwaves; ++i) {
                const float ou = part_u[t & 1][i];
                const float nm = fmaxf(tu, ou);
                if (nm == kNegInf) continue;
                const float sa = (tu == kNegInf) ? 0.0f : exp2_(tu - nm);
                const float sb = (ou == kNegInf) ? 0.0f : exp2_(ou - nm);
                tn = tn * sa + part_num[t & 1][i] * sb;
                td = td * sa + part_den[t & 1][i] * sb;
                tu = nm;
            }
            out[t - 1] = tn / td;
        }
        float *tmp = Bc;
        Bc = Bn;
        Bn = tmp;
    }
}

template <int KV, int NT>
hipError_t launch_reg(const BcjrArgs &a, int64_t nb, hipStream_t s) {
    const size_t shmem = 2 * static_cast<size_t>(pad(1 << (16 - KV))) * sizeof(float);
    auto kern = bcjr_reg_kernel<KV, NT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(shmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(NT), shmem, s, a);
    return hipGetLastError();
}

template <int KV, bool IN_LDS>
hipError_t launch_kv(const BcjrArgs &a, int64_t nb, int threads, size_t shmem, hipStream_t s) {
    auto kern = bcjr_kernel<KV, IN_LDS>;
    if (threads > max_threads(KV)) threads = max_threads(KV);
    if (shmem > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(shmem));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nb)), dim3(threads), shmem, s, a);
    return hipGetLastError();
}

template <bool IN_LDS>
hipError_t launch_lds(const BcjrArgs &a, int64_t nb, int threads, size_t shmem, hipStream_t s) {
    switch (a.kv) {
        case 1: return launch_kv<1, IN_LDS>(a, nb, threads, shmem, s);
        case 2: return launch_kv<2, IN_LDS>(a, nb, threads, shmem, s);
        case 3: return launch_kv<3, IN_LDS>(a, nb, threads, shmem, s);
        case 4: return launch_kv<4, IN_LDS>(a, nb, threads, shmem, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool bcjr_supported(int L, int kv) { return kv >= 1 && kv <= kBcjrMaxKV && kv < L && L <= 16; }

bool bcjr_in_lds(int L, int kv) {
    return (size_t{2} << (L - kv)) * sizeof(float) <= kBcjrLdsBytes;
}

size_t bcjr_per_block_bytes(int L, int kv, int n) {
    const size_t X = size_t{1} << (L - kv);
    size_t b = align_up(static_cast<size_t>(n) * X * sizeof(float), 256);
    if (!bcjr_in_lds(L, kv)) b += align_up(2 * X * sizeof(float), 256);
    return b;
}

hipError_t launch_bcjr(const float *W, int64_t ldw, const float *d, const float *C, int L, int k,
                       int V, int T, int64_t blocks_per_row, int64_t block0, int64_t nb,
                       float tau, char *ws, float *soft, int64_t ldo, float *logz,
                       hipStream_t s) {
    const int kv = k * V;
    const int64_t X = int64_t{1} << (L - kv);
    const int n = T / V;
    BcjrArgs a{};
    a.W = W;
    a.ldw = ldw;
    a.d = d;
    a.C = C;
    a.L = L;
    a.kv = kv;
    a.V = V;
    a.n = n;
    a.blocks_per_row = blocks_per_row;
    a.block0 = block0;
    a.ns = static_cast<float>(-1.4426950408889634074 / static_cast<double>(tau));
    const bool in_lds = bcjr_in_lds(L, kv);
    const size_t fbytes = align_up(static_cast<size_t>(n) * X * sizeof(float), 256);
    a.fstore = reinterpret_cast<float *>(ws);
    a.fstore_per_block = static_cast<int64_t>(bcjr_per_block_bytes(L, kv, n) / sizeof(float));
    a.gbuf = in_lds ? nullptr : reinterpret_cast<float *>(ws + fbytes);
    a.gbuf_per_block = a.fstore_per_block;
    a.soft = soft;
    a.ldo = ldo;
    a.logz = logz;
    // register-codebook kernel: L = 16, V = 1, kv = 2 (8 y values per thread) or 3 (2);
    // its two padded vectors (132 KiB at kv = 2) sit in LDS
    if (L == 16 && V == 1 && (kv == 2 || kv == 3))
        return kv == 2 ? launch_reg<2, 512>(a, nb, s) : launch_reg<3, 512>(a, nb, s);
    int threads = static_cast<int>(X < kMaxThreads ? X : kMaxThreads);
    threads = ((threads + 63) / 64) * 64;
    const size_t shmem = in_lds ? 2 * static_cast<size_t>(X) * sizeof(float) : 0;
    return in_lds ? launch_lds<true>(a, nb, threads, shmem, s)
                  : launch_lds<false>(a, nb, threads, shmem, s);
}

}  // namespace tcq
