// Decoding (Pingala-8 post, decoding paragraph): a shift register over the bitstream
// gives each step's state, and the state indexes the codebook; the same walk can feed a
// matrix-vector product directly.  Here: W_hat itself (tcq_decode) and y = W_hat x with
// the weights decoded inside the product (tcq_decode_gemv).
//
// The state of step t is the L-bit window of s_0 || b_1 || ... || b_n that ends with
// chunk b_t, so it can be read straight from two neighbouring 32-bit words of the stream
// (the word before the first one being s_0).
//
// The codebook (2^L x V floats; 256 KiB at L=16, V=1) is read at random, one entry per
// step.  From L2 every such read pulls a whole cache line into L1, so the table is staged
// through LDS instead, 128 KiB at a time: P = table / part passes, each taking the steps
// whose state falls in the part held in LDS.  Results are deterministic: every row is
// summed in a fixed order (stated with each kernel), and decoded values are copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {
namespace {

constexpr int kGemvThreads = 1024;
constexpr int kGemvWaves = kGemvThreads / 64;  // rows in flight per workgroup
constexpr int64_t kGemvPartBytes = 128 << 10;     // largest codebook part in LDS
constexpr int64_t kGemvLdsBytes = 132 << 10;      // dynamic LDS used at most

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
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Column kernel.  A unit is U = KV / gcd(KV, 32) stream words holding exactly S = 32 U / KV
// whole steps, and every block's stream is a whole number of units, so unit u of a row
// covers the row's steps u S .. u S + S - 1 (columns (u S + q) V + v).  A workgroup of
// 1024 threads is R_G row groups of NT column threads (NT a multiple of 64, R_G = 1024 /
// NT); column thread c owns units c, c + NT, ... (G of them; G = 1 is built, so rows
// of at most 1024 units) in every row, so its G S V values of x are loaded into
// registers once.  The workgroup takes a contiguous range of
// rows; row group r takes rows r, r + R_G, ... of it, up to RT at a time (a tile).  For
// each unit of a tile row the thread keeps the unit's words w_1..w_U and the words
// m_j = w_j[15:0] w_{j+1}[31:16] that straddle them (w_0 is the word before the unit, or
// s_0 for a block's first unit): every L-bit state window (L <= 16) then lies inside one
// of these registers and is one bit-field extract.  For each part of the codebook in LDS
// (P passes per tile) the state becomes an LDS offset that points at the step's table row
// when the state lies in the part and at a row of zeros past the part otherwise -- an
// unsigned clamp, no branch -- so each step adds an exact 0 in every pass but one.
// Summation order of row y[r]: each column thread keeps one fp32 chain, fmaf over passes,
// its units, steps and coordinates in that order (at most G S V nonzero terms); the 64
// chains of a wave meet in a 6-level DPP reduction; the NT / 64 wave sums of the row are
// added in wave order.
constexpr int kColThreads = 1024;
constexpr int kColWaves = kColThreads / 64;
constexpr int kColRowsMax = 14;   // rows of a tile, per thread, at most
constexpr int kColRegBudget = 66;  // registers for x, a tile's stream words and sums
constexpr int kColBatch = 8;       // table gathers in flight per thread
constexpr int kColTabFloats = static_cast<int>(kGemvPartBytes / 4);  // largest part

struct ColArgs {
    const uint32_t *bits;
    const uint32_t *s0;
    const float *C;
    const float *x;
    float *y;
    int64_t M;
    int64_t bpr;          // blocks per row
    int nwords;           // stream words per block
    int upb;              // units per block
    int64_t upr;          // units per row
    int L;
    int nt;               // column threads per row group (multiple of 64)
    int rgroups;          // row groups per workgroup
    int rt;               // rows per row group in one tile (<= the kernel's RT)
    int64_t rows_per_wg;  // contiguous rows of one workgroup
    int part_log2;        // log2(states per codebook part)
    int parts;
    int c_aligned;        // C is 16-byte aligned and a part is whole float4s
};

template <int KV, int V, int G>
struct ColShape {
    static constexpr int U = KV / gcd_c(KV, 32);
    static constexpr int S = 32 * U / KV;
    static constexpr int NR = 2 * U;  // registers per unit: m_0, w_1, ..., m_{U-1}, w_U
    // table gathers in flight per thread (fewer for rows of two or four floats)
    static constexpr int kB = kColBatch / V;
    static constexpr int B = kB < S ? kB : S;
    // registers left for a tile's stream words and sums (one per row), by the budget
    // measured to compile without spills at 128 VGPRs
    static constexpr int kBudget = U == 1 ? kColRegBudget : kColRegBudget + 6;
    static constexpr int kLeft =
        kBudget - G * S * V - (G * S * V >= 32 && V > 1 ? 16 : 0) - B * V;
    static constexpr int kFit = kLeft / (G * NR + 1);
    // (caps measured on MI355X: two-float rows run 14 rows at a time -- 14336 x 4096 in
    // one tile per workgroup -- while one- and four-float rows gain nothing past 12 and
    // spill above it; three-word units keep 32 x values and six stream registers per row)
    static constexpr int kCap = U == 1 ? (V == 2 ? 14 : 12) : 6;
    static constexpr int RT = kFit < 1 ? 1 : (kFit > kCap ? kCap : kFit);
};

// Sum over the 64 lanes of a wave, returned in every lane: a scan within each row of 16
// lanes (DPP row shifts by 1, 2, 4, 8), then row 0 into row 1 and row 2 into row 3, then
// rows 0-1 into rows 2-3 (row broadcasts); lane 63 ends with the total.  Every lane's
// value passes through at most 6 additions.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_term(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_term<0x111, 0xF>(v);  // row_shr:1
    v += dpp_term<0x112, 0xF>(v);  // row_shr:2
    v += dpp_term<0x114, 0xF>(v);  // row_shr:4
    v += dpp_term<0x118, 0xF>(v);  // row_shr:8
    v += dpp_term<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_term<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// log2 of the bytes of one table row
template <int V>
constexpr int log2_row_bytes() { return V == 1 ? 2 : (V == 2 ? 3 : 4); }

// Part p of the table into LDS by THREADS threads, then the row of zeros after it.  With
// 16-byte aligned parts of at most CHUNKS x THREADS float4, each wave moves its 64-float4
// chunks straight from global memory into LDS (buffer_load_dwordx4 ... lds: lane i's 16
// bytes land at the chunk's LDS address + 16 i), all CHUNKS in flight, then waits for
// them.  One buffer
// descriptor covers the part and the whole byte offset sits in the range-checked VGPR, so
// the lanes of a chunk that runs past the part load zeros (into LDS inside the
// 8 x THREADS float4, where the row of zeros goes anyway).  The chunk's LDS address and
// its test against the part size are scalar.  Copied through registers instead, the loads
// of a thread went out one at a time (the registers hold a tile's values), and the 64-bit
// addresses of per-lane LDS-direct loads made the GEMV kernel spill.
template <int V, int THREADS, int CHUNKS = 8>
__device__ __forceinline__ void copy_part(float *tab, bool vec, const float *C, int p,
                                          int64_t nfl, int64_t n4, int tid) {
    if (vec) {
        // one descriptor over the part; the whole offset is in the (range-checked) VGPR
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(C + static_cast<int64_t>(p) * nfl), 0,
            static_cast<int>(n4 * 16), 0x00020000);
        const int wb = __builtin_amdgcn_readfirstlane(tid & ~63);  // the wave's first thread
        const int n4i = static_cast<int>(n4);  // at most CHUNKS x THREADS
#pragma unroll
        for (int u = 0; u < CHUNKS; ++u) {
            const int base = u * THREADS + wb;  // float4 index of the wave's chunk
            if (base < n4i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(tab + 4 * base), 16,
                    (tid + u * THREADS) * 16, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the LDS writes of the loads above are done
    } else {
        const float *src = C + static_cast<int64_t>(p) * nfl;
        for (int64_t j = tid; j < nfl; j += THREADS) tab[j] = src[j];
    }
    if (tid < 4) tab[nfl + tid] = 0.0f;
}

// One table row (V floats) from LDS; rows are V * 4 bytes and V * 4-byte aligned.
template <int V>
__device__ __forceinline__ void load_row(float (&c)[V], const char *p) {
    if constexpr (V == 1) {
        c[0] = *reinterpret_cast<const float *>(p);
    } else if constexpr (V == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(p);
        c[0] = t.x;
        c[1] = t.y;
    } else {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        c[0] = t.x;
        c[1] = t.y;
        c[2] = t.z;
        c[3] = t.w;
    }
}

// Stream registers of one unit: from the word before it (w_0: the previous word of the
// block, or s_0 for a block's first unit) and its U words, the words w_j and the words
// m_j = w_j[15:0] w_{j+1}[31:16] that straddle them, as m_0, w_1, m_1, w_2, ..., w_U.  Every
// L-bit state window (L <= 16) of the unit then lies inside one of these registers.
template <int U>
__device__ __forceinline__ void unit_regs(uint32_t (&wr)[2 * U], const uint32_t (&w)[U + 1]) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
        wr[2 * j] = __builtin_amdgcn_alignbit(w[j], w[j + 1], 16);
        wr[2 * j + 1] = w[j + 1];
    }
}

// State of step q (0-based; a constant once the caller's loop is unrolled) of a unit: one
// bit-field extract from the register that holds its window.
template <int KV, int NR>
__device__ __forceinline__ uint32_t unit_state(const uint32_t (&wr)[NR], int q, int L) {
    const int e = (q + 1) * KV;  // window end, bits into the unit
    const int j = (e - 1) >> 5;  // word w_{j+1} holds bit e - 1
    // the window [e - L, e) lies in w_{j+1} when it ends past the word's first 16 bits,
    // else in m_j
    const bool in_w = e - 32 * j > 16;
    const uint32_t src = in_w ? wr[2 * j + 1] : wr[2 * j];
    const uint32_t sh = in_w ? 32 * (j + 1) - e : 32 * j + 16 - e;
    return __builtin_amdgcn_ubfe(src, sh, L);
}

template <int KV, int V, int G>
__global__ __launch_bounds__(kColThreads) void gemv_cols_kernel(ColArgs a) {
    using Sh = ColShape<KV, V, G>;
    constexpr int U = Sh::U, S = Sh::S, RT = Sh::RT, NR = Sh::NR;
    constexpr int kLog = log2_row_bytes<V>();
    // LDS: the table part at offset 0 (so a table offset is an LDS address), one row of
    // zeros after it, then the wave sums of a tile's rows
    __shared__ float tab[kColTabFloats + 4 + kColRowsMax * kColWaves];
    const int tid = threadIdx.x;
    const int rg = tid / a.nt;     // row group (uniform per wave: nt is a multiple of 64)
    const int tc = tid - rg * a.nt;
    const int wv = tid >> 6;
    const int lane = tid & 63;
    const bool active_rg = rg < a.rgroups;
    const int64_t per_part = int64_t{1} << a.part_log2;
    const uint32_t dummy = static_cast<uint32_t>(per_part) << kLog;  // the row of zeros
    const int64_t nfl = per_part * V;                                // floats per part
    const int64_t n4 = nfl / 4;
    float(*red)[kColWaves] = reinterpret_cast<float(*)[kColWaves]>(tab + kColTabFloats + 4);

    // x of this thread's units, in registers: x is first copied into LDS with coalesced
    // loads (a row holds at most 1024 units of S V values: at most 32768 floats, which fit
    // where the table parts go), then each thread reads its own S V values from there
    const int64_t xlen = a.upr * S * V;
    for (int64_t j = tid; j < xlen; j += kColThreads) tab[j] = a.x[j];
    __syncthreads();
    float xr[G][S][V];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t u = tc + static_cast<int64_t>(g) * a.nt;
#pragma unroll
        for (int q = 0; q < S; ++q)
#pragma unroll
            for (int v = 0; v < V; ++v)
                xr[g][q][v] = (active_rg && u < a.upr) ? tab[(u * S + q) * V + v] : 0.0f;
    }

    const bool vec = a.c_aligned && n4 <= 8 * kColThreads;

    // where this thread's units sit in a row: block, unit within the block, word offset
    const int64_t wpr = a.bpr * a.nwords;  // stream words per row
    int64_t ublk[G], woff[G];
    int ju[G];
    bool uok[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t u = tc + static_cast<int64_t>(g) * a.nt;
        uok[g] = u < a.upr;
        ublk[g] = u / a.upb;
        ju[g] = static_cast<int>(u - ublk[g] * a.upb);
        woff[g] = ublk[g] * a.nwords + static_cast<int64_t>(ju[g]) * U;
    }

    const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * a.rows_per_wg;
    int64_t r_end = r_begin + a.rows_per_wg;
    if (r_end > a.M) r_end = a.M;
    const int64_t tile_rows = static_cast<int64_t>(a.rgroups) * a.rt;
    for (int64_t t0 = r_begin; t0 < r_end; t0 += tile_rows) {
        // rows of this row group in the tile (uniform per wave): the rest are skipped
        int64_t here = 0;
        if (active_rg && t0 + rg < r_end)
            here = (r_end - t0 - rg + a.rgroups - 1) / a.rgroups;
        const int nrows = static_cast<int>(here < a.rt ? here : a.rt);
        // stream registers of the tile
        uint32_t wr[RT][G][NR];
        float acc[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            acc[i] = 0.0f;
            const int64_t row = t0 + rg + static_cast<int64_t>(a.rgroups) * i;
            const bool rok = i < nrows;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                uint32_t w[U + 1];
                if (rok && uok[g]) {
                    const uint32_t *wb = a.bits + row * wpr + woff[g];
                    w[0] = ju[g] ? wb[-1] : a.s0[row * a.bpr + ublk[g]];
#pragma unroll
                    for (int j = 0; j < U; ++j) w[j + 1] = wb[j];
                } else {
                    // no stream: state 0, multiplied by x = 0 or never summed into a row
#pragma unroll
                    for (int j = 0; j <= U; ++j) w[j] = 0u;
                }
                unit_regs<U>(wr[i][g], w);
            }
        }
        __syncthreads();  // the previous tile is done with the table and the row sums
        copy_part<V, kColThreads>(tab, vec, a.C, 0, nfl, n4, tid);
        __syncthreads();
        for (int p = 0; p < a.parts; ++p) {
            uint32_t negbase = 0u - static_cast<uint32_t>(p) * dummy;  // - part start
            asm volatile("" : "+s"(negbase));  // kept as an addend: one v_lshl_add per step
            // the states are extracted again in every pass (one instruction each) rather
            // than kept in registers across passes
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int j = 0; j < NR; ++j) asm volatile("" : "+v"(wr[i][g][j]));
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if (i < nrows) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        // B gathers are issued before their products are added
#pragma unroll
                        for (int q0 = 0; q0 < S; q0 += Sh::B) {
                            constexpr int B = Sh::B;
                            float c[B][V];
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const uint32_t st = unit_state<KV>(wr[i][g], q0 + b, a.L);
                                uint32_t off = (st << kLog) + negbase;  // wraps below the part
                                off = off < dummy ? off : dummy;
                                load_row<V>(c[b], reinterpret_cast<const char *>(tab) + off);
                            }
#pragma unroll
                            for (int b = 0; b < B; ++b)
#pragma unroll
                                for (int v = 0; v < V; ++v)
                                    acc[i] = __builtin_fmaf(c[b][v], xr[g][q0 + b][v], acc[i]);
                        }
                    }
                }
            }
            if (p + 1 < a.parts) {
                __syncthreads();  // every wave is done with part p
                copy_part<V, kColThreads>(tab, vec, a.C, p + 1, nfl, n4, tid);
                __syncthreads();
            }
        }
        // row sums: a 6-level DPP reduction in each wave, then the row group's waves in order
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if (i < nrows) {
                const float t = wave_sum(acc[i]);
                if (lane == 0) red[i][wv] = t;
            }
        }
        __syncthreads();
        const int cw = a.nt >> 6;  // waves per row group
        if (tc < nrows) {
            const int i = tc;
            const int64_t row = t0 + rg + static_cast<int64_t>(a.rgroups) * i;
            {
                const int w0 = rg * cw;
                float t = red[i][w0];
                for (int w = 1; w < cw; ++w) t += red[i][w0 + w];
                a.y[row] = t;
            }
        }
    }
}

// Any shape: one wave per row; lane l owns words l, l + 64, ... of the row and decodes
// every step whose chunk ends inside its word (a chunk may straddle two words); x is read
// from global memory.  Codebook parts in LDS as above.  Summation order of y[r]: per pass,
// each lane's fp32 chain over its words and their steps and coordinates, the 64 chains in
// a 6-level shuffle tree, and the pass sums added to y[r] in pass order.
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

// Decode kernel: the units above, flattened over the matrix (unit g = r * upr + u, row r,
// unit u of the row).  A workgroup of THREADS threads takes a contiguous range of units in
// tiles of THREADS * RT; thread t holds units t0 + THREADS i + t (i < RT) of a tile: their
// stream registers and the bit patterns of their S V decoded values.  For each codebook
// part in LDS (PART_BYTES at most), every step reads the row at its clamped offset (the
// row of zeros when the state lies outside the part) and ORs it into its value: every pass
// but one ORs in zero bits, so each value ends as the table's float copied bit for bit
// (-0.0 included).  After the last part the unit's S V values, consecutive in the row, are
// stored: through LDS in runs of 1 KiB per wave where the rows are contiguous (ldo = N),
// else 16 bytes at a time where the layout allows.
constexpr int kDecThreads = 1024;
constexpr int kDecPartBytes = 128 << 10;
constexpr int kDecWgPerCu = 1;     // workgroups resident per compute unit (LDS-bound)
constexpr int kDecRegBudget = 80;  // registers for a tile's values and stream registers

template <int KV, int V>
struct DecShape {
    static constexpr int U = KV / gcd_c(KV, 32);
    static constexpr int S = 32 * U / KV;
    static constexpr int NR = 2 * U;
    static constexpr int kB = 8 / V;  // table reads in flight per thread
    static constexpr int B = kB < S ? kB : S;
    // (units of 32 or more values run one per thread: two spill)
    static constexpr int kFit =
        (S * V >= 32 ? 1 : (kDecRegBudget - B * V) / (S * V + NR + 2));
    static constexpr int RT = kFit < 1 ? 1 : (kFit > 4 ? 4 : kFit);
};

struct DecArgs {
    const uint32_t *bits;
    const uint32_t *s0;
    const float *C;
    float *out;
    int64_t ldo;
    int64_t bpr;           // blocks per row
    int nwords;            // stream words per block
    uint32_t upb;          // units per block
    uint32_t upr;          // units per row
    uint32_t units;        // units of the matrix, M * upr
    uint32_t units_per_wg;
    int L;
    int part_log2;
    int parts;
    int c_aligned;         // C is 16-byte aligned and a part is whole float4s
    int vec_out;           // every unit's values start 16-byte aligned
    int dense;             // vec_out and ldo == N: unit g's values start at out + g S V
    int upb_log2;          // log2(upb) when upb is a power of two, else -1
};

// The thread index, recomputed where it is used: the part copies' addresses are then not
// kept in registers across the tile.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Workgroup barrier with a fence on LDS only: the wave's LDS accesses complete before
// it, but not its global stores (which __syncthreads() would wait for).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Stream words w_0 .. w_U of unit u (zeros past the range) and, if need_dst, the offset
// in out of its SV values (-1 past the range).  Blocks are whole units, so a block's
// words are its units' words: unit u's U words follow unit u - 1's (at u U), and its
// block is u / upb (a shift when upb is a power of two); only the row offset in out
// needs the division by the units per row.
template <int U, int SV>
__device__ __forceinline__ void dec_unit_words(const DecArgs &a, uint32_t u, uint32_t u_end,
                                               uint32_t (&w)[U + 1], int64_t &dst,
                                               bool need_dst) {
    dst = -1;
    if (u < u_end) {
        const uint32_t blk = a.upb_log2 >= 0 ? (u >> a.upb_log2) : u / a.upb;
        const uint32_t ju = u - blk * a.upb;
        const uint32_t *wb = a.bits + static_cast<int64_t>(u) * U;
        w[0] = ju ? wb[-1] : a.s0[blk];
#pragma unroll
        for (int j = 0; j < U; ++j) w[j + 1] = wb[j];
        if (need_dst) {
            const uint32_t row = u / a.upr;
            dst = static_cast<int64_t>(row) * a.ldo + static_cast<int64_t>(u - row * a.upr) * SV;
        }
    } else {
#pragma unroll
        for (int j = 0; j <= U; ++j) w[j] = 0u;
    }
}

template <int KV, int V, int THREADS, int PART_BYTES, int RT>
__global__ __launch_bounds__(THREADS, THREADS * kDecWgPerCu / 256) void decode_cols_kernel(
    DecArgs a) {
    using Sh = DecShape<KV, V>;
    constexpr int U = Sh::U, S = Sh::S, NR = Sh::NR;
    static_assert(RT >= 1 && RT <= Sh::RT, "rows of a tile");
    constexpr int kLog = log2_row_bytes<V>();
    static_assert(PART_BYTES / 16 <= 8 * THREADS, "a part is at most 8 float4 per thread");
    static_assert(THREADS * S * V * 4 <= PART_BYTES, "a tile row's values fit the part space");
    __shared__ float tab[PART_BYTES / 4 + 4];  // a table part, then one row of zeros
    const int tid = threadIdx.x;
    const int64_t per_part = int64_t{1} << a.part_log2;
    const uint32_t dummy = static_cast<uint32_t>(per_part) << kLog;
    const int64_t nfl = per_part * V;
    const int64_t n4 = nfl / 4;
    const bool vec = a.c_aligned && n4 <= 8 * THREADS;

    const uint32_t u_begin = blockIdx.x * a.units_per_wg;
    const uint32_t u_end = u_begin + a.units_per_wg < a.units ? u_begin + a.units_per_wg
                                                              : a.units;
    // Dense output (ldo = N, 16-byte aligned): the units of a tile row are consecutive in
    // out, so each row's values are restaged through LDS (the table part is done with by
    // then) and stored as 1 KiB runs per wave.  A unit's float4 c sits in LDS slot
    // j F4 + (c ^ swz(j)): 16 consecutive lanes then write, and read, 64 different banks.
    // The two halves of the workgroup take different memory roles: the first copies the
    // table parts into LDS, the second stores the decoded rows.  Vector memory operations
    // of a wave complete in order, so a wave that both stored and copied would wait for
    // its stores before each part it copies; here the stores drain while the next tile's
    // parts arrive and its passes run.  Barriers fence LDS only (__syncthreads() would
    // also wait for the global stores), and the stores go through a buffer descriptor that
    // ends with the row's values, so every storing thread issues the same number of them
    // and the tail is dropped by the range check.  The next tile's stream words are
    // requested before this tile's stores, so waiting for them does not wait for the
    // stores either.
    constexpr bool kVec = (S * V) % 4 == 0;
    if constexpr (kVec) {
        if (a.dense) {
            constexpr int F4 = (S * V) / 4;  // float4 per unit
            constexpr uint32_t kTile = THREADS * RT;
            constexpr int kHalf = THREADS / 2;  // threads of each role (whole waves)
            const bool copier = tid < kHalf;
            uint32_t wr[RT][NR];
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                uint32_t w[U + 1];
                int64_t dst;
                dec_unit_words<U, S * V>(a, u_begin + i * THREADS + tid, u_end, w, dst, false);
                unit_regs<U>(wr[i], w);
            }
            if (copier) copy_part<V, kHalf, 16>(tab, vec, a.C, 0, nfl, n4, opaque(tid));
            lds_barrier();
            for (uint32_t t0 = u_begin; t0 < u_end; t0 += kTile) {
                uint32_t val[RT][S][V];
#pragma unroll
                for (int i = 0; i < RT; ++i)
#pragma unroll
                    for (int q = 0; q < S; ++q)
#pragma unroll
                        for (int v = 0; v < V; ++v) val[i][q][v] = 0u;
                for (int p = 0; p < a.parts; ++p) {
                    uint32_t negbase = 0u - static_cast<uint32_t>(p) * dummy;
                    asm volatile("" : "+s"(negbase));
#pragma unroll
                    for (int i = 0; i < RT; ++i)
#pragma unroll
                        for (int j = 0; j < NR; ++j) asm volatile("" : "+v"(wr[i][j]));
#pragma unroll
                    for (int i = 0; i < RT; ++i) {
#pragma unroll
                        for (int q0 = 0; q0 < S; q0 += Sh::B) {
                            constexpr int B = Sh::B;
                            float c[B][V];
#pragma unroll
                            for (int b = 0; b < B; ++b) {
                                const uint32_t st = unit_state<KV>(wr[i], q0 + b, a.L);
                                uint32_t off = (st << kLog) + negbase;
                                off = off < dummy ? off : dummy;
                                load_row<V>(c[b], reinterpret_cast<const char *>(tab) + off);
                            }
#pragma unroll
                            for (int b = 0; b < B; ++b)
#pragma unroll
                                for (int v = 0; v < V; ++v)
                                    val[i][q0 + b][v] |= __float_as_uint(c[b][v]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    if (p + 1 < a.parts) {
                        lds_barrier();
                        if (copier)
                            copy_part<V, kHalf, 16>(tab, vec, a.C, p + 1, nfl, n4, opaque(tid));
                        lds_barrier();
                    }
                }
                // the next tile's stream words, requested before this tile's stores
                const uint32_t next = t0 + kTile;
                if (next < u_end) {
#pragma unroll
                    for (int i = 0; i < RT; ++i) {
                        uint32_t w[U + 1];
                        int64_t dst;
                        dec_unit_words<U, S * V>(a, next + i * THREADS + tid, u_end, w, dst, false);
                        unit_regs<U>(wr[i], w);
                    }
                }
                float4 *st4 = reinterpret_cast<float4 *>(tab);
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    lds_barrier();  // the table, or the previous row's values, are read
                    const uint32_t swz_w = (static_cast<uint32_t>(tid) * F4 / 16) & (F4 - 1);
#pragma unroll
                    for (int f = 0; f < F4; ++f)
                        st4[tid * F4 + (f ^ swz_w)] =
                            make_float4(__uint_as_float(val[i][(4 * f) / V][(4 * f) % V]),
                                        __uint_as_float(val[i][(4 * f + 1) / V][(4 * f + 1) % V]),
                                        __uint_as_float(val[i][(4 * f + 2) / V][(4 * f + 2) % V]),
                                        __uint_as_float(val[i][(4 * f + 3) / V][(4 * f + 3) % V]));
                    lds_barrier();
                    if (!copier) {
                        const uint32_t r0 = t0 + i * THREADS;
                        const uint32_t nun =
                            r0 < u_end ? (u_end - r0 < THREADS ? u_end - r0 : THREADS) : 0u;
                        const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
                            a.out + static_cast<int64_t>(r0) * (S * V), 0,
                            static_cast<int>(nun * F4 * 16u), 0x00020000);
                        const uint32_t ts = static_cast<uint32_t>(tid - kHalf);
                        float4 o[2 * F4];
#pragma unroll
                        for (int f = 0; f < 2 * F4; ++f) {
                            const uint32_t pidx = f * kHalf + ts;  // float4 of the row
                            const uint32_t j = pidx / F4, c = pidx % F4;
                            const uint32_t swz = (j * F4 / 16) & (F4 - 1);
                            o[f] = st4[j * F4 + (c ^ swz)];
                        }
#pragma unroll
                        for (int f = 0; f < 2 * F4; ++f)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, o[f]),
                                ors, static_cast<int>((f * kHalf + ts) * 16u), 0, 0);
                    }
                }
                lds_barrier();  // the last row's values are read
                if (next < u_end && copier)
                    copy_part<V, kHalf, 16>(tab, vec, a.C, 0, nfl, n4, opaque(tid));
                lds_barrier();
            }
            return;
        }
    }
    for (uint32_t t0 = u_begin; t0 < u_end; t0 += THREADS * RT) {
        uint32_t wr[RT][NR];
        uint32_t val[RT][S][V];  // bit patterns of the decoded values
        int64_t dst[RT];         // offset of the unit's first value in out
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            uint32_t w[U + 1];
            dec_unit_words<U, S * V>(a, t0 + i * THREADS + tid, u_end, w, dst[i], true);
            unit_regs<U>(wr[i], w);
#pragma unroll
            for (int q = 0; q < S; ++q)
#pragma unroll
                for (int v = 0; v < V; ++v) val[i][q][v] = 0u;
        }
        __syncthreads();  // the previous tile is done with the table
        copy_part<V, THREADS>(tab, vec, a.C, 0, nfl, n4, opaque(tid));
        __syncthreads();
        for (int p = 0; p < a.parts; ++p) {
            uint32_t negbase = 0u - static_cast<uint32_t>(p) * dummy;  // - part start
            asm volatile("" : "+s"(negbase));
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < NR; ++j) asm volatile("" : "+v"(wr[i][j]));
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                // B reads in flight, then their ORs
#pragma unroll
                for (int q0 = 0; q0 < S; q0 += Sh::B) {
                    constexpr int B = Sh::B;
                    float c[B][V];
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const uint32_t st = unit_state<KV>(wr[i], q0 + b, a.L);
                        uint32_t off = (st << kLog) + negbase;  // wraps below the part
                        off = off < dummy ? off : dummy;
                        load_row<V>(c[b], reinterpret_cast<const char *>(tab) + off);
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b)
#pragma unroll
                        for (int v = 0; v < V; ++v) val[i][q0 + b][v] |= __float_as_uint(c[b][v]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (p + 1 < a.parts) {
                __syncthreads();  // every wave is done with part p
                copy_part<V, THREADS>(tab, vec, a.C, p + 1, nfl, n4, opaque(tid));
                __syncthreads();
            }
        }
        constexpr bool kVec = (S * V) % 4 == 0;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            float *o = a.out + dst[i];
            if (dst[i] >= 0 && kVec && a.vec_out) {
#pragma unroll
                for (int f = 0; f < (kVec ? S * V : 0); f += 4)
                    *reinterpret_cast<float4 *>(o + f) =
                        make_float4(__uint_as_float(val[i][f / V][f % V]),
                                    __uint_as_float(val[i][(f + 1) / V][(f + 1) % V]),
                                    __uint_as_float(val[i][(f + 2) / V][(f + 2) % V]),
                                    __uint_as_float(val[i][(f + 3) / V][(f + 3) % V]));
            } else if (dst[i] >= 0) {
#pragma unroll
                for (int q = 0; q < S; ++q)
#pragma unroll
                    for (int v = 0; v < V; ++v) o[q * V + v] = __uint_as_float(val[i][q][v]);
            }
        }
    }
}

// Any other shape: one workgroup per coding block, one thread per step, the codebook read
// from global memory.
// s_t is the L-bit window of s_0 || b_1 || ... || b_n that ends with chunk b_t.
__device__ __forceinline__ uint32_t stream_bits(const uint32_t *words, int nwords, int pos,
                                                int nbits) {
    const int wi = pos >> 5;
    const uint64_t hi = words[wi];
    const uint64_t lo = (wi + 1 < nwords) ? words[wi + 1] : 0u;
    const uint64_t both = (hi << 32) | lo;
    const int shift = 64 - (pos & 31) - nbits;
    return static_cast<uint32_t>((both >> shift) & ((uint64_t{1} << nbits) - 1));
}

__global__ __launch_bounds__(256) void decode_kernel(
    const uint32_t *__restrict__ bitstream, const uint32_t *__restrict__ start_state,
    const float *__restrict__ C, int64_t blocks_per_row, int L, int kv, int V, int n,
    int nwords, float *__restrict__ out, int64_t ldo) {
    const int64_t blk = blockIdx.x;
    const int64_t row = blk / blocks_per_row;
    const int64_t col = blk % blocks_per_row;
    const uint32_t *words = bitstream + blk * nwords;
    const uint32_t s0 = start_state[blk];
    const uint32_t mask = (L >= 32) ? 0xFFFFFFFFu : ((1u << L) - 1u);
    float *o = out + row * ldo + col * static_cast<int64_t>(n) * V;
    for (int t = 1 + threadIdx.x; t <= n; t += blockDim.x) {
        const int P = t * kv;  // stream bits consumed after chunk t
        uint32_t s;
        if (P >= L) {
            s = stream_bits(words, nwords, P - L, L);
        } else {
            s = ((s0 << P) | stream_bits(words, nwords, 0, P)) & mask;
        }
        for (int v = 0; v < V; ++v) o[(t - 1) * V + v] = C[static_cast<int64_t>(s) * V + v];
    }
}


// Raise a kernel's dynamic LDS limit to the most this file uses, once per kernel (the
// attribute is process-wide, so later launches skip the runtime call).  Calls may come
// from several host threads at once.
hipError_t allow_lds(const void *kern) {
    static std::mutex mu;
    static const void *done[64] = {};  // every kernel of this file
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

hipError_t launch_decode(const uint32_t *bitstream, const uint32_t *start_state,
                         const float *C, int64_t M, int64_t N, int L, int k, int V, int T,
                         float *out, int64_t ldo, hipStream_t s) {
    const int64_t per_row = N / T;
    const int64_t nblocks = M * per_row;
    if (nblocks <= 0) return hipSuccess;
    const int kv = k * V;
    const int nwords = (k * T + 31) / 32;
    const int n = T / V;
    // Units kernel: every block a whole number of units, and unit indices within 32 bits.
    const int U = kv / gcd_c(kv, 32);
    const bool whole = (nwords % U == 0) &&
                       (static_cast<int64_t>(kv) * n == static_cast<int64_t>(nwords) * 32);
    const int64_t upr = whole ? per_row * (nwords / U) : 0;
    if (whole && (V == 1 || V == 2 || V == 4) && M * upr + kDecThreads * 8 < (int64_t{1} << 32)) {
        DecArgs a{};
        a.bits = bitstream;
        a.s0 = start_state;
        a.C = C;
        a.out = out;
        a.ldo = ldo;
        a.bpr = per_row;
        a.nwords = nwords;
        a.upb = static_cast<uint32_t>(nwords / U);
        a.upr = static_cast<uint32_t>(upr);
        a.units = static_cast<uint32_t>(M * upr);
        a.upb_log2 = -1;
        for (int b = 0; b < 31; ++b)
            if (a.upb == (1u << b)) a.upb_log2 = b;
        a.L = L;
        int plog = L;
        while ((int64_t{1} << plog) * V * 4 > kDecPartBytes) --plog;
        a.part_log2 = plog;
        a.parts = 1 << (L - plog);
        a.c_aligned = ((reinterpret_cast<uintptr_t>(C) & 15) == 0 &&
                       ((int64_t{1} << plog) * V) % 4 == 0) ? 1 : 0;
        const int S = 32 * U / kv;
        a.vec_out = ((S * V) % 4 == 0 && ldo % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0) ? 1 : 0;
        a.dense = (a.vec_out && ldo == N) ? 1 : 0;
        const void *kern = nullptr;
        const void *kern1 = nullptr;
        int rt = 0;
#define TCQ_DEC_CASE(KV_, V_)                                                              \
    if (kv == KV_ && V == V_) {                                                           \
        kern = reinterpret_cast<const void *>(                                            \
            decode_cols_kernel<KV_, V_, kDecThreads, kDecPartBytes, DecShape<KV_, V_>::RT>); \
        kern1 = reinterpret_cast<const void *>(                                           \
            decode_cols_kernel<KV_, V_, kDecThreads, kDecPartBytes, 1>);                  \
        rt = DecShape<KV_, V_>::RT;                                                       \
    }
        TCQ_DEC_CASE(1, 1)
        TCQ_DEC_CASE(2, 1)
        TCQ_DEC_CASE(2, 2)
        TCQ_DEC_CASE(3, 1)
        TCQ_DEC_CASE(4, 1)
        TCQ_DEC_CASE(4, 2)
        TCQ_DEC_CASE(4, 4)
        TCQ_DEC_CASE(6, 1)
        TCQ_DEC_CASE(6, 2)
        TCQ_DEC_CASE(8, 1)
        TCQ_DEC_CASE(8, 2)
        TCQ_DEC_CASE(8, 4)
#undef TCQ_DEC_CASE
        if (kern) {
            // as many workgroups as fit, each at least one tile row; tiles of one row
            // where a workgroup has fewer units than a full tile (each tile copies the
            // whole table into LDS, so rows are only worth adding when there are units)
            const int64_t units = a.units;
            int64_t grid = (units + kDecThreads - 1) / kDecThreads;
            const int64_t slots = cu_count() * kDecWgPerCu;
            if (grid > slots) grid = slots;
            a.units_per_wg = static_cast<uint32_t>((units + grid - 1) / grid);
            grid = (units + a.units_per_wg - 1) / a.units_per_wg;
            if (a.units_per_wg < static_cast<uint32_t>(kDecThreads * rt)) kern = kern1;
            void *args[] = {&a};  // (the kernel's LDS is static)
            hipError_t e = hipLaunchKernel(kern, dim3(static_cast<unsigned>(grid)),
                                           dim3(kDecThreads), args, 0, s);
            if (e != hipSuccess) return e;
            return hipGetLastError();
        }
    }

    const int threads = n >= 256 ? 256 : (n >= 64 ? ((n + 63) / 64) * 64 : 64);
    // grid.x limit is 2^31-1 blocks; the validated sizes stay far below it
    hipLaunchKernelGGL(decode_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(threads), 0, s,
                       bitstream, start_state, C, per_row, L, k * V, V, n, nwords, out, ldo);
    return hipGetLastError();
}

hipError_t launch_decode_gemv(const uint32_t *bitstream, const uint32_t *start_state,
                              const float *C, const float *x, float *y, int64_t M, int64_t N,
                              int L, int k, int V, int T, hipStream_t s) {
    const int kv = k * V;
    const int n = T / V;
    const int nwords = (k * T + 31) / 32;
    const int64_t bpr = N / T;
    const int64_t wpr = bpr * nwords;
    const int64_t cus = cu_count();
    // Column kernel: every block a whole number of units, a row of at most 1024 units.
    const int U = kv / gcd_c(kv, 32);
    const bool whole = wpr > 0 && (nwords % U == 0) &&
                       (static_cast<int64_t>(kv) * n == static_cast<int64_t>(nwords) * 32);
    const int64_t upr = whole ? wpr / U : 0;
    const int64_t nt = upr >= kColThreads ? kColThreads : ((upr + 63) / 64) * 64;
    const int64_t G = nt > 0 ? (upr + nt - 1) / nt : 0;
    // (a row group of NT threads; R_G = 1024 / NT of them share a workgroup)
    if (whole && G == 1 && (V == 1 || V == 2 || V == 4)) {
        ColArgs a{};
        a.bits = bitstream;
        a.s0 = start_state;
        a.C = C;
        a.x = x;
        a.y = y;
        a.M = M;
        a.bpr = bpr;
        a.nwords = nwords;
        a.upb = nwords / U;
        a.upr = upr;
        a.L = L;
        a.nt = static_cast<int>(nt);
        a.rgroups = static_cast<int>(kColThreads / nt);
        int plog = L;
        while ((int64_t{1} << plog) * V * 4 > kGemvPartBytes) --plog;
        a.part_log2 = plog;
        a.parts = 1 << (L - plog);
        a.c_aligned = ((reinterpret_cast<uintptr_t>(C) & 15) == 0 &&
                       ((int64_t{1} << plog) * V) % 4 == 0) ? 1 : 0;
        int64_t grid = (M + a.rgroups - 1) / a.rgroups;
        if (grid > cus) grid = cus;
        if (grid < 1) grid = 1;
        a.rows_per_wg = (M + grid - 1) / grid;
        grid = (M + a.rows_per_wg - 1) / a.rows_per_wg;
        const int64_t per_rg = (a.rows_per_wg + a.rgroups - 1) / a.rgroups;
        const void *kern = nullptr;
        int rt_max = 0;
#define TCQ_COL_CASE(KV_, V_, G_)                                                         \
    if (kv == KV_ && V == V_ && G == G_) {                                                \
        kern = reinterpret_cast<const void *>(gemv_cols_kernel<KV_, V_, G_>);             \
        rt_max = ColShape<KV_, V_, G_>::RT;                                               \
    }
#define TCQ_COL_CASES(KV_, V_) TCQ_COL_CASE(KV_, V_, 1)
        TCQ_COL_CASES(1, 1)
        TCQ_COL_CASES(2, 1)
        TCQ_COL_CASES(2, 2)
        TCQ_COL_CASES(3, 1)
        TCQ_COL_CASES(4, 1)
        TCQ_COL_CASES(4, 2)
        TCQ_COL_CASES(4, 4)
        TCQ_COL_CASES(6, 1)
        TCQ_COL_CASES(6, 2)
        TCQ_COL_CASES(8, 1)
        TCQ_COL_CASES(8, 2)
        TCQ_COL_CASES(8, 4)
#undef TCQ_COL_CASES
#undef TCQ_COL_CASE
        if (kern) {
            // the fewest tiles per row group, then rows spread evenly over them
            const int64_t tiles = (per_rg + rt_max - 1) / rt_max;
            a.rt = static_cast<int>((per_rg + tiles - 1) / tiles);
            void *args[] = {&a};  // (the kernel's LDS is static)
            hipError_t e = hipLaunchKernel(kern, dim3(static_cast<unsigned>(grid)),
                                           dim3(kColThreads), args, 0, s);
            if (e != hipSuccess) return e;
            return hipGetLastError();
        }
    }

    // Any other shape: the generic kernel (one wave per row, x from global memory).
    GemvArgs a{};
    a.bits = bitstream;
    a.s0 = start_state;
    a.C = C;
    a.x = x;
    a.y = y;
    a.M = M;
    a.bpr = bpr;
    a.nwords = nwords;
    a.wpr = wpr;
    a.L = L;
    a.kv = kv;
    a.V = V;
    a.n = n;
    a.T = T;
    a.step_c = 64 / a.nwords;
    a.step_j = 64 % a.nwords;
    int plog = 0;
    while (plog < L && (int64_t{2} << plog) * V * 4 <= kGemvPartBytes) ++plog;
    a.part_log2 = plog;
    a.parts = 1 << (L - plog);
    int64_t grid = cus;
    const int64_t need = (M + kGemvWaves - 1) / kGemvWaves;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    const size_t shmem = (size_t{1} << plog) * V * sizeof(float);
    const void *kern = reinterpret_cast<const void *>(gemv_generic_kernel);
    hipError_t e = allow_lds(kern);
    if (e != hipSuccess) return e;
    void *args[] = {&a};
    e = hipLaunchKernel(kern, dim3(static_cast<unsigned>(grid)), dim3(kGemvThreads), args, shmem,
                        s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace tcq
