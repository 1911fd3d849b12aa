/*
 * tcq_oracle.c -- plain, slow, single-threaded CPU oracle for the bitshift-trellis
 * Viterbi encoder.  TEST INFRASTRUCTURE ONLY: it exists so the GPU library can be
 * checked against something obviously correct.  Only tests/, the smoke check and the
 * CPU-baseline leg of bench.py may load it.  It shares no source with the GPU library.
 *
 * What it computes (sources are the pages' own passages):
 *  - Trellis-coded quantization with a "bitshift" trellis and a lookup-only codebook
 *    (QTIP abstract, "QTIP: Quantization with Trellises and Incoherence Processing").
 *    Reading used here: an L-bit state takes in k*V fresh bits per step,
 *    s_t = ((s_{t-1} << kV) | b_t) mod 2^L, and emits the V values in codebook row s_t.
 *  - Each state restricts the next group to one coset of the codebook; the chunk of
 *    bits coded for the group both indexes a value of that coset and determines the
 *    following state (Pingala-8 post, the trellis-coded quantization paragraph and its
 *    1-bit toy example).
 *  - The cost is a sum of squared errors (same toy: plain rounding totals 1.42).
 *  - Each squared error is weighted by d_i, the diagonal of the Hessian's LDL factor,
 *    inside the Viterbi branch metric, and each coding block carries its own start
 *    state (CurveTQ abstract on the aqora listing).
 *  - The optimum over all paths comes from Viterbi dynamic programming: after each step
 *    a state retains only its lowest-cost incoming path (Pingala-8 post, the paragraph
 *    that follows the toy).
 *  - The codebook is a closed-form quantile table (CurveTQ abstract): Gaussian quantiles
 *    Phi^-1((j+1/2)/N), placed in a seeded shuffled order.
 *
 * Arithmetic (the pages fix fp32 for the ACS but not an evaluation order; the order
 * below is the reading this project uses on both sides):
 *     e   = fl(w - c)
 *     acc = fmaf(fl(d * e), e, acc)        for v = 0..V-1 in order
 * acc starts at +0 for the first step and at the chosen predecessor cost afterwards.
 * With d == NULL the weight is exactly 1, and fmaf(e, e, acc) is used (fl(1*e) == e).
 * Ties: strict '<' over ascending predecessor index j, then the lowest end state.
 *
 * Error feedback (LDLQ) over coding blocks: oracle_ldlq_row, with its own note below.
 * Soft trellis (BCJR) at a temperature: oracle_bcjr_block, with its own note below.
 * Pre-processing: oracle_hadamard_row (randomized Hadamard rotation) and
 * oracle_scale_field (factored scale field), with their own notes below.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* ------------------------------------------------------------------------- */
/* Inverse standard normal CDF: Wichura (1988), Applied Statistics algorithm   */
/* AS 241, "PPND16" (about 1e-16 relative accuracy), evaluated in double.      */
/* ------------------------------------------------------------------------- */
static double horner8(const double *c, double x)
{
    /* c[0] + c[1] x + ... + c[7] x^7, innermost first */
    double r = c[7];
    for (int i = 6; i >= 0; --i)
        r = r * x + c[i];
    return r;
}

double oracle_inv_normal_cdf(double p)
{
    static const double A[8] = {3.3871328727963666080e0, 1.3314166789178437745e+2,
                                1.9715909503065514427e+3, 1.3731693765509461125e+4,
                                4.5921953931549871457e+4, 6.7265770927008700853e+4,
                                3.3430575583588128105e+4, 2.5090809287301226727e+3};
    static const double B[8] = {1.0, 4.2313330701600911252e+1,
                                6.8718700749205790830e+2, 5.3941960214247511077e+3,
                                2.1213794301586595867e+4, 3.9307895800092710610e+4,
                                2.8729085735721942674e+4, 5.2264952788528545610e+3};
    static const double Cc[8] = {1.42343711074968357734e0, 4.63033784615654529590e0,
                                 5.76949722146069140550e0, 3.64784832476320460504e0,
                                 1.27045825245236838258e0, 2.41780725177450611770e-1,
                                 2.27238449892691845833e-2, 7.74545014278341407640e-4};
    static const double D[8] = {1.0, 2.05319162663775882187e0,
                                1.67638483018380384940e0, 6.89767334985100004550e-1,
                                1.48103976427480074590e-1, 1.51986665636164571966e-2,
                                5.47593808499534494600e-4, 1.05075007164441684324e-9};
    static const double E[8] = {6.65790464350110377720e0, 5.46378491116411436990e0,
                                1.78482653991729133580e0, 2.96560571828504891230e-1,
                                2.65321895265761230930e-2, 1.24266094738807843860e-3,
                                2.71155556874348757815e-5, 2.01033439929228813265e-7};
    static const double F[8] = {1.0, 5.99832206555887937690e-1,
                                1.36929880922735805310e-1, 1.48753612908506148525e-2,
                                7.86869131145613259100e-4, 1.84631831751005468180e-5,
                                1.42151175831644588870e-7, 2.04426310338993978564e-15};
    if (!(p > 0.0 && p < 1.0))
        return NAN;
    double q = p - 0.5;
    if (fabs(q) <= 0.425) {
        double r = 0.180625 - q * q;
        return q * horner8(A, r) / horner8(B, r);
    }
    double r = (q < 0.0) ? p : 1.0 - p;
    r = sqrt(-log(r));
    double x;
    if (r <= 5.0) {
        r -= 1.6;
        x = horner8(Cc, r) / horner8(D, r);
    } else {
        r -= 5.0;
        x = horner8(E, r) / horner8(F, r);
    }
    return (q < 0.0) ? -x : x;
}

/* ------------------------------------------------------------------------- */
/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number     */
/* generators", OOPSLA 2014): add the golden gamma, then the variant-13 mixer. */
/* ------------------------------------------------------------------------- */
uint64_t oracle_splitmix64_next(uint64_t *state)
{
    *state += 0x9E3779B97F4A7C15ULL;
    uint64_t z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* 1-D table of 2^bits Gaussian quantiles in ascending order; antisymmetric by
 * construction: the upper half is the exact negation of the lower half. */
static void quantile_grid(int bits, float *g)
{
    long m = 1L << bits;
    for (long j = 0; j < m / 2; ++j) {
        double p = ((double)j + 0.5) / (double)m;
        float v = (float)oracle_inv_normal_cdf(p);
        g[j] = v;
        g[m - 1 - j] = -v;
    }
    if (m == 1)
        g[0] = 0.0f;
}

/*
 * Codebook with 2^L rows of V floats, row-major.
 * Row e of the unshuffled table is a product-grid point: the L index bits are split
 * into V fields (field 0 most significant, the first L mod V fields one bit wider),
 * and coordinate v is the 1-D Gaussian quantile selected by field v.  For V == 1 this
 * is the plain table Phi^-1((j+1/2)/2^L).  Rows are then placed in a seeded order by a
 * Fisher-Yates shuffle driven by SplitMix64: for i = N-1 down to 1, j = next() mod (i+1),
 * swap rows i and j.
 */
int oracle_make_codebook(int L, int V, uint64_t seed, float *out)
{
    if (L < 1 || L > 24 || V < 1 || V > 8 || V > L || out == NULL)
        return ORACLE_EINVAL;
    long n = 1L << L;
    int fbits[8];
    for (int v = 0; v < V; ++v)
        fbits[v] = L / V + ((v < L % V) ? 1 : 0);
    float *grids[8];
    for (int v = 0; v < V; ++v) {
        grids[v] = (float *)malloc(sizeof(float) * ((size_t)1 << fbits[v]));
        if (!grids[v]) {
            for (int u = 0; u < v; ++u)
                free(grids[u]);
            return ORACLE_ENOMEM;
        }
        quantile_grid(fbits[v], grids[v]);
    }
    for (long e = 0; e < n; ++e) {
        int shift = L;
        for (int v = 0; v < V; ++v) {
            shift -= fbits[v];
            long a = (e >> shift) & ((1L << fbits[v]) - 1);
            out[e * V + v] = grids[v][a];
        }
    }
    for (int v = 0; v < V; ++v)
        free(grids[v]);
    uint64_t st = seed;
    for (long i = n - 1; i >= 1; --i) {
        long j = (long)(oracle_splitmix64_next(&st) % (uint64_t)(i + 1));
        for (int v = 0; v < V; ++v) {
            float t = out[i * V + v];
            out[i * V + v] = out[j * V + v];
            out[j * V + v] = t;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Branch metric chain                                                        */
/* ------------------------------------------------------------------------- */
/* acc + sum_v d_i (w_i - c_v)^2 for the V weights of one step, in the order stated in
 * the header.  w and d point at the step's first weight; d may be NULL (weight 1). */
static float chain(float acc, const float *w, const float *d, const float *c, int V)
{
    for (int v = 0; v < V; ++v) {
        float e = w[v] - c[v];
        float de = d ? d[v] * e : e;
        acc = fmaf(de, e, acc);
    }
    return acc;
}

static int check_shape(int L, int k, int V, int T)
{
    if (L < 1 || L > 20 || k < 1 || V < 1 || T < 1)
        return 0;
    if (T % V != 0)
        return 0;
    if (k * V > L)
        return 0;
    return 1;
}

/* ------------------------------------------------------------------------- */
/* Bitstream: chunks b_1..b_n of kV bits each, chunk b_1 first, every chunk     */
/* most-significant bit first, packed into 32-bit words most-significant bit    */
/* first.  ceil(k*T/32) words per block.                                        */
/* ------------------------------------------------------------------------- */
static void put_bits(uint32_t *words, long pos, uint32_t val, int nbits)
{
    for (int i = nbits - 1; i >= 0; --i, ++pos) {
        uint32_t bit = (val >> i) & 1u;
        words[pos / 32] |= bit << (31 - (pos % 32));
    }
}

static uint32_t get_bits(const uint32_t *words, long pos, int nbits)
{
    uint32_t v = 0;
    for (int i = 0; i < nbits; ++i, ++pos)
        v = (v << 1) | ((words[pos / 32] >> (31 - (pos % 32))) & 1u);
    return v;
}

/* Replays the state sequence of a path and writes the reconstruction, T floats. */
void oracle_decode_block(const uint32_t *bits, uint32_t s0, const float *C, int L, int k,
                         int V, int T, float *out)
{
    int kv = k * V;
    int n = T / V;
    uint32_t mask = (L >= 32) ? 0xFFFFFFFFu : ((1u << L) - 1u);
    uint32_t s = s0;
    for (int t = 1; t <= n; ++t) {
        uint32_t b = get_bits(bits, (long)(t - 1) * kv, kv);
        s = ((s << kv) | b) & mask;
        for (int v = 0; v < V; ++v)
            out[(t - 1) * V + v] = C[(size_t)s * V + v];
    }
}

/* Cost of the path (s0, bits) recomputed by the same chain, step by step. */
float oracle_path_cost(const float *w, const float *d, const float *C, int L, int k, int V,
                       int T, const uint32_t *bits, uint32_t s0)
{
    int kv = k * V;
    int n = T / V;
    uint32_t mask = (1u << L) - 1u;
    uint32_t s = s0;
    float acc = 0.0f;
    for (int t = 1; t <= n; ++t) {
        uint32_t b = get_bits(bits, (long)(t - 1) * kv, kv);
        s = ((s << kv) | b) & mask;
        acc = chain(acc, w + (t - 1) * V, d ? d + (t - 1) * V : NULL, C + (size_t)s * V, V);
    }
    return acc;
}

/*
 * Viterbi over one coding block of T weights.
 *   w, d      : T floats each (d may be NULL: every weight 1)
 *   C         : 2^L rows of V floats
 *   fixed_s0  : -1 for a free start state, else the start state (< 2^(L-kV))
 * Outputs the packed bitstream (ceil(kT/32) words, zero-filled here), the start state
 * and the fp32 cost of the chosen path.
 *
 * Step t = 1: J_1(s) = chain(+0, step 1, s) for every state s reachable from an allowed
 * start (all 2^L states when the start is free).
 * Step t >= 2: the predecessors of s' = (x << kV) | b are p_j = (j << (L-kV)) | x,
 * j = 0..2^kV-1; they depend only on the group x = s' >> kV.  For each group keep the
 * smallest J_{t-1}(p_j), lowest j on ties, remember j, and extend every successor.
 * End: lowest-index argmin of J_n; trace back through the remembered j.
 */
int oracle_encode_block(const float *w, const float *d, const float *C, int L, int k,
                        int V, int T, int fixed_s0, uint32_t *bits, uint32_t *s0_out,
                        float *cost_out)
{
    if (!check_shape(L, k, V, T) || !w || !C || !bits || !s0_out || !cost_out)
        return ORACLE_EINVAL;
    int kv = k * V;
    int n = T / V;
    long nstates = 1L << L;
    long ngroups = 1L << (L - kv);
    long G = 1L << kv;
    if (fixed_s0 >= 0 && fixed_s0 >= ngroups)
        return ORACLE_EINVAL;

    float *J = (float *)malloc(sizeof(float) * nstates);
    float *Jn = (float *)malloc(sizeof(float) * nstates);
    uint8_t *bp = (uint8_t *)malloc((size_t)n * ngroups); /* bp[t-1][x], t >= 2 used */
    if (!J || !Jn || !bp) {
        free(J);
        free(Jn);
        free(bp);
        return ORACLE_ENOMEM;
    }

    /* step 1 */
    for (long s = 0; s < nstates; ++s) {
        long start = s >> kv;
        if (fixed_s0 >= 0 && start != fixed_s0)
            J[s] = INFINITY;
        else
            J[s] = chain(0.0f, w, d, C + (size_t)s * V, V);
    }
    /* steps 2..n */
    for (int t = 2; t <= n; ++t) {
        const float *wt = w + (t - 1) * V;
        const float *dt = d ? d + (t - 1) * V : NULL;
        for (long x = 0; x < ngroups; ++x) {
            float m = J[x];
            int jbest = 0;
            for (long j = 1; j < G; ++j) {
                float c = J[(j << (L - kv)) | x];
                if (c < m) {
                    m = c;
                    jbest = (int)j;
                }
            }
            bp[(size_t)(t - 1) * ngroups + x] = (uint8_t)jbest;
            for (long b = 0; b < G; ++b) {
                long sn = (x << kv) | b;
                Jn[sn] = chain(m, wt, dt, C + (size_t)sn * V, V);
            }
        }
        float *tmp = J;
        J = Jn;
        Jn = tmp;
    }
    /* final select: lowest index among the minima */
    long sbest = 0;
    for (long s = 1; s < nstates; ++s)
        if (J[s] < J[sbest])
            sbest = s;
    *cost_out = J[sbest];

    /* traceback */
    int nwords = (k * T + 31) / 32;
    memset(bits, 0, sizeof(uint32_t) * nwords);
    long s = sbest;
    for (int t = n; t >= 2; --t) {
        long b = s & (G - 1);
        long x = s >> kv;
        put_bits(bits, (long)(t - 1) * kv, (uint32_t)b, kv);
        long j = bp[(size_t)(t - 1) * ngroups + x];
        s = (j << (L - kv)) | x;
    }
    put_bits(bits, 0, (uint32_t)(s & (G - 1)), kv);
    *s0_out = (uint32_t)(s >> kv);

    free(J);
    free(Jn);
    free(bp);
    return ORACLE_OK;
}

/*
 * The two smallest fp32 path costs over all distinct paths of a block (a multiset:
 * two different paths of equal cost give best == second).  The per-step extension
 * fmaf(de, e, acc) is monotone non-decreasing in acc, so keeping the two smallest
 * costs per state (taken over all predecessors' pairs) is exact.
 */
int oracle_two_best_block(const float *w, const float *d, const float *C, int L, int k,
                          int V, int T, int fixed_s0, float *best_out, float *second_out)
{
    if (!check_shape(L, k, V, T) || !w || !C || !best_out || !second_out)
        return ORACLE_EINVAL;
    int kv = k * V;
    int n = T / V;
    long nstates = 1L << L;
    long ngroups = 1L << (L - kv);
    long G = 1L << kv;
    if (fixed_s0 >= 0 && fixed_s0 >= ngroups)
        return ORACLE_EINVAL;
    float *J1 = (float *)malloc(sizeof(float) * nstates);
    float *J2 = (float *)malloc(sizeof(float) * nstates);
    float *N1 = (float *)malloc(sizeof(float) * nstates);
    float *N2 = (float *)malloc(sizeof(float) * nstates);
    if (!J1 || !J2 || !N1 || !N2) {
        free(J1);
        free(J2);
        free(N1);
        free(N2);
        return ORACLE_ENOMEM;
    }
    for (long s = 0; s < nstates; ++s) {
        long start = s >> kv;
        J1[s] = (fixed_s0 >= 0 && start != fixed_s0) ? INFINITY
                                                     : chain(0.0f, w, d, C + (size_t)s * V, V);
        J2[s] = INFINITY;
    }
    for (int t = 2; t <= n; ++t) {
        const float *wt = w + (t - 1) * V;
        const float *dt = d ? d + (t - 1) * V : NULL;
        for (long x = 0; x < ngroups; ++x) {
            float a = INFINITY, b2 = INFINITY; /* a <= b2: two smallest so far */
            for (long j = 0; j < G; ++j) {
                long p = (j << (L - kv)) | x;
                float cands[2] = {J1[p], J2[p]};
                for (int u = 0; u < 2; ++u) {
                    float c = cands[u];
                    if (c < a) {
                        b2 = a;
                        a = c;
                    } else if (c < b2) {
                        b2 = c;
                    }
                }
            }
            for (long b = 0; b < G; ++b) {
                long sn = (x << kv) | b;
                N1[sn] = chain(a, wt, dt, C + (size_t)sn * V, V);
                N2[sn] = chain(b2, wt, dt, C + (size_t)sn * V, V);
            }
        }
        float *t1 = J1, *t2 = J2;
        J1 = N1;
        J2 = N2;
        N1 = t1;
        N2 = t2;
    }
    float a = INFINITY, b2 = INFINITY;
    for (long s = 0; s < nstates; ++s) {
        float cands[2] = {J1[s], J2[s]};
        for (int u = 0; u < 2; ++u) {
            float c = cands[u];
            if (c < a) {
                b2 = a;
                a = c;
            } else if (c < b2) {
                b2 = c;
            }
        }
    }
    *best_out = a;
    *second_out = b2;
    free(J1);
    free(J2);
    free(N1);
    free(N2);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Error feedback over coding blocks (LDLQ).                                  */
/* Pingala-8 post, error-feedback toy and LDLQ paragraph: columns are          */
/* quantized in order and each one's error is pushed onto the columns not yet  */
/* quantized, with weights that come from H.  QTIP applies this per block of   */
/* columns.  Reading: H = U diag(d) U^T with U unit upper triangular; column c */
/* of block j (columns jT..jT+T-1) is coded against the target                 */
/*     t_c = w_c + sum_{i < jT} (w_i - what_i) U[i][c],                        */
/* evaluated in fp32 as acc = w_c; acc = fmaf(fl(w_i - what_i), U[i][c], acc)  */
/* for i = 0, 1, ..., jT-1 in that order.  Then the proxy loss                 */
/* (w - what) H (w - what)^T equals sum_c d_c eta_c^2 with eta = (w - what) U, */
/* and eta_c = t_c - what_c when T = 1.  Entries of U inside a block are not   */
/* used.  One row of W at a time (rows are independent).                       */
/* ------------------------------------------------------------------------- */
int oracle_ldlq_row(const float *w, const float *U, long ldu, const float *d, const float *C,
                    int L, int k, int V, int T, long N, uint32_t *bits, uint32_t *s0_out,
                    float *cost_out, float *what, float *target)
{
    if (!check_shape(L, k, V, T) || N < 0 || N % T != 0 || ldu < N)
        return ORACLE_EINVAL;
    const long nblk = N / T;
    const long nw = ((long)k * T + 31) / 32;
    float *err = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    if (!err)
        return ORACLE_ENOMEM;
    for (long j = 0; j < nblk; ++j) {
        const long c0 = j * T;
        for (long c = c0; c < c0 + T; ++c) {
            float acc = w[c];
            for (long i = 0; i < c0; ++i)
                acc = fmaf(err[i], U[i * ldu + c], acc);
            target[c] = acc;
        }
        int rc = oracle_encode_block(target + c0, d ? d + c0 : NULL, C, L, k, V, T, -1,
                                     bits + j * nw, s0_out + j, cost_out + j);
        if (rc != ORACLE_OK) {
            free(err);
            return rc;
        }
        oracle_decode_block(bits + j * nw, s0_out[j], C, L, k, V, T, what + c0);
        for (long i = c0; i < c0 + T; ++i)
            err[i] = w[i] - what[i];
    }
    free(err);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Soft trellis (BCJR) at temperature tau.                                     */
/* BCJR-QAT abstract on the aqora listing: a tempered forward-backward (BCJR) */
/* pass takes the place of the hard minimum; its output is the mean emitted    */
/* value under a Gibbs distribution over paths, and as the temperature falls   */
/* to zero it returns to the Viterbi code.  Reading: every path of the block   */
/* (free start: s_1 may be any of the 2^L states) has energy J, the same       */
/* weighted squared error the Viterbi search minimises, and probability        */
/* exp(-J / tau) / Z.  The soft codeword of weight (t-1)V+v is the expectation */
/* of C[s_t][v].  Computed in double with natural logarithms:                  */
/*   g_t(s)     = -sum_v d (w - C[s][v])^2 / tau                               */
/*   a_1(s)     = g_1(s);  a_t(s') = g_t(s') + LSE over predecessors s of      */
/*                a_{t-1}(s)                                                   */
/*   b_n(s)     = 0;       b_t(s)  = LSE over successors s' of                 */
/*                (g_{t+1}(s') + b_{t+1}(s'))                                  */
/*   log Z      = LSE_s a_n(s);  P(s_t = s) = exp(a_t(s) + b_t(s) - log Z)     */
/* LSE(v) = max(v) + log(sum exp(v - max(v))).                                 */
/* ------------------------------------------------------------------------- */
static double lse_update(double m, double *sum, double v)
{
    /* running log-sum-exp: (m, sum) represents m + log(sum) */
    if (v <= m) {
        *sum += exp(v - m);
        return m;
    }
    *sum = *sum * exp(m - v) + 1.0;
    return v;
}

int oracle_bcjr_block(const double *w, const double *d, const float *C, int L, int k, int V,
                      int T, double tau, double *soft_out, double *logz_out)
{
    if (!check_shape(L, k, V, T) || !(tau > 0.0))
        return ORACLE_EINVAL;
    const int n = T / V;
    const int kv = k * V;
    const long S = 1L << L;
    const long mask = S - 1;
    const int G = 1 << kv;
    double *g = (double *)malloc(sizeof(double) * (size_t)S * (size_t)n);
    double *a = (double *)malloc(sizeof(double) * (size_t)S * (size_t)n);
    double *b = (double *)malloc(sizeof(double) * (size_t)S);
    double *bn = (double *)malloc(sizeof(double) * (size_t)S);
    if (!g || !a || !b || !bn) {
        free(g);
        free(a);
        free(b);
        free(bn);
        return ORACLE_ENOMEM;
    }
    for (int t = 0; t < n; ++t) {
        for (long s = 0; s < S; ++s) {
            double m = 0.0;
            for (int v = 0; v < V; ++v) {
                const int i = t * V + v;
                const double e = w[i] - (double)C[s * V + v];
                m += (d ? d[i] : 1.0) * e * e;
            }
            g[(long)t * S + s] = -m / tau;
        }
    }
    /* forward */
    for (long s = 0; s < S; ++s)
        a[s] = g[s];
    for (int t = 1; t < n; ++t) {
        for (long s2 = 0; s2 < S; ++s2) {
            const long x = s2 >> kv; /* predecessors: (j << (L - kv)) | x */
            double m = -INFINITY, sum = 0.0;
            for (int j = 0; j < G; ++j) {
                const long s1 = ((long)j << (L - kv)) | x;
                m = lse_update(m, &sum, a[(long)(t - 1) * S + s1]);
            }
            a[(long)t * S + s2] = g[(long)t * S + s2] + m + log(sum);
        }
    }
    double m = -INFINITY, sum = 0.0;
    for (long s = 0; s < S; ++s)
        m = lse_update(m, &sum, a[(long)(n - 1) * S + s]);
    const double logz = m + log(sum);
    *logz_out = logz;
    /* backward, with the expectation at each step */
    for (long s = 0; s < S; ++s)
        b[s] = 0.0;
    for (int t = n - 1; t >= 0; --t) {
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (long s = 0; s < S; ++s) {
                const double p = exp(a[(long)t * S + s] + b[s] - logz);
                acc += p * (double)C[s * V + v];
            }
            soft_out[t * V + v] = acc;
        }
        if (t == 0)
            break;
        for (long s = 0; s < S; ++s) {
            double mm = -INFINITY, ss = 0.0;
            for (int bb = 0; bb < G; ++bb) {
                const long s2 = ((s << kv) | bb) & mask;
                mm = lse_update(mm, &ss, g[(long)t * S + s2] + b[s2]);
            }
            bn[s] = mm + log(ss);
        }
        for (long s = 0; s < S; ++s)
            b[s] = bn[s];
    }
    free(g);
    free(a);
    free(b);
    free(bn);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Randomized Hadamard rotation.  Pingala-8 post, rotation paragraph and its   */
/* 4x4 example: with R orthogonal, W x = (W R^T)(R x); the usual R is a        */
/* Hadamard matrix with random signs, scaled to be orthogonal.  Reading: R =   */
/* H_n diag(sigma) / sqrt(n) with H_n the Sylvester-ordered Hadamard matrix,   */
/* H_n[k][i] = (-1)^popcount(k & i) (the page's 4x4 example is H_4 / 2).  A    */
/* row longer than n is rotated in consecutive chunks of n (block diagonal R). */
/* Forward: y = R x, i.e. y_k = sum_i H[k][i] sigma_i x_i / sqrt(n).           */
/* Inverse: x = R^T y, i.e. x_i = sigma_i sum_k H[i][k] y_k / sqrt(n).         */
/* Plain O(n^2) sums in double.                                                */
/* ------------------------------------------------------------------------- */
static int popcount_long(unsigned long v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

int oracle_hadamard_row(const double *x, long len, long n, const double *sigma, int inverse,
                        double *y)
{
    if (n < 1 || (n & (n - 1)) != 0 || len % n != 0)
        return ORACLE_EINVAL;
    const double scale = 1.0 / sqrt((double)n);
    for (long base = 0; base < len; base += n) {
        for (long k = 0; k < n; ++k) {
            double acc = 0.0;
            for (long i = 0; i < n; ++i) {
                const double h = (popcount_long((unsigned long)(k & i)) & 1) ? -1.0 : 1.0;
                const double xi = x[base + i] * ((!inverse && sigma) ? sigma[base + i] : 1.0);
                acc += h * xi;
            }
            y[base + k] = acc * scale * ((inverse && sigma) ? sigma[base + k] : 1.0);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Factored row x column scale field.  CurveTQ abstract: no rotation; the      */
/* weights' amplitude is carried by a factored (row times column) scale field. */
/* Reading: one closed-form pass each way,                                     */
/*   a_r = sqrt(mean_c W_rc^2),   b_c = sqrt(mean_r (W_rc / a_r)^2),           */
/* and W = a_r b_c Wn_rc.  Every column of Wn then has unit RMS.  A zero row   */
/* or column gets scale 1.  Double precision.                                  */
/* ------------------------------------------------------------------------- */
int oracle_scale_field(const float *W, long M, long N, long ldw, double *a, double *b,
                       double *Wn)
{
    if (M < 0 || N < 0 || ldw < N)
        return ORACLE_EINVAL;
    for (long r = 0; r < M; ++r) {
        double s = 0.0;
        for (long c = 0; c < N; ++c)
            s += (double)W[r * ldw + c] * (double)W[r * ldw + c];
        a[r] = (s > 0.0) ? sqrt(s / (double)N) : 1.0;
    }
    for (long c = 0; c < N; ++c) {
        double s = 0.0;
        for (long r = 0; r < M; ++r) {
            const double v = (double)W[r * ldw + c] / a[r];
            s += v * v;
        }
        b[c] = (s > 0.0) ? sqrt(s / (double)M) : 1.0;
    }
    if (Wn)
        for (long r = 0; r < M; ++r)
            for (long c = 0; c < N; ++c)
                Wn[r * N + c] = (double)W[r * ldw + c] / (a[r] * b[c]);
    return ORACLE_OK;
}

int oracle_version(void) { return 1; }
