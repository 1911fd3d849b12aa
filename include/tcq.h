/*
 * tcq.h -- C ABI of libtcq, a bitshift-trellis Viterbi encoder for AMD MI355X (gfx950).
 *
 * The operation (sources: QTIP abstract on the "QTIP: Quantization with Trellises and
 * Incoherence Processing" summary page; the trellis-coded quantization paragraph, the
 * 1-bit toy example and the Viterbi paragraph of the Pingala-8 post; the CurveTQ
 * abstract on the aqora listing):
 *
 *   A weight matrix W (M x N, row-major) is cut into coding blocks of T consecutive
 *   weights along each row: block b = r * (N/T) + c covers W[r, cT .. cT+T-1] and uses
 *   the per-column weights d[cT .. cT+T-1].  Each block is coded as a path through a
 *   "bitshift" trellis: an L-bit state s takes in kV fresh bits per step,
 *       s_t = ((s_{t-1} << kV) | b_t) mod 2^L,          t = 1 .. n,  n = T / V,
 *   and emits the V values C[s_t][0..V-1] of a 2^L-row lookup codebook.  The start
 *   state s_0 < 2^(L-kV) is chosen freely per block.  The encoder returns, per block,
 *   the path of minimum cost
 *       J = sum_i d_i (w_i - what_i)^2
 *   found by Viterbi dynamic programming (each state retains its lowest-cost incoming
 *   path after every step).
 *
 * Arithmetic: fp32 throughout.  Each weight contributes, in order,
 *       e = fl(w - c);  acc = fmaf(fl(d * e), e, acc)        (d == NULL: fmaf(e, e, acc))
 * starting from acc = +0; at each step the predecessor kept for a state is the one
 * with the smallest cost, the lowest predecessor index j on ties, where the
 * predecessors of s' are (j << (L-kV)) | (s' >> kV), j = 0 .. 2^kV - 1.  The chosen end
 * state is the lowest-index minimum.  Costs are never renormalised.  A square that
 * overflows fp32 makes a cost +inf, which is compared like any other value (equal costs
 * keep the lowest index), so such a block still yields a valid path of cost +inf.
 *
 * Memory: every pointer argument of tcq_encode / tcq_decode is a DEVICE pointer owned
 * by the caller (for instance torch tensors); the library never frees or retains them.
 * A workspace argument must start on a 256-byte boundary (every hipMalloc or torch
 * allocation does); others are rejected with TCQ_EINVAL.
 * Calls are asynchronous on `stream` (0 = the null stream); outputs are valid once the
 * stream has completed.  Argument checks happen on the host, synchronously, before
 * anything is enqueued; a call that returns an error has enqueued nothing.
 * The library keeps no state between calls apart from the per-thread error string, a
 * cache of per-kernel launch attributes and, for tcq_encode_noalloc only, its per-GPU
 * scratch array (see there).
 */
#ifndef TCQ_H
#define TCQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every entry point returns one of these. */
typedef enum {
    TCQ_OK = 0,
    TCQ_EINVAL = -1,       /* bad argument (shape, divisibility, null pointer, stride) */
    TCQ_EUNSUPPORTED = -2, /* valid trellis the GPU path does not handle (see limits) */
    TCQ_EWORKSPACE = -3,   /* workspace missing or smaller than the minimum */
    TCQ_EHIP = -4,         /* a HIP runtime call failed (message in tcq_last_error) */
    TCQ_ENOMEM = -5        /* host allocation failed */
} tcq_status;

/* Limits of the GPU path: 2 <= L <= 16, 1 <= k*V <= min(L-1, 8), 1 <= V <= 4,
 * 1 <= T/V <= 1024 steps per block. */
#define TCQ_MAX_L 16
#define TCQ_MAX_KV 8
#define TCQ_MAX_V 4
#define TCQ_MAX_STEPS 1024

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int tcq_version(void);

/* Message describing the last failure on the calling thread ("" if none).  The
 * pointer stays valid until the next call on the same thread. */
const char *tcq_last_error(void);

/*
 * tcq_make_codebook -- the closed-form quantile table that the CurveTQ abstract names, in a
 * seeded shuffled order.
 *   L, V      : 1 <= L <= 24, 1 <= V <= min(L, 8)
 *   seed      : shuffle seed
 *   out_host  : HOST buffer of 2^L * V floats, row-major [2^L][V]; written entirely.
 * Row e of the unshuffled table is a product-grid point: the L bits of e are split into
 * V fields (field 0 most significant; the first L mod V fields get one extra bit) and
 * coordinate v is the Gaussian quantile Phi^-1((a + 1/2) / 2^bits_v) selected by field
 * v (V = 1: the plain table Phi^-1((j + 1/2) / 2^L)).  Phi^-1 is Wichura's AS 241
 * (1988) in double, rounded to float, and made exactly antisymmetric.  Rows are then
 * shuffled by Fisher-Yates from the last row down, with j = SplitMix64(seed) mod (i+1).
 * Host-only; touches no GPU.  Errors: TCQ_EINVAL.
 */
int tcq_make_codebook(int L, int V, uint64_t seed, float *out_host);

/*
 * tcq_encode_workspace_bytes -- device workspace size tcq_encode should be given to
 * encode the whole M x N problem at full speed.  Any workspace of at least
 * tcq_encode_workspace_min_bytes() also works (blocks are then processed in several
 * batches on the stream).  Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED.
 */
int tcq_encode_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                               size_t *bytes);
int tcq_encode_workspace_min_bytes(int L, int k, int V, int T, size_t *bytes);

/*
 * tcq_encode -- Viterbi-encode every coding block of W.
 *   W          : device, M x N floats, row r at W + r * ldw (ldw >= N); finite values
 *   d          : device, N floats >= 0 (finite), or NULL for d == 1 (plain Euclidean)
 *   codebook   : device, 2^L * V floats, row-major [2^L][V]
 *   L, k, V, T : trellis parameters; N % T == 0, T % V == 0, within the GPU limits
 *   bitstream  : device out, [M * N / T][ceil(k*T/32)] uint32.  Block b's chunks
 *                b_1 .. b_n (kV bits each, b_1 first, each most-significant bit
 *                first) packed into words most-significant bit first; unused tail
 *                bits are 0.
 *   start_state: device out, [M * N / T] uint32, s_0 < 2^(L - kV)
 *   cost       : device out, [M * N / T] float, the fp32 cost of the chosen path
 *   recon      : device out or NULL; if given, M x N floats with row stride ldr >= N,
 *                the reconstruction C[s_t][v] at every weight position
 *   workspace  : device scratch of workspace_bytes (>= tcq_encode_workspace_min_bytes)
 *   stream     : HIP stream the work is enqueued on
 * M == 0 or N == 0 is a no-op.  Encoding a row range through pointer offsets gives
 * bitwise the same results as those rows inside a whole-matrix call.
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EWORKSPACE, TCQ_EHIP.
 */
int tcq_encode(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
               const float *codebook, int L, int k, int V, int T, uint32_t *bitstream,
               uint32_t *start_state, float *cost, float *recon, int64_t ldr,
               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tcq_encode_timed -- tcq_encode, plus two events recorded on `stream` for profiling:
 * `acs_begin` immediately before the first forward (add-compare-select) kernel launch
 * and `acs_end` immediately after the last one.  Either event may be NULL.  With a
 * workspace of tcq_encode_workspace_bytes() for problems whose blocks fit one batch
 * there is exactly one forward launch, so hipEventElapsedTime(acs_begin, acs_end) is
 * that kernel's duration; with several batches the span also covers the traceback
 * launches interleaved between them.  Same outputs and errors as tcq_encode.
 */
int tcq_encode_timed(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
                     const float *codebook, int L, int k, int V, int T, uint32_t *bitstream,
                     uint32_t *start_state, float *cost, float *recon, int64_t ldr,
                     void *workspace, size_t workspace_bytes, hipStream_t stream,
                     hipEvent_t acs_begin, hipEvent_t acs_end);

/*
 * tcq_l16_stream_probe -- measurement support: the codebook loads of the L = 16, k*V = 2
 * forward kernel (same per-lane offsets, order and loads in flight, one 8-wave workgroup
 * per block, `super_steps` super-steps of 3 steps per block) with the arithmetic, LDS
 * traffic and backpointer stores taken out, timed between `start` and `stop` (recorded
 * on `stream`; either may be NULL).  Each block reads 768 KiB per super-step from an
 * L2-resident 768 KiB array, so blocks * super_steps * 786432 / elapsed is the rate at which
 * the L2 delivers that access pattern to the compute units, the ceiling of the forward
 * kernel's codebook stream (4 bytes per state update).  Values read are not meaningful.
 *   workspace : device, >= tcq_l16_stream_probe_bytes(blocks) bytes, 256-byte aligned
 * Errors: TCQ_EINVAL (blocks < 1 or > 2^31 - 1, super_steps < 1, NULL or small
 * workspace), TCQ_EHIP.
 */
size_t tcq_l16_stream_probe_bytes(int64_t blocks);
int tcq_l16_stream_probe(int64_t blocks, int super_steps, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);

/*
 * tcq_encode_noalloc -- tcq_encode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and errors as tcq_encode, without the workspace: the library uses a
 * file-scope device array of TCQ_NOALLOC_SCRATCH_BYTES (256 MiB) as the workspace, which
 * every GPU it runs on holds from the first call on that GPU until the process ends.  The
 * call allocates nothing (no hipMalloc, no hipFree); the device address of the array is
 * looked up once per GPU.  Blocks are encoded in batches that fit the scratch (255 blocks
 * at L = 16, k*V = 2, T = 256), so any number of rows is accepted; a shape whose single block
 * needs more scratch than that is rejected with TCQ_EUNSUPPORTED (no shape within the GPU
 * limits does: the largest, L = 16, k = 2, V = 2, T = 2048, needs 9.5 MiB).  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (two streams, two host threads) race and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 */
#define TCQ_NOALLOC_SCRATCH_BYTES (256ull << 20)
int tcq_encode_noalloc(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
                       const float *codebook, int L, int k, int V, int T, uint32_t *bitstream,
                       uint32_t *start_state, float *cost, float *recon, int64_t ldr,
                       hipStream_t stream);

/*
 * tcq_decode -- rebuild weights from bitstreams (Pingala-8 post, decoding paragraph: the
 * state is a shift register over the chunks, and each state indexes the codebook).
 *   bitstream, start_state : device, as written by tcq_encode for an M x N problem
 *   codebook               : device, 2^L * V floats
 *   out                    : device out, M x N floats with row stride ldo >= N;
 *                            out[r, cT + (t-1)V + v] = C[s_t][v] of block r*(N/T)+c
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EHIP.
 */
int tcq_decode(const uint32_t *bitstream, const uint32_t *start_state, const float *codebook,
               int64_t M, int64_t N, int L, int k, int V, int T, float *out, int64_t ldo,
               hipStream_t stream);

/*
 * tcq_decode_gemv -- y = W_hat x with W_hat decoded inside the product (Pingala-8 post,
 * decoding paragraph: the decode is fused into the matrix-vector product).
 *   bitstream, start_state : device, as written by tcq_encode for an M x N problem
 *   codebook               : device, 2^L * V floats
 *   x                      : device, N floats
 *   y                      : device out, M floats; y[r] = sum_c W_hat[r, c] x[c]
 * fp32 products and sums (fmaf), summed per row in a fixed order, so repeated calls give
 * identical results.  N == 0 writes y = 0.
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EHIP.
 */
int tcq_decode_gemv(const uint32_t *bitstream, const uint32_t *start_state,
                    const float *codebook, int64_t M, int64_t N, int L, int k, int V, int T,
                    const float *x, float *y, hipStream_t stream);

/*
 * Error feedback over coding blocks (LDLQ).  Pingala-8 post, error-feedback toy and LDLQ
 * paragraph: the columns are quantized in order and each one's error is pushed onto the
 * columns not yet quantized, with weights from H (the average of x x^T over inputs);
 * QTIP and CurveTQ code T columns at a time, so the feedback runs over coding blocks.
 *
 * With H = U D U^T, U unit upper block-triangular (identity T x T diagonal blocks) and D
 * block diagonal, d = diag(D): block j (columns jT..jT+T-1) of every row is encoded
 * exactly as tcq_encode would encode the target
 *     t_c = w_c + sum_{i < jT} (w_i - what_i) U[i][c]
 * with per-column weights d, where what is the reconstruction of the blocks already
 * coded.  fp32 evaluation: acc = w_c; acc = fmaf(fl(w_i - what_i), U[i][c], acc) for
 * i = 0..jT-1 ascending.  Only entries U[i][c] with i / T < c / T are read.
 *
 * tcq_ldlq_workspace_bytes -- device workspace for tcq_encode_ldlq with target and
 *   recon both NULL (enough in every case).
 * tcq_encode_ldlq
 *   W           : device, M x N, leading dimension ldw >= N; not modified
 *   U           : device, N x N, leading dimension ldu >= N (may be NULL when N == T)
 *   d           : device, N floats, or NULL for d == 1
 *   codebook, L, k, V, T, bitstream, start_state, cost : as tcq_encode (matrix layout:
 *                 block r*(N/T)+j covers row r, columns jT..jT+T-1)
 *   recon       : nullable device M x ldr; receives what
 *   target      : nullable device M x ldt; receives the targets t (the library keeps them
 *                 in the workspace when NULL)
 *   workspace   : >= what tcq_ldlq_workspace_bytes reports
 * Runs N/T encodes in sequence on `stream`; rows are independent.
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EWORKSPACE, TCQ_EHIP.
 */
int tcq_ldlq_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                             size_t *bytes);
int tcq_encode_ldlq(const float *W, int64_t M, int64_t N, int64_t ldw, const float *U,
                    int64_t ldu, const float *d, const float *codebook, int L, int k, int V,
                    int T, uint32_t *bitstream, uint32_t *start_state, float *cost,
                    float *recon, int64_t ldr, float *target, int64_t ldt, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Soft trellis (BCJR) at temperature tau.  BCJR-QAT abstract on the aqora listing: a
 * tempered forward-backward pass stands in for the hard minimum of the Viterbi search;
 * each output is the mean emitted value when paths are weighted by exp(-J / tau), and
 * as tau falls to 0 the output returns to the hard (Viterbi) reconstruction.
 *
 * Every path of a block (free start, as tcq_encode) has energy J, the same weighted
 * squared error tcq_encode minimises, and probability exp(-J / tau) / Z.
 *   soft[r][cT + i] = E[ what_i ] over that distribution (block r*(N/T)+c)
 *   logz[b]         = log Z of block b (natural log), nullable
 * fp32 branch metrics (the encoder's chain), base-2 log-sum-exp in fp32 with the hardware
 * exp2/log2, per-step shifts summed in double for log Z.  Results are deterministic.
 * Supported: every tcq_encode shape with k*V <= 4.
 *
 * tcq_bcjr_workspace_bytes -- recommended workspace (a batch of blocks); the minimum is
 *   one block: (T/V) * 2^(L-kV) * 4 bytes rounded up to 256, plus 2 * 2^(L-kV) * 4 when
 *   2 * 2^(L-kV) * 4 > 128 KiB.
 * tcq_bcjr
 *   W, M, N, ldw, d, codebook, L, k, V, T : as tcq_encode (device pointers)
 *   tau    : temperature, > 0 and finite
 *   soft   : device out, M x ldo (ldo >= N)
 *   logz   : nullable device out, M*N/T floats
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED (k*V > 4), TCQ_EWORKSPACE, TCQ_EHIP.
 */
int tcq_bcjr_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                             size_t *bytes);
int tcq_bcjr(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
             const float *codebook, int L, int k, int V, int T, float tau, float *soft,
             int64_t ldo, float *logz, void *workspace, size_t workspace_bytes,
             hipStream_t stream);

/*
 * tcq_hadamard -- randomized Hadamard rotation of rows (Pingala-8 post, rotation paragraph
 * and its 4x4 example: W x = (W R^T)(R x) for orthogonal R, usually a Hadamard matrix
 * with random signs).  R = H_n diag(sigma) / sqrt(n), H_n Sylvester-ordered
 * (H_n[k][i] = (-1)^popcount(k & i)); rows longer than n are rotated in consecutive
 * chunks of n (block-diagonal R).  Forward: each row x becomes R x (for the rows of W this
 * is W R^T); inverse: R^T y.
 *   X, ldx     : device, rows x len input
 *   n          : power of two, n <= 4096; n divides len; if n < 64 then len <= 8192
 *   sigma      : device, len floats (+1/-1), or NULL for all +1
 *   Y, ldy     : device output; Y == X (with ldy == ldx) works in place
 * fp32 butterflies; |error| <= (log2(n) + 3) u sum|x_i| / sqrt(n) per output, u = 2^-24
 * (log2(n) butterfly levels, the rounded 1/sqrt(n), its multiply and the sign multiply).
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EHIP.
 */
int tcq_hadamard(const float *X, int64_t rows, int64_t len, int64_t ldx, int64_t n,
                 const float *sigma, int inverse, float *Y, int64_t ldy, hipStream_t stream);

/*
 * tcq_scale_field -- factored row x column scale field (CurveTQ abstract: the weights'
 * amplitude is carried by a factored scale field, with no rotation).  One closed-form pass
 * each way: a_r = sqrt(mean_c W_rc^2), b_c = sqrt(mean_r (W_rc / a_r)^2), and
 * Wn_rc = W_rc / (a_r b_c), so W = a_r b_c Wn_rc and every column of Wn has unit RMS.
 * An all-zero row or column gets scale 1.
 *   W, M, N, ldw : device input
 *   row_scale    : device out, M floats (a); col_scale: device out, N floats (b)
 *   Wn, ldn      : nullable device out, M x ldn
 *   workspace    : device, >= tcq_scale_field_workspace_bytes(M, N)
 * fp32 sums in a fixed order (deterministic).
 * Errors: TCQ_EINVAL, TCQ_EUNSUPPORTED, TCQ_EWORKSPACE, TCQ_EHIP.
 */
int tcq_scale_field_workspace_bytes(int64_t M, int64_t N, size_t *bytes);
int tcq_scale_field(const float *W, int64_t M, int64_t N, int64_t ldw, float *row_scale,
                    float *col_scale, float *Wn, int64_t ldn, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TCQ_H */
