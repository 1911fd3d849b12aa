// libtcq C ABI: argument checks, workspace planning, and launch ordering on the
// caller's stream.  Every numeric step runs in the HIP kernels.
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <string>

#include "tcq.h"
#include "tcq_internal.h"

namespace tcq {

namespace {
thread_local std::string g_error;

// Blocks whose backpointers are kept in the workspace at once by the recommended size.
constexpr int64_t kRecommendedBatchBytes = int64_t{24} << 30;  // per-block data cap
constexpr int64_t kMinRecommendedBatch = 1024;
}  // namespace

void set_error(const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
}

static void clear_error() { g_error.clear(); }

// Workspaces must start on a 256-byte boundary (as every hipMalloc or torch allocation
// does): the kernels lay out their buffers at 256-byte offsets from it.
static int check_workspace_alignment(const char *fn, const void *workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) {
        set_error("%s: workspace %p is not 256-byte aligned", fn, workspace);
        return TCQ_EINVAL;
    }
    return TCQ_OK;
}

Plan plan_for(const Problem &p) {
    Plan pl{};
    if (l16_supported(p)) {
        pl.variant = kL16Regs;
        pl.fixed = align_up(l16_fixed_bytes(p), 256);
        pl.bp_bytes = align_up(l16_bp_bytes(p), 256);
        pl.cost_bytes = 0;
    } else if (l16k3_supported(p)) {
        pl.variant = kL16RegsK3;
        pl.fixed = align_up(l16k3_fixed_bytes(p), 256);
        pl.bp_bytes = align_up(l16k3_bp_bytes(p), 256);
        pl.cost_bytes = 0;
    } else if (l16h_supported(p)) {
        pl.variant = kL16RegsHalf;
        pl.fixed = align_up(l16h_fixed_bytes(p), 256);
        pl.bp_bytes = align_up(l16h_bp_bytes(p), 256);
        pl.cost_bytes = 0;
    } else {
        const int64_t nw64 = (p.ngroups + 63) / 64;
        pl.bp_bytes = align_up(static_cast<size_t>(p.n) * p.kv * nw64 * 8, 256);
        if (p.L <= 13) {
            pl.variant = kGenericLds;
            pl.cost_bytes = 0;
        } else {
            pl.variant = kGenericGlobal;
            pl.cost_bytes = align_up(2 * static_cast<size_t>(p.nstates) * sizeof(float), 256);
        }
        pl.fixed = 0;
    }
    // per block: backpointers, cost buffers, and the chosen end state (4 bytes)
    pl.per_block = pl.bp_bytes + pl.cost_bytes + sizeof(uint32_t);
    return pl;
}

// Shared shape checks for encode and decode.
static int check_trellis(const char *fn, int64_t M, int64_t N, int L, int k, int V, int T) {
    if (M < 0 || N < 0) {
        set_error("%s: negative matrix size (M=%lld N=%lld)", fn, (long long)M, (long long)N);
        return TCQ_EINVAL;
    }
    if (L < 1 || k < 1 || V < 1 || T < 1) {
        set_error("%s: L, k, V, T must be positive (L=%d k=%d V=%d T=%d)", fn, L, k, V, T);
        return TCQ_EINVAL;
    }
    if (T % V != 0) {
        set_error("%s: T=%d is not a multiple of V=%d", fn, T, V);
        return TCQ_EINVAL;
    }
    if (N % T != 0) {
        set_error("%s: N=%lld is not a multiple of T=%d", fn, (long long)N, T);
        return TCQ_EINVAL;
    }
    if (static_cast<int64_t>(k) * V >= L) {
        set_error("%s: need k*V < L (k=%d V=%d L=%d)", fn, k, V, L);
        return TCQ_EINVAL;
    }
    if (L > TCQ_MAX_L || k * V > TCQ_MAX_KV || V > TCQ_MAX_V || T / V > TCQ_MAX_STEPS ||
        L < 2) {
        set_error("%s: outside the GPU limits (2<=L<=%d, k*V<=%d, V<=%d, T/V<=%d): "
                  "L=%d k=%d V=%d T=%d",
                  fn, TCQ_MAX_L, TCQ_MAX_KV, TCQ_MAX_V, TCQ_MAX_STEPS, L, k, V, T);
        return TCQ_EUNSUPPORTED;
    }
    return TCQ_OK;
}

static Problem make_problem(int64_t M, int64_t N, int64_t ldw, int L, int k, int V, int T) {
    Problem p{};
    p.L = L;
    p.k = k;
    p.V = V;
    p.T = T;
    p.kv = k * V;
    p.n = T / V;
    p.M = M;
    p.N = N;
    p.ldw = ldw;
    p.blocks_per_row = N / T;
    p.nblocks = M * (N / T);
    p.ngroups = int64_t{1} << (L - p.kv);
    p.nstates = int64_t{1} << L;
    return p;
}

static int hip_fail(const char *fn, const char *what, hipError_t e) {
    set_error("%s: %s failed: %s", fn, what, hipGetErrorString(e));
    return TCQ_EHIP;
}

}  // namespace tcq

using namespace tcq;

extern "C" int tcq_version(void) { return 100; }

extern "C" const char *tcq_last_error(void) { return g_error.c_str(); }

extern "C" int tcq_encode_workspace_min_bytes(int L, int k, int V, int T, size_t *bytes) {
    clear_error();
    int rc = check_trellis("tcq_encode_workspace_min_bytes", 1, T, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!bytes) {
        set_error("tcq_encode_workspace_min_bytes: bytes is NULL");
        return TCQ_EINVAL;
    }
    Problem p = make_problem(1, T, T, L, k, V, T);
    Plan pl = plan_for(p);
    *bytes = pl.fixed + 256 + pl.per_block;
    return TCQ_OK;
}

extern "C" int tcq_encode_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                                          size_t *bytes) {
    clear_error();
    int rc = check_trellis("tcq_encode_workspace_bytes", M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!bytes) {
        set_error("tcq_encode_workspace_bytes: bytes is NULL");
        return TCQ_EINVAL;
    }
    Problem p = make_problem(M, N, N, L, k, V, T);
    Plan pl = plan_for(p);
    int64_t batch = kRecommendedBatchBytes / static_cast<int64_t>(pl.per_block);
    if (batch < kMinRecommendedBatch) batch = kMinRecommendedBatch;
    if (batch > p.nblocks) batch = p.nblocks;
    if (batch < 1) batch = 1;
    *bytes = pl.fixed + 256 + pl.per_block * static_cast<size_t>(batch);
    return TCQ_OK;
}

int tcq::encode_impl(const char *fn, const float *W, int64_t M, int64_t N, int64_t ldw,
                     const float *d, const float *codebook, int L, int k, int V, int T,
                     uint32_t *bitstream, uint32_t *start_state, float *cost, float *recon,
                     int64_t ldr, void *workspace, size_t workspace_bytes, hipStream_t stream,
                     hipEvent_t acs_begin, hipEvent_t acs_end) {
    clear_error();
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (M == 0 || N == 0) return TCQ_OK;
    if (ldw < N) {
        set_error("%s: ldw=%lld < N=%lld", fn, (long long)ldw, (long long)N);
        return TCQ_EINVAL;
    }
    if (!W || !codebook || !bitstream || !start_state || !cost) {
        set_error("%s: W, codebook, bitstream, start_state and cost must be non-NULL", fn);
        return TCQ_EINVAL;
    }
    if (recon && ldr < N) {
        set_error("%s: ldr=%lld < N=%lld", fn, (long long)ldr, (long long)N);
        return TCQ_EINVAL;
    }
    Problem p = make_problem(M, N, ldw, L, k, V, T);
    Plan pl = plan_for(p);
    const size_t need = pl.fixed + 256 + pl.per_block;
    if (!workspace || workspace_bytes < need) {
        set_error("%s: workspace of %zu bytes is below the minimum %zu", fn,
                  workspace ? workspace_bytes : size_t{0}, need);
        return TCQ_EWORKSPACE;
    }
    rc = check_workspace_alignment(fn, workspace);
    if (rc != TCQ_OK) return rc;
    int64_t batch = static_cast<int64_t>((workspace_bytes - pl.fixed - 256) / pl.per_block);
    if (batch > p.nblocks) batch = p.nblocks;
    if (batch > (int64_t{1} << 30)) batch = int64_t{1} << 30;
    char *ws = static_cast<char *>(workspace);

    hipError_t e;
    if (pl.variant == kL16Regs) {
        e = launch_l16_prepare(p, codebook, ws, stream);
        if (e != hipSuccess) return hip_fail(fn, "codebook preparation launch", e);
    } else if (pl.variant == kL16RegsK3) {
        e = launch_l16k3_prepare(p, codebook, ws, stream);
        if (e != hipSuccess) return hip_fail(fn, "codebook preparation launch", e);
    } else if (pl.variant == kL16RegsHalf) {
        e = launch_l16h_prepare(p, codebook, ws, stream);
        if (e != hipSuccess) return hip_fail(fn, "codebook preparation launch", e);
    }
    for (int64_t b0 = 0; b0 < p.nblocks; b0 += batch) {
        const int64_t nb = (p.nblocks - b0 < batch) ? p.nblocks - b0 : batch;
        if (b0 == 0 && acs_begin) {
            e = hipEventRecord(acs_begin, stream);
            if (e != hipSuccess) return hip_fail(fn, "hipEventRecord", e);
        }
        if (pl.variant == kL16Regs) {
            e = launch_acs_l16(p, pl, W, d, b0, nb, ws, cost, stream);
            if (e != hipSuccess) return hip_fail(fn, "ACS launch", e);
            if (b0 + nb >= p.nblocks && acs_end) {
                e = hipEventRecord(acs_end, stream);
                if (e != hipSuccess) return hip_fail(fn, "hipEventRecord", e);
            }
            e = launch_traceback_l16(p, pl, b0, nb, ws, bitstream, start_state, stream);
            if (e != hipSuccess) return hip_fail(fn, "traceback launch", e);
        } else if (pl.variant == kL16RegsHalf) {
            e = launch_acs_l16h(p, pl, W, d, b0, nb, ws, cost, stream);
            if (e != hipSuccess) return hip_fail(fn, "ACS launch", e);
            if (b0 + nb >= p.nblocks && acs_end) {
                e = hipEventRecord(acs_end, stream);
                if (e != hipSuccess) return hip_fail(fn, "hipEventRecord", e);
            }
            // the 2-bit half-step view: 2n steps of k = 2, V = 1 on the relabelled state
            // (halves of every nibble exchanged), converted back by the traceback
            Problem ph = p;
            ph.k = 2;
            ph.V = 1;
            ph.kv = 2;
            ph.n = 2 * p.n;
            ph.T = 2 * p.n;
            e = launch_traceback_l16(ph, pl, b0, nb, ws, bitstream, start_state, stream, true);
            if (e != hipSuccess) return hip_fail(fn, "traceback launch", e);
        } else if (pl.variant == kL16RegsK3) {
            e = launch_acs_l16k3(p, pl, W, d, b0, nb, ws, cost, stream);
            if (e != hipSuccess) return hip_fail(fn, "ACS launch", e);
            if (b0 + nb >= p.nblocks && acs_end) {
                e = hipEventRecord(acs_end, stream);
                if (e != hipSuccess) return hip_fail(fn, "hipEventRecord", e);
            }
            e = launch_traceback_l16k3(p, pl, b0, nb, ws, bitstream, start_state, stream);
            if (e != hipSuccess) return hip_fail(fn, "traceback launch", e);
        } else {
            e = launch_acs_generic(p, pl, W, d, codebook, b0, nb, ws, cost, stream);
            if (e != hipSuccess) return hip_fail(fn, "ACS launch", e);
            if (b0 + nb >= p.nblocks && acs_end) {
                e = hipEventRecord(acs_end, stream);
                if (e != hipSuccess) return hip_fail(fn, "hipEventRecord", e);
            }
            e = launch_traceback_planes(p, pl, b0, nb, ws, bitstream, start_state, stream);
            if (e != hipSuccess) return hip_fail(fn, "traceback launch", e);
        }
    }
    if (recon) {
        e = launch_decode(bitstream, start_state, codebook, M, N, L, k, V, T, recon, ldr, stream);
        if (e != hipSuccess) return hip_fail(fn, "reconstruction launch", e);
    }
    return TCQ_OK;
}

extern "C" int tcq_encode(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
                          const float *codebook, int L, int k, int V, int T,
                          uint32_t *bitstream, uint32_t *start_state, float *cost,
                          float *recon, int64_t ldr, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return encode_impl("tcq_encode", W, M, N, ldw, d, codebook, L, k, V, T, bitstream,
                       start_state, cost, recon, ldr, workspace, workspace_bytes, stream,
                       nullptr, nullptr);
}

extern "C" int tcq_encode_timed(const float *W, int64_t M, int64_t N, int64_t ldw,
                                const float *d, const float *codebook, int L, int k, int V,
                                int T, uint32_t *bitstream, uint32_t *start_state,
                                float *cost, float *recon, int64_t ldr, void *workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t acs_begin, hipEvent_t acs_end) {
    return encode_impl("tcq_encode_timed", W, M, N, ldw, d, codebook, L, k, V, T, bitstream,
                       start_state, cost, recon, ldr, workspace, workspace_bytes, stream,
                       acs_begin, acs_end);
}

extern "C" size_t tcq_l16_stream_probe_bytes(int64_t blocks) {
    return blocks > 0 ? l16_stream_probe_bytes(blocks) : 0;
}

extern "C" int tcq_l16_stream_probe(int64_t blocks, int super_steps, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t start, hipEvent_t stop) {
    clear_error();
    const char *fn = "tcq_l16_stream_probe";
    if (blocks < 1 || blocks > 0x7FFFFFFF || super_steps < 1) {
        set_error("%s: blocks=%lld and super_steps=%d must be positive (blocks < 2^31)", fn,
                  (long long)blocks, super_steps);
        return TCQ_EINVAL;
    }
    if (!workspace || workspace_bytes < l16_stream_probe_bytes(blocks)) {
        set_error("%s: workspace of %zu bytes is below %zu", fn,
                  workspace ? workspace_bytes : size_t{0}, l16_stream_probe_bytes(blocks));
        return TCQ_EINVAL;
    }
    const int rc = check_workspace_alignment(fn, workspace);
    if (rc != TCQ_OK) return rc;
    hipError_t e = hipSuccess;
    if (start) e = hipEventRecord(start, stream);
    if (e == hipSuccess)
        e = launch_l16_stream_probe(blocks, super_steps, static_cast<char *>(workspace), stream);
    if (e == hipSuccess && stop) e = hipEventRecord(stop, stream);
    if (e != hipSuccess) return hip_fail(fn, "probe launch", e);
    return TCQ_OK;
}

extern "C" int tcq_decode(const uint32_t *bitstream, const uint32_t *start_state,
                          const float *codebook, int64_t M, int64_t N, int L, int k, int V,
                          int T, float *out, int64_t ldo, hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_decode";
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (M == 0 || N == 0) return TCQ_OK;
    if (!bitstream || !start_state || !codebook || !out) {
        set_error("%s: bitstream, start_state, codebook and out must be non-NULL", fn);
        return TCQ_EINVAL;
    }
    if (ldo < N) {
        set_error("%s: ldo=%lld < N=%lld", fn, (long long)ldo, (long long)N);
        return TCQ_EINVAL;
    }
    hipError_t e = launch_decode(bitstream, start_state, codebook, M, N, L, k, V, T, out, ldo,
                                 stream);
    if (e != hipSuccess) return hip_fail(fn, "decode launch", e);
    return TCQ_OK;
}

extern "C" int tcq_decode_gemv(const uint32_t *bitstream, const uint32_t *start_state,
                               const float *codebook, int64_t M, int64_t N, int L, int k,
                               int V, int T, const float *x, float *y, hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_decode_gemv";
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (M == 0) return TCQ_OK;
    if (!y || (N > 0 && (!bitstream || !start_state || !codebook || !x))) {
        set_error("%s: bitstream, start_state, codebook, x and y must be non-NULL", fn);
        return TCQ_EINVAL;
    }
    if (M > 0x7FFFFFFF || N / V > 0x7FFFFFFF) {
        set_error("%s: M=%lld, N=%lld exceed one launch (at most 2^31-1 rows and 2^31-1 "
                  "trellis steps per row)", fn, (long long)M, (long long)N);
        return TCQ_EUNSUPPORTED;
    }
    hipError_t e = launch_decode_gemv(bitstream, start_state, codebook, x, y, M, N, L, k, V, T,
                                      stream);
    if (e != hipSuccess) return hip_fail(fn, "decode-GEMV launch", e);
    return TCQ_OK;
}

// Error feedback (LDLQ) driver: workspace layout
//   [targets M x N, unless the caller passes `target`]
//   [reconstruction slice M x T, unless the caller passes `recon`]
//   [slice bitstreams M x nwords][slice start states M][slice costs M]
//   [encoder workspace for an M x T problem: the rest]
namespace {
struct LdlqLayout {
    size_t tgt, rh, sbits, sstart, scost, enc;  // byte offsets
    size_t fixed;                               // bytes before the encoder workspace
};

LdlqLayout ldlq_layout(int64_t M, int64_t N, int k, int T, bool own_tgt, bool own_rh) {
    LdlqLayout l{};
    const size_t nw = (static_cast<size_t>(k) * T + 31) / 32;
    size_t off = 0;
    l.tgt = off;
    if (own_tgt) off += align_up(static_cast<size_t>(M) * N * sizeof(float), 256);
    l.rh = off;
    if (own_rh) off += align_up(static_cast<size_t>(M) * T * sizeof(float), 256);
    l.sbits = off;
    off += align_up(static_cast<size_t>(M) * nw * sizeof(uint32_t), 256);
    l.sstart = off;
    off += align_up(static_cast<size_t>(M) * sizeof(uint32_t), 256);
    l.scost = off;
    off += align_up(static_cast<size_t>(M) * sizeof(float), 256);
    l.enc = off;
    l.fixed = off;
    return l;
}
}  // namespace

extern "C" int tcq_ldlq_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                                        size_t *bytes) {
    clear_error();
    const char *fn = "tcq_ldlq_workspace_bytes";
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!bytes) {
        set_error("%s: bytes is NULL", fn);
        return TCQ_EINVAL;
    }
    if (M == 0 || N == 0) {
        *bytes = 0;
        return TCQ_OK;
    }
    size_t enc = 0;
    rc = tcq_encode_workspace_bytes(M, T, L, k, V, T, &enc);
    if (rc != TCQ_OK) return rc;
    *bytes = ldlq_layout(M, N, k, T, true, true).fixed + enc;
    return TCQ_OK;
}

extern "C" int tcq_encode_ldlq(const float *W, int64_t M, int64_t N, int64_t ldw,
                               const float *U, int64_t ldu, const float *d,
                               const float *codebook, int L, int k, int V, int T,
                               uint32_t *bitstream, uint32_t *start_state, float *cost,
                               float *recon, int64_t ldr, float *target, int64_t ldt,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_encode_ldlq";
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (M == 0 || N == 0) return TCQ_OK;
    const int64_t nbpr = N / T;
    if (!W || !codebook || !bitstream || !start_state || !cost || (nbpr > 1 && !U)) {
        set_error("%s: W, codebook, bitstream, start_state, cost and (for N > T) U must be "
                  "non-NULL", fn);
        return TCQ_EINVAL;
    }
    if (ldw < N || (nbpr > 1 && ldu < N) || (recon && ldr < N) || (target && ldt < N)) {
        set_error("%s: leading dimensions must be >= N=%lld (ldw=%lld ldu=%lld ldr=%lld "
                  "ldt=%lld)", fn, (long long)N, (long long)ldw, (long long)ldu,
                  (long long)ldr, (long long)ldt);
        return TCQ_EINVAL;
    }
    const LdlqLayout lay = ldlq_layout(M, N, k, T, target == nullptr, recon == nullptr);
    size_t enc_min = 0;
    rc = tcq_encode_workspace_min_bytes(L, k, V, T, &enc_min);
    if (rc != TCQ_OK) return rc;
    clear_error();
    if (!workspace || workspace_bytes < lay.fixed + enc_min) {
        set_error("%s: workspace of %zu bytes is below the minimum %zu", fn,
                  workspace ? workspace_bytes : size_t{0}, lay.fixed + enc_min);
        return TCQ_EWORKSPACE;
    }
    rc = check_workspace_alignment(fn, workspace);
    if (rc != TCQ_OK) return rc;
    char *ws = static_cast<char *>(workspace);
    float *tgt = target ? target : reinterpret_cast<float *>(ws + lay.tgt);
    const int64_t lt = target ? ldt : N;
    uint32_t *sbits = reinterpret_cast<uint32_t *>(ws + lay.sbits);
    uint32_t *sstart = reinterpret_cast<uint32_t *>(ws + lay.sstart);
    float *scost = reinterpret_cast<float *>(ws + lay.scost);
    const int nw = (k * T + 31) / 32;

    hipError_t e = hipMemcpy2DAsync(tgt, static_cast<size_t>(lt) * sizeof(float), W,
                                    static_cast<size_t>(ldw) * sizeof(float),
                                    static_cast<size_t>(N) * sizeof(float),
                                    static_cast<size_t>(M), hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(fn, "target copy", e);
    for (int64_t j = 0; j < nbpr; ++j) {
        const int64_t c0 = j * T;
        float *rh = recon ? recon + c0 : reinterpret_cast<float *>(ws + lay.rh);
        const int64_t ldh = recon ? ldr : T;
        rc = encode_impl(fn, tgt + c0, M, T, lt, d ? d + c0 : nullptr, codebook, L, k, V, T,
                         sbits, sstart, scost, rh, ldh, ws + lay.enc,
                         workspace_bytes - lay.enc, stream, nullptr, nullptr);
        if (rc != TCQ_OK) return rc;
        e = launch_ldlq_scatter(sbits, sstart, scost, M, nw, nbpr, j, bitstream, start_state,
                                cost, stream);
        if (e != hipSuccess) return hip_fail(fn, "slice scatter launch", e);
        if (j + 1 < nbpr) {
            e = launch_ldlq_update(tgt, lt, W, ldw, rh, ldh, U, ldu, M, c0 + T, N, c0, T,
                                   stream);
            if (e != hipSuccess) return hip_fail(fn, "feedback update launch", e);
        }
    }
    return TCQ_OK;
}

// Soft trellis (BCJR): workspace = per-block forward vectors for a batch of blocks.
namespace {
constexpr int64_t kBcjrRecommendedBytes = int64_t{8} << 30;

int check_bcjr(const char *fn, int64_t M, int64_t N, int L, int k, int V, int T) {
    int rc = check_trellis(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!bcjr_supported(L, k * V)) {
        set_error("%s: the soft trellis supports k*V <= %d (k=%d V=%d)", fn, kBcjrMaxKV, k, V);
        return TCQ_EUNSUPPORTED;
    }
    return TCQ_OK;
}
}  // namespace

extern "C" int tcq_bcjr_workspace_bytes(int64_t M, int64_t N, int L, int k, int V, int T,
                                        size_t *bytes) {
    clear_error();
    const char *fn = "tcq_bcjr_workspace_bytes";
    int rc = check_bcjr(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!bytes) {
        set_error("%s: bytes is NULL", fn);
        return TCQ_EINVAL;
    }
    const size_t per = bcjr_per_block_bytes(L, k * V, T / V);
    const int64_t nblocks = (T > 0 && N > 0) ? M * (N / T) : 0;
    int64_t batch = kBcjrRecommendedBytes / static_cast<int64_t>(per);
    if (batch > nblocks) batch = nblocks;
    if (batch < 1) batch = 1;
    *bytes = per * static_cast<size_t>(batch);
    return TCQ_OK;
}

extern "C" int tcq_bcjr(const float *W, int64_t M, int64_t N, int64_t ldw, const float *d,
                        const float *codebook, int L, int k, int V, int T, float tau,
                        float *soft, int64_t ldo, float *logz, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_bcjr";
    int rc = check_bcjr(fn, M, N, L, k, V, T);
    if (rc != TCQ_OK) return rc;
    if (!(tau > 0.0f) || !std::isfinite(tau) ||
        !std::isfinite(static_cast<float>(-1.4426950408889634074 / static_cast<double>(tau)))) {
        set_error("%s: tau=%g must be positive, finite and not below 1e-38", fn, (double)tau);
        return TCQ_EINVAL;
    }
    if (M == 0 || N == 0) return TCQ_OK;
    if (!W || !codebook || !soft) {
        set_error("%s: W, codebook and soft must be non-NULL", fn);
        return TCQ_EINVAL;
    }
    if (ldw < N || ldo < N) {
        set_error("%s: ldw=%lld and ldo=%lld must be >= N=%lld", fn, (long long)ldw,
                  (long long)ldo, (long long)N);
        return TCQ_EINVAL;
    }
    const size_t per = bcjr_per_block_bytes(L, k * V, T / V);
    if (!workspace || workspace_bytes < per) {
        set_error("%s: workspace of %zu bytes is below the minimum %zu", fn,
                  workspace ? workspace_bytes : size_t{0}, per);
        return TCQ_EWORKSPACE;
    }
    rc = check_workspace_alignment(fn, workspace);
    if (rc != TCQ_OK) return rc;
    const int64_t bpr = N / T;
    const int64_t nblocks = M * bpr;
    int64_t batch = static_cast<int64_t>(workspace_bytes / per);
    if (batch > nblocks) batch = nblocks;
    if (batch > 0x7FFFFFFF) batch = 0x7FFFFFFF;
    for (int64_t b0 = 0; b0 < nblocks; b0 += batch) {
        const int64_t nb = (nblocks - b0 < batch) ? nblocks - b0 : batch;
        hipError_t e = launch_bcjr(W, ldw, d, codebook, L, k, V, T, bpr, b0, nb, tau,
                                   static_cast<char *>(workspace), soft, ldo, logz, stream);
        if (e != hipSuccess) return hip_fail(fn, "soft-trellis launch", e);
    }
    return TCQ_OK;
}

extern "C" int tcq_hadamard(const float *X, int64_t rows, int64_t len, int64_t ldx, int64_t n,
                            const float *sigma, int inverse, float *Y, int64_t ldy,
                            hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_hadamard";
    if (rows < 0 || len < 0 || n < 1 || (n & (n - 1)) != 0) {
        set_error("%s: rows=%lld, len=%lld must be >= 0 and n=%lld a power of two", fn,
                  (long long)rows, (long long)len, (long long)n);
        return TCQ_EINVAL;
    }
    if (len % n != 0) {
        set_error("%s: len=%lld is not a multiple of n=%lld", fn, (long long)len, (long long)n);
        return TCQ_EINVAL;
    }
    if (n > kHadamardMaxN || (n < 64 && len > kHadamardSmallMaxLen)) {
        set_error("%s: n=%lld above %lld, or len=%lld above %lld with n < 64", fn,
                  (long long)n, (long long)kHadamardMaxN, (long long)len,
                  (long long)kHadamardSmallMaxLen);
        return TCQ_EUNSUPPORTED;
    }
    if (rows == 0 || len == 0) return TCQ_OK;
    if (!X || !Y || ldx < len || ldy < len) {
        set_error("%s: X and Y must be non-NULL with ldx, ldy >= len", fn);
        return TCQ_EINVAL;
    }
    if (X != Y && ((X < Y + rows * ldy) && (Y < X + rows * ldx))) {
        set_error("%s: X and Y overlap without being the same buffer", fn);
        return TCQ_EINVAL;
    }
    if (X == Y && ldx != ldy) {
        set_error("%s: in place needs ldx == ldy", fn);
        return TCQ_EINVAL;
    }
    hipError_t e = launch_hadamard(X, ldx, Y, ldy, rows, len, n, sigma, inverse ? 1 : 0, stream);
    if (e != hipSuccess) return hip_fail(fn, "Hadamard launch", e);
    return TCQ_OK;
}

extern "C" int tcq_scale_field_workspace_bytes(int64_t M, int64_t N, size_t *bytes) {
    clear_error();
    if (M < 0 || N < 0 || !bytes) {
        set_error("tcq_scale_field_workspace_bytes: negative size or NULL bytes");
        return TCQ_EINVAL;
    }
    *bytes = scale_field_slabs(M) * static_cast<size_t>(N) * sizeof(float);
    return TCQ_OK;
}

extern "C" int tcq_scale_field(const float *W, int64_t M, int64_t N, int64_t ldw,
                               float *row_scale, float *col_scale, float *Wn, int64_t ldn,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    const char *fn = "tcq_scale_field";
    if (M < 0 || N < 0) {
        set_error("%s: negative size", fn);
        return TCQ_EINVAL;
    }
    if (M == 0 || N == 0) return TCQ_OK;
    if (!W || !row_scale || !col_scale || ldw < N || (Wn && ldn < N)) {
        set_error("%s: W, row_scale, col_scale must be non-NULL, ldw >= N, ldn >= N", fn);
        return TCQ_EINVAL;
    }
    if (M > 0x7FFFFFFF) {
        set_error("%s: M=%lld rows exceed one launch", fn, (long long)M);
        return TCQ_EUNSUPPORTED;
    }
    const size_t need = scale_field_slabs(M) * static_cast<size_t>(N) * sizeof(float);
    if (!workspace || workspace_bytes < need) {
        set_error("%s: workspace of %zu bytes is below %zu", fn,
                  workspace ? workspace_bytes : size_t{0}, need);
        return TCQ_EWORKSPACE;
    }
    const int rc = check_workspace_alignment(fn, workspace);
    if (rc != TCQ_OK) return rc;
    hipError_t e = launch_scale_field(W, ldw, M, N, row_scale, col_scale, Wn, ldn,
                                      static_cast<float *>(workspace), stream);
    if (e != hipSuccess) return hip_fail(fn, "scale-field launch", e);
    return TCQ_OK;
}
