// Internal declarations shared by the sources of libtcq (not part of the ABI).
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace tcq {

// Shape of one encode problem after validation.
struct Problem {
    int L, k, V, T;
    int kv;            // k * V: fresh bits per step
    int n;             // steps per block, T / V
    int64_t M, N;
    int64_t ldw;
    int64_t blocks_per_row;
    int64_t nblocks;
    int64_t ngroups;   // 2^(L - kv)
    int64_t nstates;   // 2^L
};

// Workspace plan for one kernel family: per-block bytes, fixed bytes.
struct Plan {
    int variant;              // see kernels
    size_t per_block;         // bytes per block in flight
    size_t fixed;             // bytes independent of the batch size
    size_t bp_bytes;          // backpointer bytes per block
    size_t cost_bytes;        // global cost-vector bytes per block (0: on chip)
};

enum Variant : int {
    kGenericLds = 0,     // any supported shape, cost vectors double-buffered in LDS
    kGenericGlobal = 1,  // any supported shape, cost vectors in the workspace (L2)
    kL16Regs = 2,        // L = 16, k*V = 2, costs in VGPRs (three-step super-steps)
    kL16RegsK3 = 3,      // L = 16, k*V = 3, costs in VGPRs (two-step super-steps)
    kL16RegsHalf = 4,    // L = 16, k*V = 4 (V = 1, 2), run as 2-bit half-steps in VGPRs
};

Plan plan_for(const Problem &p);

// The encoder behind tcq_encode / tcq_encode_timed (tcq_api.cpp): checks the arguments,
// plans the batches for the given workspace and enqueues every kernel.  `fn` names the
// entry point in error messages.  It allocates nothing.
int encode_impl(const char *fn, const float *W, int64_t M, int64_t N, int64_t ldw,
                const float *d, const float *codebook, int L, int k, int V, int T,
                uint32_t *bitstream, uint32_t *start_state, float *cost, float *recon,
                int64_t ldr, void *workspace, size_t workspace_bytes, hipStream_t stream,
                hipEvent_t acs_begin, hipEvent_t acs_end);

// Per-thread error message of the C ABI (tcq_last_error).
void set_error(const char *fmt, ...);

// Kernel launchers (return hipError_t of the launch).
hipError_t launch_acs_generic(const Problem &p, const Plan &pl, const float *W,
                              const float *d, const float *C, int64_t block0, int64_t nb,
                              char *ws, float *cost, hipStream_t s);
hipError_t launch_traceback_planes(const Problem &p, const Plan &pl, int64_t block0,
                                   int64_t nb, const char *ws, uint32_t *bitstream,
                                   uint32_t *start_state, hipStream_t s);
hipError_t launch_decode(const uint32_t *bitstream, const uint32_t *start_state,
                         const float *C, int64_t M, int64_t N, int L, int k, int V, int T,
                         float *out, int64_t ldo, hipStream_t s);

// Codebook-stream probe of the L = 16 forward kernel (measurement only).
size_t l16_stream_probe_bytes(int64_t blocks);
hipError_t launch_l16_stream_probe(int64_t blocks, int super_steps, char *ws, hipStream_t s);

hipError_t launch_decode_gemv(const uint32_t *bitstream, const uint32_t *start_state,
                              const float *C, const float *x, float *y, int64_t M, int64_t N,
                              int L, int k, int V, int T, hipStream_t s);

// Soft trellis (BCJR).
constexpr int kBcjrMaxKV = 4;                    // 2^kv terms per group kept in registers
constexpr size_t kBcjrLdsBytes = size_t{128} << 10;  // two group vectors in LDS up to this
bool bcjr_supported(int L, int kv);
bool bcjr_in_lds(int L, int kv);
size_t bcjr_per_block_bytes(int L, int kv, int n);
hipError_t launch_bcjr(const float *W, int64_t ldw, const float *d, const float *C, int L, int k,
                       int V, int T, int64_t blocks_per_row, int64_t block0, int64_t nb,
                       float tau, char *ws, float *soft, int64_t ldo, float *logz,
                       hipStream_t s);

// Pre-processing: randomized Hadamard rotation and factored scale field.
constexpr int64_t kHadamardMaxN = 4096;          // longest chunk of the wave kernel
constexpr int64_t kHadamardSmallMaxLen = 8192;   // row length limit when n < 64
hipError_t launch_hadamard(const float *X, int64_t ldx, float *Y, int64_t ldy, int64_t rows,
                           int64_t len, int64_t n, const float *sigma, int inverse,
                           hipStream_t s);
size_t scale_field_slabs(int64_t M);
hipError_t launch_scale_field(const float *W, int64_t ldw, int64_t M, int64_t N, float *a,
                              float *b, float *Wn, int64_t ldn, float *part, hipStream_t s);

// Error feedback over coding blocks.
hipError_t launch_ldlq_update(float *tgt, int64_t ldt, const float *W, int64_t ldw,
                              const float *what, int64_t ldh, const float *U, int64_t ldu,
                              int64_t M, int64_t c_begin, int64_t c_end, int64_t i0, int T,
                              hipStream_t s);
hipError_t launch_ldlq_scatter(const uint32_t *sbits, const uint32_t *sstart,
                               const float *scost, int64_t M, int nwords, int64_t nbpr,
                               int64_t j, uint32_t *bitstream, uint32_t *start_state,
                               float *cost, hipStream_t s);

// L = 16 register-resident path.
bool l16_supported(const Problem &p);
size_t l16_fixed_bytes(const Problem &p);
size_t l16_bp_bytes(const Problem &p);
hipError_t launch_l16_prepare(const Problem &p, const float *C, char *fixed_ws, hipStream_t s);
hipError_t launch_acs_l16(const Problem &p, const Plan &pl, const float *W, const float *d,
                          int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s);
// swap_halves: the k*V = 4 kernel's relabelled trellis (kernels_l16h.hip)
hipError_t launch_traceback_l16(const Problem &p, const Plan &pl, int64_t block0, int64_t nb,
                                const char *ws, uint32_t *bitstream, uint32_t *start_state,
                                hipStream_t s, bool swap_halves = false);

// L = 16, k*V = 4 register-resident path (half-steps).
bool l16h_supported(const Problem &p);
size_t l16h_fixed_bytes(const Problem &p);
size_t l16h_bp_bytes(const Problem &p);
hipError_t launch_l16h_prepare(const Problem &p, const float *C, char *fixed_ws, hipStream_t s);
hipError_t launch_acs_l16h(const Problem &p, const Plan &pl, const float *W, const float *d,
                           int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s);

// L = 16, k*V = 3 register-resident path.
bool l16k3_supported(const Problem &p);
size_t l16k3_fixed_bytes(const Problem &p);
size_t l16k3_bp_bytes(const Problem &p);
hipError_t launch_l16k3_prepare(const Problem &p, const float *C, char *fixed_ws,
                                hipStream_t s);
hipError_t launch_acs_l16k3(const Problem &p, const Plan &pl, const float *W, const float *d,
                            int64_t block0, int64_t nb, char *ws, float *cost, hipStream_t s);
hipError_t launch_traceback_l16k3(const Problem &p, const Plan &pl, int64_t block0, int64_t nb,
                                  const char *ws, uint32_t *bitstream, uint32_t *start_state,
                                  hipStream_t s);

// Workspace layout helpers: [fixed area][per-block area x batch]
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace tcq
