// tcq_encode_noalloc: tcq_encode for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
// workspace is a file-scope device array that every GPU the library runs on holds until
// the process ends; the caller passes only the inputs and outputs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tcq.h"
#include "tcq_internal.h"

namespace {

// The array lives in device memory of every GPU that loads this code object.  In host
// code its name is only a host-side stand-in: the device address of each GPU's copy comes
// from hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[TCQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void *ptr = nullptr;
    bool done = false;
    hipError_t err = hipSuccess;
};

std::mutex g_mu;
DeviceScratch g_scratch[kMaxDevices];

// Address of the current device's copy of `scratch` (resolved on the first call made on
// that device), or nullptr with the HIP error in *err.
void *scratch_ptr(hipError_t *err) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &s = g_scratch[dev];
    if (!s.done) {
        void *p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        s.ptr = s.err == hipSuccess ? p : nullptr;
        s.done = true;
    }
    *err = s.err;
    return s.ptr;
}

}  // namespace

extern "C" int tcq_encode_noalloc(const float *W, int64_t M, int64_t N, int64_t ldw,
                                  const float *d, const float *codebook, int L, int k, int V,
                                  int T, uint32_t *bitstream, uint32_t *start_state,
                                  float *cost, float *recon, int64_t ldr,
                                  hipStream_t stream) {
    const char *fn = "tcq_encode_noalloc";
    hipError_t e = hipSuccess;
    void *ws = scratch_ptr(&e);
    if (!ws) {
        tcq::set_error("%s: hipGetSymbolAddress of the scratch array failed: %s", fn,
                       hipGetErrorString(e));
        return TCQ_EHIP;
    }
    // The scratch is the workspace of tcq_encode: blocks are encoded in batches that fit
    // it.  Every byte the kernels read from it is written earlier in the same call (codebook
    // copies, backpointers, end states, cost vectors), so nothing is cleared first.
    const int rc = tcq::encode_impl(fn, W, M, N, ldw, d, codebook, L, k, V, T, bitstream,
                                    start_state, cost, recon, ldr, ws,
                                    TCQ_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
    if (rc == TCQ_EWORKSPACE) {
        // a single coding block of this shape needs more than the scratch holds
        tcq::set_error("%s: one coding block of this shape (L=%d k=%d V=%d T=%d) needs more "
                       "than the %llu bytes of scratch the library holds per GPU",
                       fn, L, k, V, T,
                       static_cast<unsigned long long>(TCQ_NOALLOC_SCRATCH_BYTES));
        return TCQ_EUNSUPPORTED;
    }
    return rc;
}
