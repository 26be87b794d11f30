// The conditioning vector without a context and without allocating: for
// callers that cannot call hipMalloc (code under HIP graph capture, tight
// serving loops, harnesses that forbid device allocation).
//
// The computation is dit_time_vector's ("gizai:dit" reference: sinusoids and
// the time MLP) with the same kernels; its two intermediate rows -- the
// sinusoid embedding [time_dim] and the time MLP's hidden row [hidden] --
// live in `scratch`, a file-scope device array of fixed size that every
// device holds once for the life of the process.  Its device address is
// looked up once per device (hipGetSymbolAddress, on that device's first
// call) and kept; host code never passes the array's own name to a kernel
// (on the host it is only a stand-in for the symbol, not a device address).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/dit.h"
#include "kernels.h"

namespace {

constexpr int kMaxDim = 4096;                 // time_dim and hidden each at most this
constexpr int kScratchFloats = 2 * kMaxDim;   // [time_dim] embedding, then [hidden] hidden row
constexpr int kMaxDevices = 64;

__device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_mu;
float *g_scratch[kMaxDevices] = {};

dit_status fail_msg(dit_status s, const char *msg) {
    dit_set_global_error(msg);
    return s;
}

// The scratch array's address on `dev` (the current device), looked up on
// the device's first call.
dit_status scratch_of(int dev, float **out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char buf[160];
            snprintf(buf, sizeof buf, "scratch lookup on device %d failed: %s", dev, hipGetErrorString(e));
            return fail_msg(DIT_EDEVICE, buf);
        }
        g_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_scratch[dev];
    return DIT_OK;
}

}  // namespace

extern "C" dit_status dit_time_vector_noalloc(void *stream, int hidden, int time_dim, const uint16_t *w_t1,
                                              const uint16_t *w_t2, float t, float *vec) {
    if (!w_t1 || !w_t2 || !vec) return fail_msg(DIT_EINVAL, "w_t1, w_t2 or vec is NULL");
    if (hidden < 8 || hidden % 8 || hidden > kMaxDim || time_dim < 8 || time_dim % 8 || time_dim > kMaxDim) {
        char buf[160];
        snprintf(buf, sizeof buf, "hidden %d, time_dim %d: each must be a multiple of 8 in 8..%d (the scratch holds %d floats)",
                 hidden, time_dim, kMaxDim, kScratchFloats);
        return fail_msg(DIT_ERANGE, buf);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail_msg(DIT_EDEVICE, "no current HIP device");
    float *base = nullptr;
    const dit_status s = scratch_of(dev, &base);
    if (s != DIT_OK) return s;
    float *temb = base, *hid = base + kMaxDim;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = dit::launch_time_embedding(t, time_dim, temb, st);
    if (e == hipSuccess) e = dit::launch_gemv(w_t1, temb, hidden, time_dim, false, hid, st);
    if (e == hipSuccess) e = dit::launch_gemv(w_t2, hid, hidden, hidden, true, vec, st);
    if (e != hipSuccess) {
        char buf[160];
        snprintf(buf, sizeof buf, "time vector: launch failed: %s", hipGetErrorString(e));
        return fail_msg(DIT_EDEVICE, buf);
    }
    return DIT_OK;
}
