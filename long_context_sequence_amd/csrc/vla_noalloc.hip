// vla_noalloc.hip -- vla_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the forward's workspace is a file-scope device array of fixed
// size instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of the array (VLA_NOALLOC_
// SCRATCH_BYTES) for the life of the process.  Its device address is taken once
// per device with hipGetSymbolAddress, with that device current; host code uses
// only that address (the array's name is a host-side stand-in, not a device
// address).  The call allocates nothing.  The workspace needs no initial
// contents (every value the forward reads from it, it has written in the same
// call), so nothing is cleared.  Calls that overlap in time on one GPU share
// the array and race.
#include <mutex>

#include <stdint.h>

#include "../../include/vla.h"
#include "vla_common.h"

static __device__ __align__(256) unsigned char scratch[VLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES] = {};

// The device address of this device's array (taken on first use), or NULL.
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" vla_status vla_forward_noalloc(const void *q, const void *k, const void *v, const void *u,
                                          vla_dtype in_dtype, int B, int H, int T, int d_h,
                                          float lambda0, float eps,
                                          float *o, float *S_out, float *A_out, float *zkey_out,
                                          const float *S0, const float *A0, const float *zkey0,
                                          void *stream)
{
    // every argument is checked before the runtime is touched
    vla_status st = vla::check_forward(q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps, o, S_out,
                                       A_out, zkey_out, S0, A0, zkey0);
    if (st != VLA_OK) return st;
    size_t need = 0;
    st = vla_forward_workspace_size(B, H, T, d_h, &need);
    if (st != VLA_OK) return st;
    if (need > (size_t)VLA_NOALLOC_SCRATCH_BYTES) return VLA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (!ws) return VLA_ERR_HIP;
    }
    return vla_forward(q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps, o, S_out, A_out, zkey_out,
                       S0, A0, zkey0, ws, need > 0 ? (size_t)VLA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
