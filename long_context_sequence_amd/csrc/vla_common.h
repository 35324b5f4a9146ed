// vla_common.h -- internal declarations shared by the library's HIP sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vla.h"

namespace vla {

// Launch arguments after the C-ABI checks (see include/vla.h for meaning).
struct FwdArgs {
    const void *q, *k, *v, *u;
    int dtype;            // 0 = fp32, 1 = bf16
    int B, H, T, d;
    float lambda0, eps;
    float *o, *S_out, *A_out, *zk_out;
    const float *S0, *A0, *zk0;
    hipStream_t stream;
    void *ws;             // workspace of the two-pass forward (device memory)
    size_t ws_bytes;
    // two-pass forward only: when set, the per-token quantities the gradients
    // need ((4 d + 8) floats per token and head, see vla_bwd.h) go here too
    float *keep = nullptr;
};

// Input widening: fp32 as is, bf16 (stored as its 16 bit pattern) exactly.
__device__ __forceinline__ float load_in(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t *p, size_t i)
{
    return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// phi = ELU + 1 (ELU with alpha = 1): x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }

hipError_t launch_forward_ref(const FwdArgs &a);

// every argument check of vla_forward except the workspace's (vla_abi.hip)
vla_status check_forward(const void *q, const void *k, const void *v, const void *u, int in_dtype,
                         int B, int H, int T, int d_h, float lambda0, float eps, const float *o,
                         const float *S_out, const float *A_out, const float *zkey_out,
                         const float *S0, const float *A0, const float *zkey0);

// T = 0: the initial state (given, or the defaults) to the requested outputs
hipError_t launch_state_init(const FwdArgs &a);

// Chunked matrix-core kernels (d_h in {64, 96, 128}).
bool chunk_supported(int d);
// one decode token, state in place (a.T == 1; S_out, A_out, zk_out are the state)
hipError_t launch_step(const FwdArgs &a);
// two passes over the sequence (forward, T >= 1); needs the workspace below.
// phases: 1 = penalty pass (Grams, segment inverses, penalty chain and the
// per-chunk factors in the workspace), 2 = memory pass, 3 = both.
size_t twopass_workspace_bytes(int BH, int T, int d);
// whether every per-head buffer of the forward (and, with keep, of the
// gradients' per-token records) stays below 2^31 bytes at this T
bool twopass_size_ok(int T, int d, bool keep);
// byte offset of the per-chunk records (vla_record.h) in that workspace; the
// record of chunk c of head bh is at index bh * ceil(T / 16) + c
size_t twopass_records_offset(int BH, int T, int d);
hipError_t launch_forward_twopass(const FwdArgs &a, int phases);
// the memory pass alone, on per-chunk records at rec laid out as the penalty
// pass leaves them (vla_record.h); lin: records with k^ = 0 and (I + N)^-1 = I
// (linear attention), whose errors are the values themselves
hipError_t launch_memory_pass(const FwdArgs &a, const float *rec, bool lin);
// the baselines (vla_baseline.hip): records from the inputs, then the memory pass
size_t baseline_workspace_bytes(int BH, int T, int d);
hipError_t launch_baseline(const FwdArgs &a, bool delta, float beta);
// the memory chain as a scan over chunks (d_h = 64, T >= 1): the penalty pass,
// then per-chunk affine maps of S, a work-efficient scan of them and the
// chunk-local readout; needs the workspace below.
bool scan_supported(int d);   // d_h in {64, 96, 128}
size_t scan_workspace_bytes(int BH, int T, int d);
hipError_t launch_forward_scan(const FwdArgs &a);

}  // namespace vla
