// vla_peak.hip -- attainable FP32 throughput of the device, for the benchmark's
// roofline: the fp32 matrix-core instruction the kernels use
// (v_mfma_f32_16x16x4_f32) and the plain fp32 vector FMA (v_fma_f32; packed FP32
// is disabled in this build, so this is the unpacked rate, half the published
// FP32 vector peak).  Measurement only: not part of libvla's interface.
//
//   int vla_peak_probe(int kind, int iters, double *tflops)
//     kind 0: MFMA fp32, kind 1: VALU fp32 FMA.  Runs one timed launch that
//     fills every compute unit (after one warm-up launch) on the null stream and
//     writes the achieved TFLOP/s.  Returns 0, or -1 on a bad argument or a HIP
//     error.
#include <hip/hip_runtime.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;   // four waves
constexpr int NACC = 8;        // independent accumulators per wave

__global__ void __launch_bounds__(THREADS) mfma_loop(int iters, float seed, float *out)
{
    f4 acc[NACC];
    for (int i = 0; i < NACC; ++i) acc[i] = f4{seed * i, 0.f, 0.f, 0.f};
    const float a = seed + threadIdx.x * 1e-7f, b = seed - threadIdx.x * 1e-7f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < NACC; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    if (s == 1234.5f) out[blockIdx.x * THREADS + threadIdx.x] = s;   // never true; keeps the work
}

__global__ void __launch_bounds__(THREADS) fma_loop(int iters, float seed, float *out)
{
    float x[NACC];
    for (int i = 0; i < NACC; ++i) x[i] = seed + i + threadIdx.x * 1e-7f;
    const float m = 1.f - seed * 1e-9f, c = seed * 1e-9f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int i = 0; i < NACC; ++i) x[i] = fmaf(x[i], m, c);
        }
    }
    float s = 0.f;
    for (int i = 0; i < NACC; ++i) s += x[i];
    if (s == 1234.5f) out[blockIdx.x * THREADS + threadIdx.x] = s;
}

}  // namespace

extern "C" int vla_peak_probe(int kind, int iters, double *tflops)
{
    if ((kind != 0 && kind != 1) || iters < 1 || !tflops) return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    const int blocks = cus * 8;   // two waves per SIMD
    float *out = nullptr;
    if (hipMalloc(&out, (size_t)blocks * THREADS * sizeof(float)) != hipSuccess) return -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = -1;
    if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
        auto launch = [&]() {
            if (kind == 0)
                hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(THREADS), 0, nullptr, iters, 0.5f, out);
            else
                hipLaunchKernelGGL(fma_loop, dim3(blocks), dim3(THREADS), 0, nullptr, iters, 0.5f, out);
        };
        launch();
        float ms = 0.f;
        if (hipGetLastError() == hipSuccess && hipEventRecord(e0, nullptr) == hipSuccess) {
            launch();
            if (hipGetLastError() == hipSuccess && hipEventRecord(e1, nullptr) == hipSuccess &&
                hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
                ms > 0.f) {
                const double per_wave_iter = kind == 0 ? NACC * 16.0 * 16.0 * 4.0 * 2.0   // per MFMA: 2 M N K
                                                       : NACC * 8.0 * 64.0 * 2.0;        // 64 lanes x FMA
                const double flop = per_wave_iter * iters * blocks * (THREADS / 64);
                *tflops = flop / (ms * 1e-3) / 1e12;
                rc = 0;
            }
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(out);
    return rc;
}
