// vla_chunk_kernel.hip -- chunked matrix-core kernels of the VLA recurrence for
// d_h in {64, 96, 128}: the blocked chains of vla_chunk_parts.h arranged in time.
//
// Source: "Variational Linear Attention" (arXiv 2605.11196), section 3.3,
// Eqs. (9)-(11); A_0 = I / lambda0 (section 3.2).
//
// Two arrangements of the same arithmetic:
//
// split (selected with the environment variable VLA_SPLIT=1, when every
//   workgroup of the launch can be resident at once): two
//   workgroups per head on two compute units, one per chain.  The penalty chain
//   hands W' and the |w|^2 partials of each chunk to the memory chain through a
//   ring of RING chunk slots per head in device memory, with two counters per
//   head (chunks produced, chunks consumed) written with agent-scope
//   release/acquire.  The launch is cooperative, so all workgroups are resident
//   and every wait ends; a bounded spin is kept as a guard all the same.
//     penalty workgroup, chunk p:  [wait until slot p%RING is free]  Z0,
//        Grams; wait for this wave's stores of chunk p-1 | barrier | publish
//        chunks < p; peek the consumed counter; stage chunk p+1, prefetch p+2;
//        factorise, update A, W' -> ring slot | barrier.
//     memory workgroup, chunk q:   publish consumed q+1 (its slot is in LDS);
//        counter peek; S K^, S Phi, key-sum prefix | barrier | 1/|w|, Grams,
//        readout denominators, wait until chunk q+1 is published | barrier |
//        loads of slot q+1, stage q+1, prefetch q+2; (I+N)^-1, E, readout,
//        update S; loads of V of q+1; slot q+1 -> LDS | barrier.
//   Every wait on device memory finds its operations a segment old or more.
//
// fused (any grid size): one workgroup per head with both chains, NA waves
//   each, so every SIMD holds a wave of each chain.  Period p has two segments
//   separated by LDS barriers:
//     segment 1:  penalty waves: Z0, Y0, Grams of chunk p; key-sum prefix of
//                                chunk p.
//                 memory waves:  S K^, S Phi, 1/|w|, Grams of chunk p-1.
//     segment 2:  penalty waves: factorise, update A, W of chunk p (into LDS).
//                 memory waves:  (I+N)^-1, E, readout, update S for chunk p-1;
//                                readout denominators of chunk p; staging of p+1.
#include <mutex>
#include <stdlib.h>
#include <string.h>

#include "vla_chunk_parts.h"

namespace vla {
namespace {

using namespace chunk;

constexpr int RING = 8;   // chunk slots per head between the two chains (power of 2)

// ---------------------------------------------------------------- fused kernel
template <int D, typename Tin>
__global__ void __launch_bounds__(128 * Cfg<D>::NA)
vla_fwd_fused(const Tin *__restrict__ q, const Tin *__restrict__ k,
              const Tin *__restrict__ v, const Tin *__restrict__ u,
              int T, float lambda0, float eps,
              float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
              const float *S0, const float *A0, const float *zk0)
{
    using Hd = Head<D, Tin>;
    constexpr int NA = Cfg<D>::NA, BPW = Cfg<D>::BPW, C = Cfg<D>::C;
    __shared__ __align__(16) Lds<D> L;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const bool awave = w < NA;
    const size_t bh = blockIdx.x;
    const size_t DD = (size_t)D * D;
    const int NC = (T + C - 1) / C;

    // memory waves stage the inputs; penalty-wave threads 0..D-1 own the key sums
    Hd hd(L, q, k, v, u, o, T, eps, bh, tid & 63, awave ? w : w - NA, tid - 64 * NA, !awave,
          awave ? tid : -1);
    typename Hd::State st;
    if (hd.kcol >= 0 && zk0) hd.zk_run = zk0[bh * D + hd.kcol];
    if (awave) {
        hd.load_state(st, A0 ? A0 + bh * DD : nullptr, 1.f / lambda0);
    } else {
        hd.load_state(st, S0 ? S0 + bh * DD : nullptr, 0.f);
        if (NC > 0) {
            hd.template prefetch<true, true>(0);
            hd.template stage1<true, true>(0);
            hd.template prefetch<true, true>(1);
        }
    }
    vmem_drain();
    __syncthreads();

    if (awave) {
        WToLds<D> wl{L, 0, hd.g, hd.n};
        for (int p = 0; p <= NC; ++p) {
            hd.pp = p;
            VLA_PROBE(p, 0);
            if (p < NC) {
                hd.a_products(st, p);
                hd.stage2();
            }
            VLA_PROBE(p, 1);
            lds_barrier();
            VLA_PROBE(p, 2);
            if (p < NC) {
                wl.sp = p & 1;
                hd.a_update(st, p, wl);
            }
            VLA_PROBE(p, 3);
            lds_barrier();
        }
    } else {
        f4 sk[BPW], sq[BPW], invn4 = {0.f, 0.f, 0.f, 0.f};
        Raw1<Tin> vraw[BPW][4];
        for (int p = 0; p <= NC; ++p) {
            const int cq = p - 1;   // chunk of this period's memory-chain work
            hd.pp = p;
            VLA_PROBE(p, 0);
            if (p >= 1) {
                hd.s_products(st, cq, sk, sq);
                hd.s_grams(cq, invn4);
            }
            VLA_PROBE(p, 1);
            lds_barrier();
            VLA_PROBE(p, 2);
            if (p >= 1) hd.s_update(st, cq, sk, sq, invn4, vraw, L.wt[cq & 1]);
            VLA_PROBE(p, 10);
            if (p < NC) {
                hd.stage3(p);
                hd.load_v(p, vraw);   // used in the next period
            }
            if (p + 1 < NC) {
                hd.template stage1<true, true>(p + 1);
                hd.template prefetch<true, true>(p + 2);
            }
            VLA_PROBE(p, 3);
            lds_barrier();
        }
    }

    float *const out = awave ? A_out : S_out;
    if (out) hd.store_state(st, out + bh * DD);
    if (hd.kcol >= 0 && zk_out) zk_out[bh * D + hd.kcol] = hd.zk_run;
    VLA_PROBE_FLUSH();
}

// ---------------------------------------------------------------- split kernel
// Counter waits and posts between the two workgroups of a head (agent scope:
// the two may sit on different XCDs with separate L2 caches).  A wait gives up
// after about a million polls; once one has given up (only possible if the two
// workgroups were not resident together), the workgroup stops waiting, so the
// launch still ends.
__device__ __forceinline__ uint64_t peek(const uint64_t *flag)
{
    return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// `seen` is an earlier peek of the counter (issued ahead so that its latency is
// hidden); polls again only if it was not yet enough.
__device__ __forceinline__ void wait_from(const uint64_t *flag, uint64_t want, uint64_t seen,
                                          bool &alive)
{
    if (alive && seen < want) {
        int it = 0;
        while (peek(flag) < want) {
            if (++it == (1 << 20)) {
                alive = false;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void wait_at_least(const uint64_t *flag, uint64_t want, bool &alive)
{
    wait_from(flag, want, 0, alive);
}
__device__ __forceinline__ void post(uint64_t *flag, uint64_t val)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void post_relaxed(uint64_t *flag, uint64_t val)
{
    __hip_atomic_store(flag, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups [0, BHp) run penalty chains, [BHp, 2 BHp) memory chains; head h
// uses workgroups h and BHp + h (BHp = BH rounded up to a multiple of 8, so
// both sit on the same XCD under round-robin placement; correctness does not
// depend on it).  Counters of head h: flags[32 h] (produced), flags[32 h + 16]
// (consumed), tagged with the launch epoch in the high 32 bits.
template <int D, typename Tin>
__global__ void __launch_bounds__(64 * Cfg<D>::NA)
vla_fwd_split(const Tin *__restrict__ q, const Tin *__restrict__ k,
              const Tin *__restrict__ v, const Tin *__restrict__ u,
              int BH, int BHp, int T, float lambda0, float eps,
              float *__restrict__ o, float *S_out, float *A_out, float *zk_out,
              const float *S0, const float *A0, const float *zk0,
              float *ring, uint64_t *flags, uint64_t epoch)
{
    using Hd = Head<D, Tin>;
    constexpr int BPW = Cfg<D>::BPW, C = Cfg<D>::C, WSLOT = Cfg<D>::WSLOT, LT = Cfg<D>::LT;
    constexpr int LD = Cfg<D>::LD, NA = Cfg<D>::NA;
    __shared__ __align__(16) Lds<D> L;

    const bool achain = (int)blockIdx.x < BHp;
    const int head = achain ? blockIdx.x : blockIdx.x - BHp;
    if (head >= BH) return;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t DD = (size_t)D * D;
    const int NC = (T + C - 1) / C;
    float *const ringh = ring + (size_t)head * RING * WSLOT;
    uint64_t *const produced = flags + (size_t)head * 32;
    uint64_t *const consumed = produced + 16;
    const uint64_t tag = epoch << 32;
    bool alive = true;   // waits of thread 0 still honoured

    Hd hd(L, q, k, v, u, o, T, eps, head, tid & 63, w, tid, true, achain ? -1 : tid);
    typename Hd::State st;

    if (achain) {
        hd.load_state(st, A0 ? A0 + head * DD : nullptr, 1.f / lambda0);
        if (NC > 0) {
            hd.template prefetch<false, true>(0);
            hd.template stage1<false, true>(0);
            hd.template prefetch<false, true>(1);
        }
        vmem_drain();
        __syncthreads();
        uint64_t seen_c = 0;   // consumed counter peeked one segment ahead (thread 0)
        for (int p = 0; p < NC; ++p) {
            hd.pp = p;
            VLA_PROBE(p, 0);
            if (tid == 0 && p >= RING) wait_from(consumed, tag | (uint64_t)(p - RING + 1), seen_c, alive);
            VLA_PROBE(p, 10);
            hd.a_products(st, p);
            VLA_PROBE(p, 11);
            // this wave's slot stores of chunk p-1 (the youngest of its memory
            // operations, issued a segment ago) are done
            vmem_drain();
            VLA_PROBE(p, 1);
            lds_barrier();
            if (tid == 0 && p > 0) post(produced, tag | (uint64_t)p);
            VLA_PROBE(p, 2);
            if (tid == 0) seen_c = peek(consumed);
            if (p + 1 < NC) hd.template stage1<false, true>(p + 1);
            if (p + 2 < NC) hd.template prefetch<false, true>(p + 2);
            VLA_PROBE(p, 12);
            hd.a_update(st, p, WToGlobal<D>{ringh + (p & (RING - 1)) * WSLOT, hd.g, hd.n});
            VLA_PROBE(p, 3);
            lds_barrier();
        }
        vmem_drain();
        __syncthreads();
        if (tid == 0 && NC > 0) post(produced, tag | (uint64_t)NC);
        if (A_out) hd.store_state(st, A_out + head * DD);
    } else {
        hd.load_state(st, S0 ? S0 + head * DD : nullptr, 0.f);
        if (hd.kcol >= 0 && zk0) hd.zk_run = zk0[head * D + hd.kcol];
        f4 sk[BPW], sq[BPW], invn4 = {0.f, 0.f, 0.f, 0.f};
        Raw1<Tin> vraw[BPW][4];      // V' of the chunk in flight
        // thread tid holds entries e = tid + 64 NA j (j < BPW) of a slot's W' (4 D
        // float4s) and, for tid < 4 NA, one float4 of the |w|^2 partials
        f4 wreg[BPW], nreg = {0.f, 0.f, 0.f, 0.f};
        auto slot_load = [&](int cq) {
            const float *slot = ringh + (cq & (RING - 1)) * WSLOT;
            sfor<BPW>([&](auto j) {
                const int e = tid + 64 * NA * j;
                wreg[j] = ld4(&slot[16 * (e >> 2) + 4 * (e & 3)]);
            });
            if (tid < 4 * NA) nreg = ld4(&slot[16 * D + 4 * tid]);
        };
        // W' [i][token] and the |w|^2 partials of chunk cq from registers into LDS
        auto slot_store = [&](int cq) {
            sfor<BPW>([&](auto j) {
                const int e = tid + 64 * NA * j, i = e >> 2, c4 = 4 * (e & 3);
                st4(&L.wt[cq & 1][i * LT + c4], wreg[j]);
                sfor<4>([&](auto r) { L.w[(c4 + r) * LD + i] = wreg[j][int(r)]; });
            });
            if (tid < 4 * NA) st4(&L.nrm[tid >> 2][4 * (tid & 3)], nreg);
        };
        if (NC > 0) {
            if (tid == 0) wait_at_least(produced, tag | 1u, alive);
            hd.template prefetch<true, false>(0);
            hd.load_v(0, vraw);
            hd.template stage1<true, false>(0);
            hd.template prefetch<true, false>(1);
        }
        __syncthreads();
        if (NC > 0) {
            slot_load(0);
            slot_store(0);
        }
        vmem_drain();
        __syncthreads();
        for (int cq = 0; cq < NC; ++cq) {
            const int sl = cq & 1;
            hd.pp = cq;
            VLA_PROBE(cq, 0);
            // the slot of chunk cq is in LDS since the last barrier
            if (tid == 0) post_relaxed(consumed, tag | (uint64_t)(cq + 1));
            const uint64_t seen = tid == 0 ? peek(produced) : 0;
            VLA_PROBE(cq, 10);
            hd.s_products(st, cq, sk, sq);
            hd.stage2();
            VLA_PROBE(cq, 1);
            lds_barrier();
            VLA_PROBE(cq, 2);
            hd.s_grams(cq, invn4);
            hd.stage3(cq);
            VLA_PROBE(cq, 11);
            if (tid == 0 && cq + 1 < NC) wait_from(produced, tag | (uint64_t)(cq + 2), seen, alive);
            VLA_PROBE(cq, 12);
            lds_barrier();
            VLA_PROBE(cq, 13);
            // loads for the next period first, so that they are old when used
            if (cq + 1 < NC) {
                slot_load(cq + 1);
                hd.template stage1<true, false>(cq + 1);
                hd.template prefetch<true, false>(cq + 2);
            }
            hd.s_update(st, cq, sk, sq, invn4, vraw, L.wt[sl]);
            VLA_PROBE(cq, 14);
            if (cq + 1 < NC) {
                hd.load_v(cq + 1, vraw);
                slot_store(cq + 1);
            }
            VLA_PROBE(cq, 3);
            lds_barrier();
        }
        if (S_out) hd.store_state(st, S_out + head * DD);
        if (hd.kcol >= 0 && zk_out) zk_out[head * D + hd.kcol] = hd.zk_run;
    }
    VLA_PROBE_FLUSH();
}

// ---------------------------------------------------------------- host side
// Per-device ring and counters of the split kernel, grown on demand; the epoch
// makes counters of earlier launches read as "nothing produced yet".
struct SplitScratch {
    float *ring = nullptr;
    uint64_t *flags = nullptr;
    size_t ring_bytes = 0, flag_bytes = 0;
    uint64_t epoch = 0;
};
constexpr int kMaxDevices = 64;
SplitScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t split_scratch(int dev, size_t ring_bytes, size_t flag_bytes, float **ring,
                         uint64_t **flags, uint64_t *epoch)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    SplitScratch &s = g_scratch[dev];
    if (s.ring_bytes < ring_bytes) {
        if (s.ring) (void)hipFree(s.ring);
        s.ring = nullptr;
        s.ring_bytes = 0;
        hipError_t e = hipMalloc(&s.ring, ring_bytes);
        if (e != hipSuccess) return e;
        s.ring_bytes = ring_bytes;
    }
    if (s.flag_bytes < flag_bytes) {
        if (s.flags) (void)hipFree(s.flags);
        s.flags = nullptr;
        s.flag_bytes = 0;
        hipError_t e = hipMalloc(&s.flags, flag_bytes);
        if (e != hipSuccess) return e;
        e = hipMemset(s.flags, 0, flag_bytes);
        if (e != hipSuccess) return e;
        s.flag_bytes = flag_bytes;
        s.epoch = 0;
    }
    *ring = s.ring;
    *flags = s.flags;
    *epoch = ++s.epoch;
    return hipSuccess;
}

// Largest grid of the split kernel that can be resident at once on `dev`, or 0
// when cooperative launches are not available.
template <int D, typename Tin>
int split_capacity(int dev)
{
    static int cache[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(once[dev], [dev] {
        int coop = 0, cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void *>(vla_fwd_split<D, Tin>), 64 * Cfg<D>::NA, 0) !=
                hipSuccess)
            coop = 0;
        // one workgroup per compute unit keeps the two chains of a head apart
        cache[dev] = coop ? cus * (per_cu < 1 ? 0 : 1) : 0;
    });
    return cache[dev];
}

template <int D, typename Tin>
hipError_t launch_chunk(const FwdArgs &a)
{
    const int BH = a.B * a.H;
    const int BHp = (BH + 7) / 8 * 8;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const char *sel = getenv("VLA_SPLIT");
    const bool want_split = sel && strcmp(sel, "1") == 0;
    if (want_split && a.T > 0 && 2 * BHp <= split_capacity<D, Tin>(dev)) {
        float *ring = nullptr;
        uint64_t *flags = nullptr;
        uint64_t epoch = 0;
        e = split_scratch(dev, (size_t)BH * RING * Cfg<D>::WSLOT * sizeof(float),
                          (size_t)BH * 32 * sizeof(uint64_t), &ring, &flags, &epoch);
        if (e != hipSuccess) return e;
        const Tin *q = (const Tin *)a.q, *k = (const Tin *)a.k, *v = (const Tin *)a.v,
                  *u = (const Tin *)a.u;
        int T = a.T;
        float lambda0 = a.lambda0, eps = a.eps;
        float *o = a.o, *S_out = a.S_out, *A_out = a.A_out, *zk_out = a.zk_out;
        const float *S0 = a.S0, *A0 = a.A0, *zk0 = a.zk0;
        int bh = BH, bhp = BHp;
        void *args[] = {&q, &k, &v, &u, &bh, &bhp, &T, &lambda0, &eps, &o, &S_out, &A_out,
                        &zk_out, &S0, &A0, &zk0, &ring, &flags, &epoch};
        return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(vla_fwd_split<D, Tin>),
                                          dim3(2 * BHp), dim3(64 * Cfg<D>::NA), args, 0, a.stream);
    }
    hipLaunchKernelGGL((vla_fwd_fused<D, Tin>), dim3(BH), dim3(128 * Cfg<D>::NA), 0, a.stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.u,
                       a.T, a.lambda0, a.eps, a.o, a.S_out, a.A_out, a.zk_out, a.S0, a.A0, a.zk0);
    return hipGetLastError();
}

}  // namespace

bool chunk_supported(int d) { return d == 64 || d == 96 || d == 128; }

hipError_t launch_forward_chunk(const FwdArgs &a)
{
    const bool bf = a.dtype == 1;
    switch (a.d) {
    case 64: return bf ? launch_chunk<64, uint16_t>(a) : launch_chunk<64, float>(a);
    case 96: return bf ? launch_chunk<96, uint16_t>(a) : launch_chunk<96, float>(a);
    case 128: return bf ? launch_chunk<128, uint16_t>(a) : launch_chunk<128, float>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vla
