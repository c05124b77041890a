// probe_barrier.hip -- measurement aid, not part of the projection library: what a
// device-wide barrier between dependent steps costs on this GPU (libdfssm_probe.so).
//
// A persistent multi-layer decode kernel would replace each kernel boundary between
// dependent projections with such a barrier, so its cost against the dispatch
// interval of back-to-back launches decides whether that design pays.
//
// The probe launches `groups` co-resident workgroups of 512 threads (cooperative
// launch, so every group is resident or the launch fails) for kRounds rounds.  Each
// round: every group writes 64 floats of a shared vector, all groups meet at a
// barrier, then every group reads 2048 floats written by other groups and counts
// mismatches.  The barrier is hierarchical: each group adds 1 to one of eight
// counters (group index mod 8, one 128-byte line each); the last arrival of a
// counter adds 1 to the top counter, which every group polls.
//   fenced = 1: the arrival is preceded by an agent-scope release fence and the wait
//               followed by an agent-scope acquire fence (the memory model's form for
//               plain loads and stores of the shared data);
//   fenced = 0: no fences; the shared data goes through agent-scope relaxed atomic
//               loads and stores, and each writer waits for its stores to complete
//               before it arrives.
// Every wait is bounded: a poll limit ends it with an error flag, and a group that
// timed out skips its later waits, so the kernel always finishes.
//
// Entry point (C, synchronous, allocates and frees its own device memory):
//   int dfssm_probe_grid_barrier_us(int groups, int fenced, double* us)
//     groups: a positive multiple of 8 within the device's co-resident capacity
//     us:     out, microseconds per round (barrier plus the small exchange)
//   returns 0 on success, 1 on bad arguments, 2 on a timeout or a data mismatch,
//   3 on a HIP error (including a cooperative launch the device refuses).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512, kRounds = 2000, kSlot = 64, kReads = 2048, kLine = 32;
constexpr unsigned kPollLimit = 1u << 20;

struct BarState {
    unsigned* count;  // [9 * kLine]: top counter at 0, sub-counter c at kLine * (1 + c)
    int* err;
    int* bad;
    float* v;  // [2][groups * kSlot]
};

__device__ __forceinline__ bool wait_for(unsigned* p, unsigned target, int* err) {
    for (unsigned polls = 0; __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++polls) {
        __builtin_amdgcn_s_sleep(1);
        if (polls > kPollLimit) {
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    return true;
}

template <bool kFenced>
__global__ __launch_bounds__(kThreads) void barrier_kernel(BarState st) {
    const unsigned G = gridDim.x, per = G / 8, cls = blockIdx.x % 8;
    __shared__ int timed_out;
    if (threadIdx.x == 0) timed_out = 0;
    __syncthreads();
    int nbad = 0;
    for (int r = 0; r < kRounds; ++r) {
        float* const buf = st.v + (r & 1) * G * kSlot;
        if (threadIdx.x < kSlot) {
            const float val = (float)(r * 131 + blockIdx.x * kSlot + threadIdx.x);
            if constexpr (kFenced) {
                buf[blockIdx.x * kSlot + threadIdx.x] = val;
            } else {
                __hip_atomic_store(&buf[blockIdx.x * kSlot + threadIdx.x], val, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);  // stores complete before the arrival
            }
        }
        __syncthreads();
        if (threadIdx.x == 0 && !timed_out) {
            if constexpr (kFenced) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const unsigned old = __hip_atomic_fetch_add(st.count + kLine * (1 + cls), 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            if (old == (unsigned)(r + 1) * per - 1)
                __hip_atomic_fetch_add(st.count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!wait_for(st.count, (unsigned)(r + 1) * 8, st.err)) timed_out = 1;
            if constexpr (kFenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        for (int e = threadIdx.x; e < kReads; e += kThreads) {
            const unsigned idx = (blockIdx.x * kSlot + 4096u + 7u * e) % (G * kSlot);
            const float want = (float)(r * 131 + (int)idx);
            const float got = kFenced ? buf[idx]
                                      : __hip_atomic_load(&buf[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nbad += got != want;
        }
    }
    if (nbad) atomicAdd(st.bad, nbad);
}

}  // namespace

extern "C" int dfssm_probe_grid_barrier_us(int groups, int fenced, double* us) {
    if (!us || groups <= 0 || groups % 8 != 0) return 1;
    int dev = 0, cus = 0, per_cu = 0;
    const void* fn = fenced ? (const void*)barrier_kernel<true> : (const void*)barrier_kernel<false>;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess)
        return 3;
    if (groups > cus * per_cu) return 1;
    BarState st{};
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = 3, herr = 0, hbad = 0;
    float ms = 0.0f;
    void* args[] = {&st};
    if (hipMalloc(&st.count, 9 * kLine * sizeof(unsigned)) != hipSuccess) return 3;
    if (hipMalloc(&st.err, sizeof(int)) != hipSuccess || hipMalloc(&st.bad, sizeof(int)) != hipSuccess ||
        hipMalloc(&st.v, 2 * (size_t)groups * kSlot * sizeof(float)) != hipSuccess)
        goto done;
    if (hipMemset(st.count, 0, 9 * kLine * sizeof(unsigned)) != hipSuccess ||
        hipMemset(st.err, 0, sizeof(int)) != hipSuccess || hipMemset(st.bad, 0, sizeof(int)) != hipSuccess)
        goto done;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
    (void)hipEventRecord(e0, 0);
    if (hipLaunchCooperativeKernel(fn, dim3(groups), dim3(kThreads), args, 0, 0) != hipSuccess) goto done;
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess || hipGetLastError() != hipSuccess) goto done;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (hipMemcpy(&herr, st.err, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&hbad, st.bad, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
        goto done;
    *us = (double)ms * 1e3 / kRounds;
    rc = (herr || hbad) ? 2 : 0;
done:
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (st.v) (void)hipFree(st.v);
    if (st.bad) (void)hipFree(st.bad);
    if (st.err) (void)hipFree(st.err);
    (void)hipFree(st.count);
    return rc;
}
