// Measured ceilings for the roofline figures: what one MI355X sustains for a
// plain streaming read of HBM, a device-to-device copy, and back-to-back bf16
// MFMAs with no memory traffic.  Measurement aids beside the forward library
// (libdec_probe.so, declared in include/dec_probe.h); nothing on the forward
// path calls them.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"
#include "dec_probe.h"

#define DECP_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int PROBE_THREADS = 256;

// One launch reads every 16-byte word once: block b takes the 16 KB at
// [b * 16 KB, (b + 1) * 16 KB), four non-temporal 16-byte loads a thread (lane
// t of the block at words t, t + 256, t + 512, t + 768), as many blocks as
// the buffer holds 16 KB runs (this one-shot form measured 7.3 TB/s where
// grid-stride loops of 2048-32768 blocks read 6.2-6.4).  The block's XOR of
// its words goes to sink[b], which keeps the loads live.
constexpr int READ_WORDS = 4 * PROBE_THREADS;   // 16-byte words a block

__global__ void __launch_bounds__(PROBE_THREADS) stream_read_kernel(const u32x4 *__restrict__ p,
                                                                   uint32_t *__restrict__ sink) {
    __shared__ uint32_t red[PROBE_THREADS / 64];
    const u32x4 *q = p + (size_t)blockIdx.x * READ_WORDS + threadIdx.x;
    u32x4 a[4];
#pragma unroll
    for (int u = 0; u < 4; u++) a[u] = __builtin_nontemporal_load(q + u * PROBE_THREADS);
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) x ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// The same one-shot form for a copy: four 16-byte words a thread.
__global__ void __launch_bounds__(PROBE_THREADS) copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst) {
    const size_t o = (size_t)blockIdx.x * READ_WORDS + threadIdx.x;
    u32x4 a[4];
#pragma unroll
    for (int u = 0; u < 4; u++) a[u] = __builtin_nontemporal_load(src + o + u * PROBE_THREADS);
#pragma unroll
    for (int u = 0; u < 4; u++) dst[o + u * PROBE_THREADS] = a[u];
}

// Four independent 32x32x16 bf16 MFMA chains a wave, `iters` steps each; the
// operands come from the thread index so nothing folds, and each thread's sum
// of its accumulators is stored.
__global__ void __launch_bounds__(PROBE_THREADS) mfma_loop_kernel(int iters, float *__restrict__ sink) {
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        a[j] = (__bf16)(float)((t + j) & 7);
        b[j] = (__bf16)(float)((t * 3 + j) & 7);
    }
    floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j++) s += c0[j] + c1[j] + c2[j] + c3[j];
    sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// hipEvents around `reps` launches on `st` after one untimed launch: mean ms.
template <typename F>
int time_reps(hipStream_t st, int reps, F launch, double *ms) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -1;
    if (hipEventCreate(&e1) != hipSuccess) {
        hipEventDestroy(e0);
        return -1;
    }
    launch();
    hipEventRecord(e0, st);
    for (int r = 0; r < reps; r++) launch();
    hipEventRecord(e1, st);
    int rc = 0;
    float t = 0.f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&t, e0, e1) != hipSuccess)
        rc = -1;
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    *ms = (double)t / reps;
    return rc;
}

}  // namespace

DECP_API int decp_mfma_sink_floats(void) { return DECP_GRID_BLOCKS * PROBE_THREADS; }

DECP_API int decp_stream_read(const void *buf, size_t bytes, void *sink, int reps, void *stream, double *ms) {
    if (!buf || !sink || !ms || reps <= 0 || bytes == 0 || bytes % DECP_RUN_BYTES || (uintptr_t)buf % 16 ||
        bytes / DECP_RUN_BYTES > 0x7FFFFFFFu)
        return -2;
    hipStream_t st = (hipStream_t)stream;
    const unsigned blocks = (unsigned)(bytes / DECP_RUN_BYTES);
    return time_reps(st, reps, [&] {
        hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(PROBE_THREADS), 0, st, (const u32x4 *)buf,
                           (uint32_t *)sink);
    }, ms);
}

DECP_API int decp_copy(const void *src, void *dst, size_t bytes, int reps, void *stream, double *ms) {
    if (!src || !dst || !ms || reps <= 0 || bytes == 0 || bytes % DECP_RUN_BYTES || (uintptr_t)src % 16 ||
        (uintptr_t)dst % 16 || bytes / DECP_RUN_BYTES > 0x7FFFFFFFu)
        return -2;
    hipStream_t st = (hipStream_t)stream;
    const unsigned blocks = (unsigned)(bytes / DECP_RUN_BYTES);
    return time_reps(st, reps, [&] {
        hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(PROBE_THREADS), 0, st, (const u32x4 *)src,
                           (u32x4 *)dst);
    }, ms);
}

DECP_API int decp_mfma_bf16(int iters, void *sink, int reps, void *stream, double *ms, double *flops) {
    if (!sink || !ms || !flops || reps <= 0 || iters <= 0) return -2;
    hipStream_t st = (hipStream_t)stream;
    // per wave: iters x 4 MFMAs of 32 x 32 x 16 (2 flops a product)
    *flops = (double)DECP_GRID_BLOCKS * (PROBE_THREADS / 64) * iters * 4.0 * (2.0 * 32 * 32 * 16);
    return time_reps(st, reps, [&] {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(DECP_GRID_BLOCKS), dim3(PROBE_THREADS), 0, st, iters,
                           (float *)sink);
    }, ms);
}
