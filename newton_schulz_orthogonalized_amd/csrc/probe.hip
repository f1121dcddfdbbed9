// Measured ceilings for the benchmark (not part of the optimizer library):
// a dense bf16 MFMA loop with no memory traffic, timed with HIP events, with
// each wave stamping the shader clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around its loop, so the clock the chip ran
// at during the loop is measured next to the rate it reached.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHR = 256;
constexpr int CHAINS = 16;   // independent accumulators per wave, as in a 4 x 4 fragment block

// Every wave issues iters x CHAINS v_mfma_f32_16x16x32_bf16 on register
// operands (16 * 16 * 32 * 2 flop each). Lane 0 of each wave writes its
// counter deltas and a value depending on every accumulator (vector stores).
__global__ __launch_bounds__(NTHR) void k_mfma_loop(const bf16x8* src, int iters, uint64_t* stamps, float* sink) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (NTHR / 64) + (threadIdx.x >> 6);
    const bf16x8 a = src[lane], b = src[64 + lane];
    f32x4 acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    asm volatile("s_nop 1" ::: "memory");
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < CHAINS; ++j)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (lane == 0) {
        stamps[2 * wave] = c1 - c0;
        stamps[2 * wave + 1] = r1 - r0;
        sink[wave] = s;
    }
}

}  // namespace

extern "C" {

// Runs the loop on every compute unit (four workgroups of four waves each per
// compute unit) for about `target_ms`, after two sizing runs. Outputs: the achieved dense bf16 rate in TFLOP/s, the kernel time in
// ms, and the shader clock in GHz (mean over waves of shader cycles over
// elapsed 100 MHz ticks). Returns 0, or the HIP error code.
int probe_mfma_bf16(double target_ms, double* tflops, double* ms_out, double* clock_ghz) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    // four workgroups per compute unit, so that an uneven placement by the
    // dispatcher cannot leave a compute unit idle for the whole loop
    const int grid = 4 * cus;
    const int waves = grid * (NTHR / 64);
    bf16x8* src = nullptr;
    uint64_t* stamps = nullptr;
    float* sink = nullptr;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    auto cleanup = [&]() {
        if (src) (void)hipFree(src);
        if (stamps) (void)hipFree(stamps);
        if (sink) (void)hipFree(sink);
        if (ev0) (void)hipEventDestroy(ev0);
        if (ev1) (void)hipEventDestroy(ev1);
    };
    bf16x8 host[128];
    for (int i = 0; i < 128; ++i)
        for (int k = 0; k < 8; ++k) host[i][k] = (__bf16)(0.001f * (float)((i * 8 + k) % 7));
    if ((e = hipMalloc(&src, sizeof(host))) != hipSuccess ||
        (e = hipMalloc(&stamps, sizeof(uint64_t) * 2 * waves)) != hipSuccess ||
        (e = hipMalloc(&sink, sizeof(float) * waves)) != hipSuccess ||
        (e = hipMemcpy(src, host, sizeof(host), hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipEventCreate(&ev0)) != hipSuccess || (e = hipEventCreate(&ev1)) != hipSuccess) {
        cleanup();
        return (int)e;
    }
    // size the loop from a short calibration run
    int iters = 2000;
    float ms = 0.f;
    for (int pass = 0; pass < 3; ++pass) {
        (void)hipEventRecord(ev0, 0);
        hipLaunchKernelGGL(k_mfma_loop, dim3(grid), dim3(NTHR), 0, 0, src, iters, stamps, sink);
        (void)hipEventRecord(ev1, 0);
        if ((e = hipEventSynchronize(ev1)) != hipSuccess || (e = hipGetLastError()) != hipSuccess) {
            cleanup();
            return (int)e;
        }
        (void)hipEventElapsedTime(&ms, ev0, ev1);
        if (pass < 2) {
            const double scale = target_ms / (ms > 1e-3f ? ms : 1e-3f);
            const double next = (double)iters * (scale > 64.0 ? 64.0 : scale);
            iters = (int)(next > 2e9 ? 2e9 : (next < 100 ? 100 : next));
        }
    }
    std::vector<uint64_t> st((size_t)2 * waves);
    if ((e = hipMemcpy(st.data(), stamps, sizeof(uint64_t) * 2 * waves, hipMemcpyDeviceToHost)) != hipSuccess) {
        cleanup();
        return (int)e;
    }
    double ghz = 0.0;
    int counted = 0;
    for (int w = 0; w < waves; ++w) {
        if (st[2 * w + 1] == 0) continue;
        ghz += (double)st[2 * w] / ((double)st[2 * w + 1] * 10.0);   // cycles per ns: ticks are 10 ns
        ++counted;
    }
    const double flops = (double)waves * iters * CHAINS * 16.0 * 16.0 * 32.0 * 2.0;
    *tflops = flops / (ms * 1e-3) / 1e12;
    *ms_out = ms;
    *clock_ghz = counted ? ghz / counted : 0.0;
    cleanup();
    return 0;
}

}  // extern "C"
