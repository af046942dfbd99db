// Sustained dense bf16 matrix-core rate of this GPU, as a yardstick for the
// attention kernels' roofline fraction.
//
// A stream of independent v_mfma_f32_32x32x16_bf16 (4 accumulator chains per
// wave, 512-thread workgroups, no memory traffic in the loop) runs back to
// back for a warm-up period and then a timed period, first with operands
// drawn from a standard normal distribution (as the attention inputs are) and
// then with all-zero operands.  Under sustained load the board holds its power
// cap by lowering the shader clock, and the clock it can hold depends on how
// much the operand bits toggle, so the two rates bracket what any kernel can
// sustain on this board; neither is the published peak, which assumes the
// maximum shader clock.
//
// Usage: mfma_rate [timed seconds per operand kind, default 2; a third more of warm-up]
// Prints one JSON line.  Exit status 0 on success, 1 on a HIP error.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kIters = 256;          // loop trips per wave
constexpr int kChains = 4;           // independent accumulators per wave
constexpr int kThreads = 512;        // 8 waves: 2 per SIMD
constexpr int kOperands = 1 << 20;   // 16-byte operand granules in the pool

__global__ __launch_bounds__(kThreads) void mfma_stream(float* out, const uint4* pool) {
    const uint32_t base = blockIdx.x * 4096u + threadIdx.x * 8u;
    bf16x8 a[4], b[4];
    for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_bit_cast(bf16x8, pool[(base + i) % kOperands]);
        b[i] = __builtin_bit_cast(bf16x8, pool[(base + 4 + i) % kOperands]);
    }
    f32x16 c[kChains];
    for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int k = 0; k < kChains; ++k)
                c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + k) & 3], b[(j * 3 + k) & 3], c[k], 0, 0, 0);
    }
    float s = 0.f;
    for (int k = 0; k < kChains; ++k)
        for (int r = 0; r < 16; ++r) s += c[k][r];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

bool ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    fprintf(stderr, "mfma_rate: %s: %s\n", what, hipGetErrorString(e));
    return false;
}

// bf16 bits of standard normal draws (Box-Muller over a 64-bit LCG), rounded
// to nearest even.
std::vector<uint32_t> normal_pool(uint64_t seed) {
    std::vector<uint32_t> w((size_t)kOperands * 4);
    uint64_t s = seed;
    auto uni = [&]() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return ((s >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    auto bf = [](float f) {
        uint32_t u;
        memcpy(&u, &f, 4);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    };
    for (size_t i = 0; i < w.size(); ++i) {
        const double r = std::sqrt(-2.0 * std::log(uni())), t = 6.283185307179586 * uni();
        w[i] = bf((float)(r * std::cos(t))) | (bf((float)(r * std::sin(t))) << 16);
    }
    return w;
}

}  // namespace

int main(int argc, char** argv) {
    const double seconds = argc > 1 ? atof(argv[1]) : 2.0;
    int dev = 0, ncu = 0;
    if (!ok(hipGetDevice(&dev), "hipGetDevice") ||
        !ok(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev), "device attribute"))
        return 1;
    const int grid = ncu * 16;
    const double flops = (double)grid * (kThreads / 64) * kIters * 4 * kChains * 32768.0;
    float* out = nullptr;
    uint4 *pool = nullptr, *zero = nullptr;
    if (!ok(hipMalloc(&out, (size_t)grid * kThreads * sizeof(float)), "hipMalloc") ||
        !ok(hipMalloc(&pool, (size_t)kOperands * 16), "hipMalloc") ||
        !ok(hipMalloc(&zero, (size_t)kOperands * 16), "hipMalloc"))
        return 1;
    const std::vector<uint32_t> h = normal_pool(20261202);
    if (!ok(hipMemcpy(pool, h.data(), (size_t)kOperands * 16, hipMemcpyHostToDevice), "hipMemcpy") ||
        !ok(hipMemset(zero, 0, (size_t)kOperands * 16), "hipMemset"))
        return 1;
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate")) return 1;
    double rate[2] = {0, 0};
    int launches[2] = {0, 0};
    for (int kind = 0; kind < 2; ++kind) {
        const uint4* src = kind == 0 ? pool : zero;
        // one launch to size the batches, then warm-up for a third of the time
        if (!ok(hipEventRecord(e0), "record")) return 1;
        hipLaunchKernelGGL(mfma_stream, dim3(grid), dim3(kThreads), 0, 0, out, src);
        if (!ok(hipEventRecord(e1), "record") || !ok(hipEventSynchronize(e1), "launch")) return 1;
        float ms = 0.f;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
        const int n = (int)std::fmax(10.0, seconds * 1e3 / std::fmax(ms, 1e-3));
        for (int i = 0; i < n / 3; ++i) hipLaunchKernelGGL(mfma_stream, dim3(grid), dim3(kThreads), 0, 0, out, src);
        if (!ok(hipEventRecord(e0), "record")) return 1;
        for (int i = 0; i < n; ++i) hipLaunchKernelGGL(mfma_stream, dim3(grid), dim3(kThreads), 0, 0, out, src);
        if (!ok(hipEventRecord(e1), "record") || !ok(hipEventSynchronize(e1), "launch")) return 1;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
        rate[kind] = flops * n / (ms * 1e-3) / 1e12;
        launches[kind] = n;
    }
    printf("{\"instruction\": \"v_mfma_f32_32x32x16_bf16\", \"waves_per_simd\": 2, \"chains_per_wave\": %d, "
           "\"normal_operands_tflops\": %.1f, \"zero_operands_tflops\": %.1f, \"timed_launches\": [%d, %d], "
           "\"flops_per_launch\": %.4e}\n",
           kChains, rate[0], rate[1], launches[0], launches[1], flops);
    return 0;
}
