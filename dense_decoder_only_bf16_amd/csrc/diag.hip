// Diagnostics: what the chip sustains on its own, measured with plain kernels, to put the
// roofline fractions of the forward's kernels in context.
//  * MFMA: 2048 workgroups of 8 waves, each wave 8 independent 32x32x16 bf16 accumulators
//    fed by register operands that rotate every round, so the matrix cores see data that
//    keeps toggling (random) or stays fixed (constant).
//  * HBM: a 1 GiB read stream, 16 independent 16-byte loads per lane in flight.
#include "common.h"
#include "kernels.h"
#include "nc.h"

namespace nc {
namespace {

__global__ __launch_bounds__(256) void diag_fill_kernel(uint32_t* p, long long n, int random) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    if (!random) {
        p[i] = 0x3c003c00u;  // bf16 pairs of 1.0 scaled down: a fixed pattern
        return;
    }
    uint32_t x = (uint32_t)i * 2654435761u + 0x9e3779b9u;  // integer hash of the index
    x ^= x >> 16; x *= 0x85ebca6bu; x ^= x >> 13; x *= 0xc2b2ae35u; x ^= x >> 16;
    // two bf16 values: random sign and mantissa, exponents 2^-1 .. 2^2
    const uint32_t lo = (x & 0x807Fu) | ((126u + ((x >> 8) & 3u)) << 7);
    const uint32_t hi = ((x >> 16) & 0x807Fu) | ((126u + ((x >> 24) & 3u)) << 7);
    p[i] = lo | (hi << 16);
}

__global__ __launch_bounds__(512) void diag_mfma_kernel(const bf16x8* __restrict__ src, float* out, int rounds) {
    const int lane = threadIdx.x & 63;
    bf16x8 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = src[((long long)blockIdx.x * 8 + i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 2; ++i) b[i] = src[((long long)blockIdx.x * 8 + 4 + i) * 64 + lane];
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero_vec<f32x16>();
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mma32(a[i], b[j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // rotate the operand words
            u4 t = __builtin_bit_cast(u4, a[i]);
            t = (u4){t[1], t[2], t[3], t[0]};
            a[i] = __builtin_bit_cast(bf16x8, t);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    out[(long long)blockIdx.x * 512 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void diag_stream_kernel(const char* __restrict__ src, long long per_wg,
                                                           uint32_t* out) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const char* base = src + (long long)blockIdx.x * per_wg + wave * (per_wg / 4);
    const int n = (int)(per_wg / 4 / 1024);  // 1 KB per wave load; a multiple of 16
    u4 acc = {0u, 0u, 0u, 0u};
    for (int i = 0; i < n; i += 16) {
        u4 v[16];
#pragma unroll
        for (int d = 0; d < 16; ++d) v[d] = *(const u4*)(base + (long long)(i + d) * 1024 + lane * 16);
#pragma unroll
        for (int d = 0; d < 16; ++d) acc ^= v[d];
    }
    out[(long long)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <typename F>
hipError_t time_ms(F launch, int reps, float* ms) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = launch();  // warm-up
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipEventRecord(e0, 0);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return e;
}

}  // namespace
}  // namespace nc

using namespace nc;

extern "C" {

nc_status nc_diag_mfma_rate(int32_t random_operands, double* tflops) {
    if (!tflops) return NC_ERR_INVALID_ARG;
    const int blocks = 256 * 8, rounds = 2000;
    const long long words = (long long)blocks * 8 * 64 * 4;  // bf16x8 = 4 words
    uint32_t* src = nullptr;
    float* out = nullptr;
    hipError_t e = hipMalloc((void**)&src, words * 4);
    if (e == hipSuccess) e = hipMalloc((void**)&out, (size_t)blocks * 512 * 4);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(diag_fill_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, 0, src, words,
                           random_operands ? 1 : 0);
        e = hipGetLastError();
    }
    float ms = 0.f;
    if (e == hipSuccess)
        e = time_ms([&] {
            hipLaunchKernelGGL(diag_mfma_kernel, dim3(blocks), dim3(512), 0, 0, (const bf16x8*)src, out, rounds);
            return hipGetLastError();
        }, 1, &ms);
    if (src) (void)hipFree(src);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return NC_ERR_DEVICE;
    *tflops = (double)blocks * 8 * rounds * 8 * 32768.0 / (ms * 1e-3) / 1e12;
    return NC_OK;
}

nc_status nc_diag_hbm_read_rate(double* tbps) {
    if (!tbps) return NC_ERR_INVALID_ARG;
    const long long total = 1LL << 30;
    const int blocks = 1024;
    char* src = nullptr;
    uint32_t* out = nullptr;
    hipError_t e = hipMalloc((void**)&src, total);
    if (e == hipSuccess) e = hipMalloc((void**)&out, (size_t)blocks * 256 * 4);
    if (e == hipSuccess) e = hipMemset(src, 1, total);
    float ms = 0.f;
    if (e == hipSuccess)
        e = time_ms([&] {
            hipLaunchKernelGGL(diag_stream_kernel, dim3(blocks), dim3(256), 0, 0, (const char*)src, total / blocks, out);
            return hipGetLastError();
        }, 5, &ms);
    if (src) (void)hipFree(src);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return NC_ERR_DEVICE;
    *tbps = (double)total * 5 / (ms * 1e-3) / 1e12;
    return NC_OK;
}

}  // extern "C"
