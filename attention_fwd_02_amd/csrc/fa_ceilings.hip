// fa_ceilings.hip -- same-machine ceilings for the attention kernels' rooflines.
//
// The datasheet peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16) are what a kernel
// is finally measured against; these loops measure what this GPU actually
// sustains at its running clock, one resource at a time, so that a kernel's
// fraction of peak can be read against a bandwidth ceiling and an
// instruction-issue ceiling measured on the same machine ("从 Volta/Turing、
// Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程范式演进", section
// "到不了理论性能：硬件限制还是优化问题", step 2: first the bandwidth
// ceiling, then the instruction ceiling).
//
//  * HBM streaming read: every workgroup reads disjoint 16-byte-per-lane
//    chunks of a buffer much larger than the caches and folds them into one
//    word per lane, so only the reads cost.
//  * MFMA loop: one wave per SIMD issuing independent
//    v_mfma_f32_32x32x16_bf16 (or the FP8 v_mfma_f32_32x32x64_f8f6f4) on four
//    accumulators; also reports the shader clock the loop ran at, from the
//    wave's cycle counter against the constant-rate real-time counter.
//  * LDS read: conflict-free ds_read_b128 or ds_read_b64_tr_b16 streams, eight
//    waves per CU, in bytes per clock per CU.
//  * VALU: independent v_fma_f32 or v_exp_f32 streams, cycles per wave-wide
//    instruction.
//  * MFMA + VALU co-issue: cycles per MFMA when k independent v_fma_f32 sit
//    between consecutive MFMAs of one wave (how much vector work an MFMA's
//    shadow holds).
//
// The loops are inline asm so that the measured instruction stream is exactly
// the one named; every address stays inside the buffers the host sizes.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "../../include/fa_ceilings.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef int i32x8_t __attribute__((__vector_size__(32)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));

// ---- HBM streaming read ------------------------------------------------------
// Workgroup w of G reads 16-byte lanes of chunk c = w, w + G, ...: chunk c is
// 256 lanes x 16 B x UNROLL = 16 KiB at UNROLL = 4, contiguous.
template <int UNROLL>
__global__ void __launch_bounds__(256) ceil_hbm_read_kernel(const u32x4_t *__restrict__ buf,
                                                            long n_chunks, uint32_t *out)
{
    const int t = threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (long c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const u32x4_t *p = buf + c * (256 * UNROLL) + t;
        u32x4_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + u * 256);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    out[blockIdx.x * 256 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---- MFMA loop -----------------------------------------------------------------
// Each wave: iters x 8 independent MFMAs on four accumulators.  cyc[w] gets
// the wave's shader-clock cycles, rt[w] its real-time ticks.
template <bool FP8>
__global__ void __launch_bounds__(256) ceil_mfma_kernel(int iters, float *out, long long *cyc,
                                                        long long *rt)
{
    const int l = threadIdx.x;
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (FP8) {
        i32x8_t a, b;
        for (int i = 0; i < 8; ++i) { a[i] = 0x38383838 + l + i; b[i] = 0x30303030 + l - i; }
        for (int it = 0; it < iters; ++it) {
            asm volatile(
                "v_mfma_f32_32x32x64_f8f6f4 %0, %4, %5, %0\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %1, %4, %5, %1\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %2, %4, %5, %2\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %3, %4, %5, %3\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %0, %4, %5, %0\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %1, %4, %5, %1\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %2, %4, %5, %2\n\t"
                "v_mfma_f32_32x32x64_f8f6f4 %3, %4, %5, %3"
                : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
                : "v"(a), "v"(b));
        }
    } else {
        bf16x8_t a, b;
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(0.001f * (l + i));
            b[i] = (__bf16)(0.002f * (l - i));
        }
        for (int it = 0; it < iters; ++it) {
            asm volatile(
                "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
                "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
                "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
                "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3\n\t"
                "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
                "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
                "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
                "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
                : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
                : "v"(a), "v"(b));
        }
    }
    // the last MFMAs finish before the counters are read again
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * 256 + l] = s;
    if ((l & 63) == 0) {
        cyc[blockIdx.x * 4 + (l >> 6)] = t1 - t0;
        rt[blockIdx.x * 4 + (l >> 6)] = r1 - r0;
    }
}

// ---- MFMA + VALU co-issue ------------------------------------------------------
// 8 MFMAs per trip, K independent v_fma_f32 (or v_exp_f32 when EXP) after each.
template <int K, bool EXP = false>
__global__ void __launch_bounds__(256) ceil_coissue_kernel(int iters, float *out, long long *cyc)
{
    const int l = threadIdx.x;
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (l + i));
        b[i] = (__bf16)(0.002f * (l - i));
    }
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = l * 1e-3f + i;
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            f32x16_t &c = (m & 3) == 0 ? c0 : (m & 3) == 1 ? c1 : (m & 3) == 2 ? c2 : c3;
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float &y = x[(m * K + k) & 7];
                if constexpr (EXP)
                    asm volatile("v_exp_f32 %0, %1" : "=v"(y) : "v"(x[(m * K + k + 3) & 7]));
                else
                    asm volatile("v_fma_f32 %0, %0, %1, %2"
                                 : "+v"(y)
                                 : "v"(x[(m * K + k + 3) & 7]), "v"(x[(m * K + k + 5) & 7]));
            }
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    for (int i = 0; i < 8; ++i) s += x[i];
    out[blockIdx.x * 256 + l] = s;
    if ((l & 63) == 0) cyc[blockIdx.x * 4 + (l >> 6)] = t1 - t0;
}

// ---- LDS read --------------------------------------------------------------------
// 8 waves; wave w reads half h = w & 1 of a 64 KiB array: 16 reads per trip,
// lane l at l * 16 (b128, 1 KiB per read) or l * 8 (tr16, 512 B per read)
// plus an immediate offset below 16 KiB, a wait after every 8.
template <bool TR>
__global__ void __launch_bounds__(512) ceil_lds_kernel(int iters, float *out, long long *cyc)
{
    __shared__ __attribute__((aligned(1024))) char lds[65536];
    const int t = threadIdx.x;
    for (int i = t; i < 65536 / 4; i += blockDim.x) reinterpret_cast<float *>(lds)[i] = i * 0.5f;
    __syncthreads();
    const int lane = t & 63;
    const uint32_t ad =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)(lds + ((t >> 6) & 1) * 32768) +
        lane * (TR ? 8 : 16);
    u32x4_t r[8];
    u32x2_t h[8];
    for (int i = 0; i < 8; ++i) {
        r[i] = (u32x4_t){0u, 0u, 0u, 0u};
        h[i] = (u32x2_t){0u, 0u};
    }
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (TR) {
            asm volatile(
                "ds_read_b64_tr_b16 %0, %8 offset:0\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\t"
                "ds_read_b64_tr_b16 %2, %8 offset:1024\n\tds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
                "ds_read_b64_tr_b16 %4, %8 offset:2048\n\tds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
                "ds_read_b64_tr_b16 %6, %8 offset:3072\n\tds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
                "s_waitcnt lgkmcnt(0)\n\t"
                "ds_read_b64_tr_b16 %0, %8 offset:4096\n\tds_read_b64_tr_b16 %1, %8 offset:4608\n\t"
                "ds_read_b64_tr_b16 %2, %8 offset:5120\n\tds_read_b64_tr_b16 %3, %8 offset:5632\n\t"
                "ds_read_b64_tr_b16 %4, %8 offset:6144\n\tds_read_b64_tr_b16 %5, %8 offset:6656\n\t"
                "ds_read_b64_tr_b16 %6, %8 offset:7168\n\tds_read_b64_tr_b16 %7, %8 offset:7680\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "+v"(h[0]), "+v"(h[1]), "+v"(h[2]), "+v"(h[3]), "+v"(h[4]), "+v"(h[5]),
                  "+v"(h[6]), "+v"(h[7])
                : "v"(ad)
                : "memory");
        } else {
            asm volatile(
                "ds_read_b128 %0, %8 offset:0\n\tds_read_b128 %1, %8 offset:1024\n\t"
                "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
                "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
                "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
                "s_waitcnt lgkmcnt(0)\n\t"
                "ds_read_b128 %0, %8 offset:8192\n\tds_read_b128 %1, %8 offset:9216\n\t"
                "ds_read_b128 %2, %8 offset:10240\n\tds_read_b128 %3, %8 offset:11264\n\t"
                "ds_read_b128 %4, %8 offset:12288\n\tds_read_b128 %5, %8 offset:13312\n\t"
                "ds_read_b128 %6, %8 offset:14336\n\tds_read_b128 %7, %8 offset:15360\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                  "+v"(r[6]), "+v"(r[7])
                : "v"(ad)
                : "memory");
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    uint32_t s = 0;
    for (int i = 0; i < 8; ++i) s += r[i][0] + r[i][1] + r[i][2] + r[i][3] + h[i][0] + h[i][1];
    out[blockIdx.x * 512 + t] = (float)s;
    if (lane == 0) cyc[blockIdx.x * 8 + (t >> 6)] = t1 - t0;
}

// ---- VALU ------------------------------------------------------------------------
// 64 independent-enough instructions per trip over 8 registers.
template <bool EXP>
__global__ void __launch_bounds__(256) ceil_valu_kernel(int iters, float *out, long long *cyc)
{
    const int l = threadIdx.x;
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = l * 1e-3f + i * 0.01f;
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            float &y = x[k & 7];
            if constexpr (EXP)
                asm volatile("v_exp_f32 %0, %0" : "+v"(y));
            else
                asm volatile("v_fma_f32 %0, %0, %1, %2"
                             : "+v"(y)
                             : "v"(x[(k + 3) & 7]), "v"(x[(k + 5) & 7]));
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.0f;
    for (int i = 0; i < 8; ++i) s += x[i];
    out[blockIdx.x * 256 + l] = s;
    if ((l & 63) == 0) cyc[blockIdx.x * 4 + (l >> 6)] = t1 - t0;
}

// ---- host side -----------------------------------------------------------------------
thread_local char g_err[256];

int set_err(const char *what, hipError_t e)
{
    snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
    return 1;
}

#define CEIL_CK(x)                                     \
    do {                                               \
        hipError_t e_ = (x);                           \
        if (e_ != hipSuccess) return set_err(#x, e_); \
    } while (0)

struct Timer {
    hipEvent_t a = nullptr, b = nullptr;
    ~Timer()
    {
        if (a) (void)hipEventDestroy(a);
        if (b) (void)hipEventDestroy(b);
    }
};

struct DevBuf {
    void *p = nullptr;
    ~DevBuf()
    {
        if (p) (void)hipFree(p);
    }
};

double mean_of(const long long *v, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += (double)v[i];
    return n ? s / n : 0.0;
}

int cu_count(int *cus)
{
    int dev = 0;
    CEIL_CK(hipGetDevice(&dev));
    CEIL_CK(hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev));
    return 0;
}

}  // namespace

extern "C" {

const char *fa_ceil_last_error(void) { return g_err; }

int fa_ceil_hbm_read(const void *buf, size_t bytes, int reps, double *gbps)
{
    if (!buf || !gbps || reps < 1 || ((uintptr_t)buf & 15u)) {
        snprintf(g_err, sizeof(g_err), "bad arguments");
        return 1;
    }
    constexpr int UNROLL = 4;
    const long chunk = 256L * 16 * UNROLL;
    const long n_chunks = (long)(bytes / (size_t)chunk);
    if (n_chunks < 1) {
        snprintf(g_err, sizeof(g_err), "buffer smaller than one 16 KiB chunk");
        return 1;
    }
    int cus = 0;
    if (cu_count(&cus)) return 1;
    const int grid = (int)std::min<long>(n_chunks, (long)cus * 8);
    DevBuf out;
    CEIL_CK(hipMalloc(&out.p, (size_t)grid * 256 * 4));
    Timer t;
    CEIL_CK(hipEventCreate(&t.a));
    CEIL_CK(hipEventCreate(&t.b));
    const u32x4_t *src = static_cast<const u32x4_t *>(buf);
    hipLaunchKernelGGL((ceil_hbm_read_kernel<UNROLL>), dim3(grid), dim3(256), 0, 0, src, n_chunks,
                       static_cast<uint32_t *>(out.p));
    CEIL_CK(hipGetLastError());
    CEIL_CK(hipEventRecord(t.a, 0));
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL((ceil_hbm_read_kernel<UNROLL>), dim3(grid), dim3(256), 0, 0, src,
                           n_chunks, static_cast<uint32_t *>(out.p));
    CEIL_CK(hipEventRecord(t.b, 0));
    CEIL_CK(hipEventSynchronize(t.b));
    float ms = 0.0f;
    CEIL_CK(hipEventElapsedTime(&ms, t.a, t.b));
    *gbps = (double)n_chunks * chunk * reps / (ms * 1e-3) / 1e9;
    return 0;
}

int fa_ceil_mfma(int fp8, int iters, double *tflops, double *clock_mhz)
{
    if (!tflops || !clock_mhz || iters < 1) {
        snprintf(g_err, sizeof(g_err), "bad arguments");
        return 1;
    }
    int cus = 0;
    if (cu_count(&cus)) return 1;
    int dev = 0, rt_khz = 0;
    CEIL_CK(hipGetDevice(&dev));
    CEIL_CK(hipDeviceGetAttribute(&rt_khz, hipDeviceAttributeWallClockRate, dev));
    const int grid = cus, waves = grid * 4;
    DevBuf out, cyc, rt;
    CEIL_CK(hipMalloc(&out.p, (size_t)grid * 256 * 4));
    CEIL_CK(hipMalloc(&cyc.p, (size_t)waves * 8));
    CEIL_CK(hipMalloc(&rt.p, (size_t)waves * 8));
    Timer t;
    CEIL_CK(hipEventCreate(&t.a));
    CEIL_CK(hipEventCreate(&t.b));
    auto launch = [&](int n) {
        if (fp8)
            hipLaunchKernelGGL((ceil_mfma_kernel<true>), dim3(grid), dim3(256), 0, 0, n,
                               static_cast<float *>(out.p), static_cast<long long *>(cyc.p),
                               static_cast<long long *>(rt.p));
        else
            hipLaunchKernelGGL((ceil_mfma_kernel<false>), dim3(grid), dim3(256), 0, 0, n,
                               static_cast<float *>(out.p), static_cast<long long *>(cyc.p),
                               static_cast<long long *>(rt.p));
    };
    launch(iters / 4 + 1);   // clock ramp
    CEIL_CK(hipGetLastError());
    CEIL_CK(hipEventRecord(t.a, 0));
    launch(iters);
    CEIL_CK(hipEventRecord(t.b, 0));
    CEIL_CK(hipEventSynchronize(t.b));
    float ms = 0.0f;
    CEIL_CK(hipEventElapsedTime(&ms, t.a, t.b));
    std::vector<long long> hc(waves), hr(waves);
    CEIL_CK(hipMemcpy(hc.data(), cyc.p, (size_t)waves * 8, hipMemcpyDeviceToHost));
    CEIL_CK(hipMemcpy(hr.data(), rt.p, (size_t)waves * 8, hipMemcpyDeviceToHost));
    const double flop_per_mfma = fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
    *tflops = (double)waves * iters * 8 * flop_per_mfma / (ms * 1e-3) / 1e12;
    const double c = mean_of(hc.data(), waves), r = mean_of(hr.data(), waves);
    *clock_mhz = r > 0 ? c / (r / (rt_khz * 1e3)) / 1e6 : 0.0;
    return 0;
}

int fa_ceil_coissue(int k_valu, int iters, double *cycles_per_mfma)
{
    if (!cycles_per_mfma || iters < 1) {
        snprintf(g_err, sizeof(g_err), "bad arguments");
        return 1;
    }
    int cus = 0;
    if (cu_count(&cus)) return 1;
    const int grid = cus, waves = grid * 4;
    DevBuf out, cyc;
    CEIL_CK(hipMalloc(&out.p, (size_t)grid * 256 * 4));
    CEIL_CK(hipMalloc(&cyc.p, (size_t)waves * 8));
    float *o = static_cast<float *>(out.p);
    long long *cy = static_cast<long long *>(cyc.p);
    switch (k_valu) {
    case 0: hipLaunchKernelGGL((ceil_coissue_kernel<0>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case 2: hipLaunchKernelGGL((ceil_coissue_kernel<2>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case 4: hipLaunchKernelGGL((ceil_coissue_kernel<4>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case 5: hipLaunchKernelGGL((ceil_coissue_kernel<5>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case 6: hipLaunchKernelGGL((ceil_coissue_kernel<6>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case 8: hipLaunchKernelGGL((ceil_coissue_kernel<8>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case -1: hipLaunchKernelGGL((ceil_coissue_kernel<1, true>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case -2: hipLaunchKernelGGL((ceil_coissue_kernel<2, true>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    case -4: hipLaunchKernelGGL((ceil_coissue_kernel<4, true>), dim3(grid), dim3(256), 0, 0, iters, o, cy); break;
    default: snprintf(g_err, sizeof(g_err), "k_valu must be 0, 2, 4, 5, 6, 8, -1, -2 or -4"); return 1;
    }
    CEIL_CK(hipGetLastError());
    CEIL_CK(hipDeviceSynchronize());
    std::vector<long long> hc(waves);
    CEIL_CK(hipMemcpy(hc.data(), cyc.p, (size_t)waves * 8, hipMemcpyDeviceToHost));
    *cycles_per_mfma = mean_of(hc.data(), waves) / ((double)iters * 8);
    return 0;
}

int fa_ceil_lds(int transposing, int iters, double *bytes_per_clk_cu)
{
    if (!bytes_per_clk_cu || iters < 1) {
        snprintf(g_err, sizeof(g_err), "bad arguments");
        return 1;
    }
    int cus = 0;
    if (cu_count(&cus)) return 1;
    const int grid = cus, waves = grid * 8;
    DevBuf out, cyc;
    CEIL_CK(hipMalloc(&out.p, (size_t)grid * 512 * 4));
    CEIL_CK(hipMalloc(&cyc.p, (size_t)waves * 8));
    if (transposing)
        hipLaunchKernelGGL((ceil_lds_kernel<true>), dim3(grid), dim3(512), 0, 0, iters,
                           static_cast<float *>(out.p), static_cast<long long *>(cyc.p));
    else
        hipLaunchKernelGGL((ceil_lds_kernel<false>), dim3(grid), dim3(512), 0, 0, iters,
                           static_cast<float *>(out.p), static_cast<long long *>(cyc.p));
    CEIL_CK(hipGetLastError());
    CEIL_CK(hipDeviceSynchronize());
    std::vector<long long> hc(waves);
    CEIL_CK(hipMemcpy(hc.data(), cyc.p, (size_t)waves * 8, hipMemcpyDeviceToHost));
    const double cyc_per_trip = mean_of(hc.data(), waves) / iters;
    const double bytes_per_trip_cu = 8.0 * 16 * (transposing ? 512 : 1024);
    *bytes_per_clk_cu = bytes_per_trip_cu / cyc_per_trip;
    return 0;
}

int fa_ceil_valu(int exp, int iters, double *cycles_per_instr)
{
    if (!cycles_per_instr || iters < 1) {
        snprintf(g_err, sizeof(g_err), "bad arguments");
        return 1;
    }
    int cus = 0;
    if (cu_count(&cus)) return 1;
    const int grid = cus, waves = grid * 4;
    DevBuf out, cyc;
    CEIL_CK(hipMalloc(&out.p, (size_t)grid * 256 * 4));
    CEIL_CK(hipMalloc(&cyc.p, (size_t)waves * 8));
    if (exp)
        hipLaunchKernelGGL((ceil_valu_kernel<true>), dim3(grid), dim3(256), 0, 0, iters,
                           static_cast<float *>(out.p), static_cast<long long *>(cyc.p));
    else
        hipLaunchKernelGGL((ceil_valu_kernel<false>), dim3(grid), dim3(256), 0, 0, iters,
                           static_cast<float *>(out.p), static_cast<long long *>(cyc.p));
    CEIL_CK(hipGetLastError());
    CEIL_CK(hipDeviceSynchronize());
    std::vector<long long> hc(waves);
    CEIL_CK(hipMemcpy(hc.data(), cyc.p, (size_t)waves * 8, hipMemcpyDeviceToHost));
    *cycles_per_instr = mean_of(hc.data(), waves) / ((double)iters * 64);
    return 0;
}

}  // extern "C"
