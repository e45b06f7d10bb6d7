// fab_probe.hip -- a measurement hook of libfab (gfx950): the sustained rate of
// the bf16 matrix cores and the shader clock that goes with it.
//
// Every wave of a fully resident grid (two 8-wave work-groups per CU, four rounds)
// runs back-to-back v_mfma_f32_32x32x16_bf16 products on four independent
// accumulators, so the matrix pipe of every SIMD always has an independent
// product to start.  The rate this loop reaches is the practical ceiling of the
// dense products on the part (the chip lowers its clock under this load); the
// kernels' roofline fractions are priced against the published peak, this
// figure is context for them.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fab.h"
#include "fab_common.h"
#include "fab_launch.h"

namespace fab {
namespace {

constexpr int kProbeNT = 512, kProbeGrid = 2048;

__global__ __launch_bounds__(kProbeNT) void mfma_loop_kernel(float *out, unsigned long long *clk, int iters)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(1e-3f * (float)(i - (int)threadIdx.x));
    }
    f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = mfma_bf16(a, b, c0);
        c1 = mfma_bf16(a, b, c1);
        c2 = mfma_bf16(a, b, c2);
        c3 = mfma_bf16(a, b, c3);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[(size_t)blockIdx.x * kProbeNT + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace
}  // namespace fab

extern "C" size_t fab_probe_scratch_bytes(void)
{
    return (size_t)fab::kProbeGrid * fab::kProbeNT * sizeof(float) + (size_t)fab::kProbeGrid * 16;
}

extern "C" int fab_measure_mfma_loop(void *scratch, size_t scratch_bytes, int iters, double *tflops, double *clock_ghz,
                                     void *stream)
{
    using namespace fab;
    set_error(FAB_OK, "");
    if (!scratch || !tflops || !clock_ghz || iters <= 0 || iters > (1 << 24))
        return set_error(FAB_E_INVAL, "NULL argument or iters outside [1, 2^24]");
    if (scratch_bytes < fab_probe_scratch_bytes())
        return set_error(FAB_E_INVAL, "scratch holds %zu bytes, the probe needs %zu", scratch_bytes,
                         fab_probe_scratch_bytes());
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *out = static_cast<float *>(scratch);
    unsigned long long *clk = reinterpret_cast<unsigned long long *>(out + (size_t)kProbeGrid * kProbeNT);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    if (err == hipSuccess) {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(kProbeGrid), dim3(kProbeNT), 0, s, out, clk, iters < 64 ? iters : 64);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e0, s);
    if (err == hipSuccess) {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(kProbeGrid), dim3(kProbeNT), 0, s, out, clk, iters);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, s);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    unsigned long long host[2 * 64];
    if (err == hipSuccess) err = hipMemcpyAsync(host, clk, sizeof(host), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (err != hipSuccess)
        return set_error(FAB_E_HIP, "HIP error %d (%s) in the matrix-core probe", (int)err, hipGetErrorString(err));
    // flops: waves x iterations x 4 products x 32*32*16*2
    const double flops = (double)kProbeGrid * (kProbeNT / 64) * iters * 4.0 * 32768.0;
    *tflops = flops / (ms * 1e-3) / 1e12;
    // shader cycles over 100 MHz real-time ticks of the first 64 work-groups
    double cyc = 0.0, rt = 0.0;
    for (int i = 0; i < 64; ++i) {
        cyc += (double)host[2 * i];
        rt += (double)host[2 * i + 1];
    }
    *clock_ghz = rt > 0.0 ? cyc / rt * 0.1 : 0.0;
    return FAB_OK;
}
