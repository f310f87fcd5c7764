// Measurement kernels (declared in include/probe.h): the FMA-rate probe that
// times what a given number of compute units sustain on non-packed fp32 FMA.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/probe.h"
#include "api_common.h"

namespace {

constexpr int kProbeChains = 8;
constexpr int kProbeLds = 96 * 1024 / 4;   // floats reserved per workgroup for one_per_cu

// Every lane: kProbeChains independent chains, kProbeChains links each per
// iteration (64 dependent-free v_fma_f32 per iteration over the lane).
template <bool ONE_PER_CU>
__global__ __launch_bounds__(1024) void fma_probe_kernel(float* out, float m, float c, int iters)
{
    float x[kProbeChains];
#pragma unroll
    for (int i = 0; i < kProbeChains; ++i) x[i] = (float)(threadIdx.x & 63) * 1e-3f + (float)i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kProbeChains; ++r)
#pragma unroll
            for (int i = 0; i < kProbeChains; ++i) x[i] = fmaf(x[i], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kProbeChains; ++i) s += x[i];
    if constexpr (ONE_PER_CU) {
        // The reservation: a never-taken path (iters >= 1) keeps the array,
        // and with it 96 KiB of LDS per workgroup, in the kernel.
        __shared__ float pad[kProbeLds];
        if (iters < 0) {
            pad[threadIdx.x] = s;
            __syncthreads();
            s = pad[kProbeLds - 1 - threadIdx.x];
        }
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int cfc_probe_fma(int blocks, int threads, int one_per_cu, int iters, float* out, void* stream)
{
    if (blocks < 1 || blocks > 65536)
        return cfc_host::fail(CFC_EINVAL, "cfc_probe_fma: blocks=%d outside [1, 65536]", blocks);
    if (threads < 64 || threads > 1024 || threads % 64 != 0)
        return cfc_host::fail(CFC_EINVAL, "cfc_probe_fma: threads=%d is not a multiple of 64 in [64, 1024]", threads);
    if (iters < 1 || iters > (1 << 20))
        return cfc_host::fail(CFC_EINVAL, "cfc_probe_fma: iters=%d outside [1, 2^20]", iters);
    if (out == nullptr) return cfc_host::fail(CFC_EINVAL, "cfc_probe_fma: out is NULL");
    hipStream_t s = (hipStream_t)stream;
    // m < 1 and c > 0 keep every chain bounded (it tends to c / (1 - m) = 1)
    const float m = 0.999f, c = 0.001f;
    if (one_per_cu)
        hipLaunchKernelGGL(fma_probe_kernel<true>, dim3((unsigned)blocks), dim3((unsigned)threads), 0, s, out, m, c,
                           iters);
    else
        hipLaunchKernelGGL(fma_probe_kernel<false>, dim3((unsigned)blocks), dim3((unsigned)threads), 0, s, out, m, c,
                           iters);
    CFC_HIP(hipGetLastError(), "FMA probe launch");
    return CFC_OK;
}

}  // extern "C"
