// probe.hip -- machine-rate probes (include/moe_probe.h): the HBM read rate
// through the global -> LDS copies the expert GEMMs use, and the rate of a
// register-resident loop of their MFMA instruction.  Measurement helpers
// only; nothing in the layer calls them.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_probe.h"

namespace moe {
namespace {

constexpr int PR_STEP = 65536;  // bytes per block and step
constexpr int PR_THREADS = 512;

// Each block streams its share of buf through two 64 KB LDS stages: wave w
// copies the 1 KB pieces w, w + 8, ... of a step (16 B per lane), the copy of
// step kt + 1 is issued after the barrier that retires step kt's, as in the
// GEMMs' pipeline.
__global__ void __launch_bounds__(PR_THREADS, 1) probe_hbm_read_kernel(const uint8_t* __restrict__ buf,
                                                                      int64_t per,
                                                                      uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * PR_STEP];
    constexpr int PW = PR_STEP / 1024 / 8;  // copies per wave and step
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* base = buf + blockIdx.x * per;
    const int nk = (int)(per / PR_STEP);
    auto issue = [&](int kt) {
        uint8_t* s = smem + (kt & 1) * PR_STEP;
#pragma unroll
        for (int c = 0; c < PW; ++c) {
            const int b = wave + 8 * c;
            __builtin_amdgcn_global_load_lds(
                (const void*)(base + (int64_t)kt * PR_STEP + b * 1024 + lane * 16),
                (__attribute__((address_space(3))) void*)(s + b * 1024), 16, 0, 0);
        }
    };
    uint32_t acc = 0;
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // step kt landed for every wave; step kt-1 is read
        if (kt + 1 < nk) issue(kt + 1);
        acc ^= *(const uint32_t*)(smem + (kt & 1) * PR_STEP + threadIdx.x * 4);
    }
    sink[blockIdx.x * PR_THREADS + threadIdx.x] = acc;
}

// 10 accumulators per wave (160 registers, as a GEMM wave holds) fed from
// registers; the operands differ per lane so the loop cannot be folded.
template <int DT>
__global__ void __launch_bounds__(PR_THREADS, 1) probe_mfma_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    f32x16_t acc[10];
#pragma unroll
    for (int i = 0; i < 10; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    float s = 0.0f;
    if constexpr (DT == MOE_BF16) {
        bf16x8_t a, b;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            a[v] = (__bf16)(1.0f + 0.001f * (lane + v));
            b[v] = (__bf16)(0.5f - 0.002f * (lane ^ v));
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 10; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    } else {
        i32x8_t a, b;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            a[v] = 0x38303830 + lane + v;  // E4M3 codes of magnitude ~0.5 .. 1
            b[v] = 0x30383038 + (lane ^ v);
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 10; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int i = 0; i < 10; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[i][v];
    sink[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_probe_hbm_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream) {
    if (!buf || !sink || ((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u))
        return moe::set_error(MOE_ERR_ARG, "moe_probe_hbm_read: buf / sink NULL or misaligned");
    if (blocks < 1 || blocks > 65536)
        return moe::set_error(MOE_ERR_ARG, "moe_probe_hbm_read: blocks must be in 1..65536");
    const uint64_t unit = (uint64_t)blocks * moe::PR_STEP;
    if (bytes == 0 || bytes % unit || bytes >= ((uint64_t)1 << 40))
        return moe::set_error(MOE_ERR_ARG,
                              "moe_probe_hbm_read: bytes must be a positive multiple of blocks * 65536, below 2^40");
    moe::probe_hbm_read_kernel<<<blocks, moe::PR_THREADS, 0, (hipStream_t)stream>>>(
        (const uint8_t*)buf, (int64_t)(bytes / blocks), sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, hipGetErrorString(e));
    return moe::set_error(MOE_OK, "");
}

int moe_probe_mfma(int32_t dtype, int32_t iters, int blocks, float* sink, void* stream) {
    if (!sink || ((uintptr_t)sink & 3u))
        return moe::set_error(MOE_ERR_ARG, "moe_probe_mfma: sink NULL or misaligned");
    if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3)
        return moe::set_error(MOE_ERR_ARG, "moe_probe_mfma: dtype must be MOE_BF16 or MOE_FP8_E4M3");
    if (iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > 65536)
        return moe::set_error(MOE_ERR_ARG, "moe_probe_mfma: iters in 1..2^24, blocks in 1..65536");
    if (dtype == MOE_BF16)
        moe::probe_mfma_kernel<MOE_BF16><<<blocks, moe::PR_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    else
        moe::probe_mfma_kernel<MOE_FP8_E4M3><<<blocks, moe::PR_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, hipGetErrorString(e));
    return moe::set_error(MOE_OK, "");
}

}  // extern "C"
