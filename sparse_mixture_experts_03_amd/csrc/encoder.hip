// Hidden layer of the two-layer router (P3 §3.1: a small MLP of width d/4
// encodes the token before the gate; P3 §4.2: GeLU between the two linear
// layers): h = GeLU(W_in x + b_in), stored in the activation dtype.
//
// The product W_in x is the grouped expert GEMM with one expert holding all
// T rows (fp32 out, no gather); this file holds the two small kernels around
// it: the one-expert dispatch offsets {0, T}, written by a kernel so that a
// captured stream records no memset, and the bias + GeLU + rounding pass.
// GeLU here is h * erfc(-h / sqrt 2) / 2, accurate in the negative tail, so
// the stored hidden values match a binary64 evaluation to within the final
// rounding.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

__global__ void encoder_offsets_kernel(int32_t* offsets, int32_t T) {
    if (threadIdx.x == 0) offsets[0] = 0;
    if (threadIdx.x == 1) offsets[1] = T;
}

// Four consecutive hidden values per thread.
template <int ACT>
__global__ void __launch_bounds__(256)
encoder_act_kernel(const float* __restrict__ pre, const float* __restrict__ b_in, void* __restrict__ h, int64_t n4,
                   int d_r) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4*>(pre)[i];
    float r[4] = {v.x, v.y, v.z, v.w};
    const int j0 = (int)((i * 4) % d_r);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float s = b_in ? r[c] + b_in[j0 + c] : r[c];
        r[c] = 0.5f * s * erfcf(-s * 0.70710678118654752440f);
    }
    if constexpr (ACT == kF32) {
        reinterpret_cast<float4*>(h)[i] = make_float4(r[0], r[1], r[2], r[3]);
    } else {
        uint2 packed;
        packed.x = pack_bf16x2(r[0], r[1]);
        packed.y = pack_bf16x2(r[2], r[3]);
        reinterpret_cast<uint2*>(h)[i] = packed;
    }
}

}  // namespace

hipError_t launch_encoder_offsets(int32_t* offsets, int64_t T, hipStream_t stream) {
    hipLaunchKernelGGL(encoder_offsets_kernel, dim3(1), dim3(64), 0, stream, offsets, (int32_t)T);
    return hipGetLastError();
}

hipError_t launch_encoder_act(const float* pre, const float* b_in, void* h, int64_t T, int d_r, int act_dtype,
                              hipStream_t stream) {
    const int64_t n4 = T * (int64_t)d_r / 4;  // d_r is a multiple of 64
    if (n4 == 0) return hipSuccess;
    const int64_t blocks = (n4 + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (act_dtype == kF32)
        hipLaunchKernelGGL(encoder_act_kernel<kF32>, dim3((unsigned)blocks), dim3(256), 0, stream, pre, b_in, h, n4,
                           d_r);
    else
        hipLaunchKernelGGL(encoder_act_kernel<kBF16>, dim3((unsigned)blocks), dim3(256), 0, stream, pre, b_in, h, n4,
                           d_r);
    return hipGetLastError();
}

}  // namespace moe
