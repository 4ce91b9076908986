// Combine: y[t] = sum_j gate[t][j] * Y[pos[t][j]]   (P2 §2.2 step 4: the
// chosen experts' outputs are summed weighted by their confidences; P5 §3.2).
// Pure streaming: each thread owns 4 consecutive columns of one token row,
// sums the k expert rows in ascending j with fp32 FMAs and stores in the
// activation dtype (bf16: round to nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kCombineCols = 1024;  // columns per workgroup (256 threads x 4)

template <int ACT, bool SPLIT>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ Y, const float* __restrict__ Y2, const int32_t* __restrict__ pos,
               const float* __restrict__ gates, void* __restrict__ y, int64_t d, int k, int chunks) {
    const int64_t t = blockIdx.x / chunks;
    const int64_t c = (int64_t)(blockIdx.x % chunks) * kCombineCols + threadIdx.x * 4;
    if (c >= d) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int p = pos[t * k + j];
        if (p < 0) continue;  // an assignment the dispatch rejected (expert id out of range)
        const float g = gates[t * k + j];
        float4 v = *reinterpret_cast<const float4*>(Y + (int64_t)p * d + c);
        if (SPLIT) {  // the two K halves of the expert output, added in a fixed order
            const float4 v2 = *reinterpret_cast<const float4*>(Y2 + (int64_t)p * d + c);
            v.x += v2.x;
            v.y += v2.y;
            v.z += v2.z;
            v.w += v2.w;
        }
        acc.x = fmaf(g, v.x, acc.x);
        acc.y = fmaf(g, v.y, acc.y);
        acc.z = fmaf(g, v.z, acc.z);
        acc.w = fmaf(g, v.w, acc.w);
    }
    if constexpr (ACT == kF32) {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + t * d + c) = acc;
    } else {
        uint2 packed;
        packed.x = pack_bf16x2(acc.x, acc.y);
        packed.y = pack_bf16x2(acc.z, acc.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + t * d + c) = packed;
    }
}

}  // namespace

hipError_t launch_combine(const float* Y, const int32_t* pos, const float* gates, void* y, int64_t T, int64_t d,
                          int k, int act_dtype, hipStream_t stream, const float* Y2) {
    if (T == 0) return hipSuccess;
    const int chunks = (int)((d + kCombineCols - 1) / kCombineCols);
    const int64_t blocks = T * chunks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
#define MOE_COMBINE_LAUNCH(ACT_, SPLIT_)                                                                     \
    hipLaunchKernelGGL((combine_kernel<ACT_, SPLIT_>), dim3((unsigned)blocks), dim3(256), 0, stream, Y, Y2, pos, \
                       gates, y, d, k, chunks)
    if (act_dtype == kF32) {
        if (Y2) MOE_COMBINE_LAUNCH(kF32, true); else MOE_COMBINE_LAUNCH(kF32, false);
    } else {
        if (Y2) MOE_COMBINE_LAUNCH(kBF16, true); else MOE_COMBINE_LAUNCH(kBF16, false);
    }
#undef MOE_COMBINE_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
