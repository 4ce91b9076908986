// fp32 grouped expert GEMM (fp32 experts with fp32 activations).
//
// Same grouped layout as the MFMA kernels (P3 §3.2 homogeneous experts, P3
// §4.2 grouped per-expert GEMM, GeLU fused into the first GEMM as in P2
// §3.3), computed with fp32 FMAs so that fp32 layers keep fp32 accuracy:
// 64 x 64 output tiles, K in steps of 16 through LDS, 4 x 4 outputs per thread.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kFB = 64;   // tile edge (dispatch rows and weight rows)
constexpr int kFK = 16;   // K per step

template <int WHICH>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, const int32_t* __restrict__ a_rows,
                const int32_t* __restrict__ offsets, int E, const float* __restrict__ W, int64_t W_stride_elems,
                float* __restrict__ out, int N, int K, int ntiles_n, int act) {
    __shared__ float As[kFK][kFB + 4];
    __shared__ float Bs[kFK][kFB + 4];
    const int tid = threadIdx.x;
    const int mt = blockIdx.x / ntiles_n;
    const int nt = blockIdx.x - mt * ntiles_n;
    int e, p0, rows;
    if (!find_mtile(offsets, E, kFB, mt, &e, &p0, &rows)) return;
    const int n0 = nt * kFB;
    const float* Wexp = W + (int64_t)e * W_stride_elems;

    const int lrow = tid >> 2;       // 0..63
    const int lk = (tid & 3) * 4;    // 0,4,8,12
    const bool aok = lrow < rows;
    int64_t arow = 0;
    if (aok) arow = (WHICH == 1) ? (int64_t)a_rows[p0 + lrow] : (int64_t)(p0 + lrow);
    const float* asrc = A + arow * K + lk;
    const float* wsrc = Wexp + (int64_t)(n0 + lrow) * K + lk;

    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < K; k0 += kFK) {
        float4 av = aok ? *reinterpret_cast<const float4*>(asrc + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 wv = *reinterpret_cast<const float4*>(wsrc + k0);
        As[lk + 0][lrow] = av.x;
        As[lk + 1][lrow] = av.y;
        As[lk + 2][lrow] = av.z;
        As[lk + 3][lrow] = av.w;
        Bs[lk + 0][lrow] = wv.x;
        Bs[lk + 1][lrow] = wv.y;
        Bs[lk + 2][lrow] = wv.z;
        Bs[lk + 3][lrow] = wv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kFK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    if (WHICH == 1 && act == kActSwiglu) {
        // weight rows 4 tx + j: tx % 8 < 4 holds gate rows of a 32-row block, tx + 4 the matching up rows
        float up[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) up[i][j] = __shfl_xor(acc[i][j], 4, 64);
        if ((tx & 4) == 0) {
            const int Nh = N >> 1;
            const int unit = (n0 >> 1) + 16 * (tx >> 3) + 4 * (tx & 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ty * 4 + i;
                if (m >= rows) continue;
                const float4 v = make_float4(silu_f(acc[i][0]) * up[i][0], silu_f(acc[i][1]) * up[i][1],
                                             silu_f(acc[i][2]) * up[i][2], silu_f(acc[i][3]) * up[i][3]);
                *reinterpret_cast<float4*>(out + (int64_t)(p0 + m) * Nh + unit) = v;
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = ty * 4 + i;
        if (m >= rows) continue;
        float4 v = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        if (WHICH == 1) {
            // fp32 H: the erff GeLU, not the bf16-grade one
            v.x = act == kActSilu ? silu_f(v.x) : gelu_erf(v.x);
            v.y = act == kActSilu ? silu_f(v.y) : gelu_erf(v.y);
            v.z = act == kActSilu ? silu_f(v.z) : gelu_erf(v.z);
            v.w = act == kActSilu ? silu_f(v.w) : gelu_erf(v.w);
        }
        *reinterpret_cast<float4*>(out + (int64_t)(p0 + m) * N + n0 + tx * 4) = v;
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t stream) {
    const int64_t Tk = a.T * a.k;
    const int64_t max_mtiles = Tk / kFB + (Tk < a.E ? Tk : a.E);
    const int ntiles_n = (int)(a.N / kFB);
    const int64_t blocks = max_mtiles * ntiles_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(256);
    const float* A = static_cast<const float*>(a.A);
    const float* W = static_cast<const float*>(a.W);
    float* out = static_cast<float*>(a.out);
    if (a.which == 1)
        hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                           a.W_stride / 4, out, (int)a.N, (int)a.K, ntiles_n, a.act);
    else
        hipLaunchKernelGGL(gemm_f32_kernel<2>, grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                           a.W_stride / 4, out, (int)a.N, (int)a.K, ntiles_n, 0);
    return hipGetLastError();
}

}  // namespace moe
