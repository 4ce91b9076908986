// LDS-tiled MFMA grouped expert GEMM for prefill-sized token counts.
//
// P3 §3.2: every expert is the same d -> 4d -> d GELU MLP with its own W1 and
// W2, so one kernel serves all experts; P3 §4.2 notes the per-expert work is
// really a grouped GEMM over the tokens scattered to each expert, and P2 §3.3
// credits fusing the activation into the expert GEMM.  Here:
//   workgroup tile = 128 weight rows x 128 dispatch rows (one expert), K in
//   steps of 64 through double-buffered, row-padded LDS;
//   4 wavefronts in a 2 x 2 arrangement, each 64 x 64 outputs as 4 x 4
//   MFMA 16x16x32 bf16 tiles with fp32 accumulation;
//   GEMM1's epilogue applies GeLU and stores bf16 H; GEMM2's stores fp32 Y.
// The m-tiles of all experts are numbered expert-major and located from the
// offsets on the device, so skewed loads (0 .. thousands of rows per expert)
// need no host round trip; tiles past the last real one exit at once.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTBN = 128;  // weight rows per tile
constexpr int kTBM = 128;  // dispatch rows per tile
constexpr int kTBK = 64;   // K per step
constexpr int kLdsStride = kTBK + 8;  // bf16 elements per LDS row (16-byte pad: conflict-free b128 reads)

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <int WHICH>
__global__ void __launch_bounds__(256, 2)
gemm_tiled_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                       const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ W,
                       int64_t W_stride_elems, void* __restrict__ out, int N, int K, int ntiles_n) {
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kTBN * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTBM * kLdsStride];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mt = blockIdx.x / ntiles_n;
    const int nt = blockIdx.x - mt * ntiles_n;
    int e, p0, rows;
    if (!find_mtile(offsets, E, kTBM, mt, &e, &p0, &rows)) return;
    const int n0 = nt * kTBN;
    const uint16_t* Wexp = W + (int64_t)e * W_stride_elems;

    // global -> register staging: 4 x 16 B of W and of X per thread per step
    const int lrow = tid >> 3;  // 0..31 (+32 per i)
    const int lcol = (tid & 7) * 8;
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[4];
    bool wok[4], xok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int row = lrow + 32 * i;
        wok[i] = n0 + row < N;  // N is a multiple of 64: the tile's upper half may lie past N
        wsrc[i] = Wexp + (int64_t)(wok[i] ? n0 + row : 0) * K + lcol;
        xok[i] = row < rows;
        int64_t arow = 0;
        if (xok[i]) arow = (WHICH == 1) ? (int64_t)a_rows[p0 + row] : (int64_t)(p0 + row);
        xsrc[i] = A + arow * K + lcol;
    }
    uint4 wreg[4], xreg[4];
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wreg[i] = wok[i] ? ld16(wsrc[i] + k0) : zero4;
            xreg[i] = xok[i] ? ld16(xsrc[i] + k0) : zero4;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = lrow + 32 * i;
            *reinterpret_cast<uint4*>(&Ws[buf][row * kLdsStride + lcol]) = wreg[i];
            *reinterpret_cast<uint4*>(&Xs[buf][row * kLdsStride + lcol]) = xreg[i];
        }
    };

    const int wn = (wave & 1) * 64;   // this wave's weight rows within the tile
    const int wm = (wave >> 1) * 64;  // this wave's dispatch rows within the tile
    const int r = lane & 15;
    const int g = lane >> 4;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int nk = K / kTBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kTBK);
#pragma unroll
        for (int ks = 0; ks < kTBK / 32; ++ks) {
            bf16x8 wf[4], xf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &Ws[buf][(wn + 16 * i + r) * kLdsStride + ks * 32 + 8 * g]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &Xs[buf][(wm + 16 * j + r) * kLdsStride + ks * 32 + 8 * g]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(wf[i], xf[j], acc[i][j]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds D[n = wn + 16i + 4g + q][m = wm + 16j + r]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = wm + 16 * j + r;
        if (m >= rows) continue;
        const int64_t orow = (int64_t)(p0 + m) * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + wn + 16 * i + 4 * g;
            if (n >= N) continue;
            f32x4 v = acc[i][j];
            if constexpr (WHICH == 1) {
                uint2 packed;
                packed.x = float_to_bf16_bits(gelu_erf(v[0])) | (float_to_bf16_bits(gelu_erf(v[1])) << 16);
                packed.y = float_to_bf16_bits(gelu_erf(v[2])) | (float_to_bf16_bits(gelu_erf(v[3])) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + n) = packed;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + n) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
    const int64_t Tk = a.T * a.k;
    const int64_t max_mtiles = Tk / kTBM + (Tk < a.E ? Tk : a.E);
    const int ntiles_n = (int)((a.N + kTBN - 1) / kTBN);
    const int64_t blocks = max_mtiles * ntiles_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    dim3 grid((unsigned)blocks), block(256);
    if (a.which == 1)
        hipLaunchKernelGGL(gemm_tiled_bf16_kernel<1>, grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                           a.W_stride / 2, a.out, (int)a.N, (int)a.K, ntiles_n);
    else
        hipLaunchKernelGGL(gemm_tiled_bf16_kernel<2>, grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                           a.W_stride / 2, a.out, (int)a.N, (int)a.K, ntiles_n);
    return hipGetLastError();
}

}  // namespace moe
