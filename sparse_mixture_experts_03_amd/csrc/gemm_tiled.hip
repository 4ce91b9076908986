// LDS-tiled MFMA grouped expert GEMM for prefill-sized token counts.
//
// P3 §3.2: every expert is the same d -> 4d -> d GELU MLP with its own W1 and
// W2, so one kernel serves all experts; P3 §4.2 notes the per-expert work is
// really a grouped GEMM over the tokens scattered to each expert, and P2 §3.3
// credits fusing the activation into the expert GEMM.  Here:
//   workgroup tile = 256 weight rows x 256 dispatch rows (one expert), K in
//   steps of 64;
//   tiles go straight from HBM/L2 into LDS with gfx950's global_load_lds
//   (16 bytes per lane, no register staging), double-buffered in four 32 KB
//   arrays: stage k+1 streams in while stage k is multiplied, one barrier per
//   step.  Every 128-byte tile row keeps its eight 16-byte segments in slots
//   permuted by (row & 7) (an XOR swizzle), so both the loads and the 16-row
//   MFMA fragment reads are free of LDS bank conflicts without padding;
//   4 wavefronts in a 2 x 2 arrangement, each 128 x 128 outputs as 16 MFMA
//   32x32x16 bf16 tiles with fp32 accumulation (256 accumulators in AGPRs:
//   64 flops per byte read from LDS);
//   GEMM1's epilogue applies GeLU and stores bf16 H; GEMM2's stores fp32 Y.
// The m-tiles of all experts are numbered expert-major and located from the
// offsets on the device, so skewed loads (0 .. thousands of rows per expert)
// need no host round trip; tiles past the last real one exit at once.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTBN = 256;   // weight rows per tile
constexpr int kTBM = 256;   // dispatch rows per tile
constexpr int kTBK = 64;    // K per step (128 bytes of every tile row)
constexpr int kTileBytes = 256 * kTBK * 2;

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// One wavefront copies 8 tile rows x 128 bytes (1 KB) of the current K step
// into LDS: lane L fetches logical segment (L & 7) ^ (L >> 3) of row L >> 3,
// which lands at LDS byte 16 * L of the 1 KB block, i.e. physical slot L & 7
// of that row.  `base` is wave-uniform and `off` a 32-bit byte offset (one
// expert's weights and every activation array stay below 4 GiB), so the load
// takes the scalar-base + vector-offset form.
__device__ __forceinline__ void copy_rows_to_lds(const char* base, uint32_t off, uint8_t* lds_block) {
    __builtin_amdgcn_global_load_lds((gvoid*)(base + off), (lvoid*)lds_block, 16, 0, 0);
}

// MFMA fragment: 8 bf16 of logical segment `seg` of tile row `row`.
__device__ __forceinline__ bf16x8 frag(const uint8_t* tile, int row, int seg) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(tile + row * 128 + 16 * (seg ^ (row & 7))));
}

template <int WHICH>
__global__ void __launch_bounds__(256, 1)
gemm_tiled_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                       const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ W,
                       int64_t W_stride_elems, void* __restrict__ out, int N, int K, int ntiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t Wt0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t Wt1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t Xt0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t Xt1[kTileBytes];

    // An (empty) statement that clobbers an AGPR tells the backend this kernel
    // uses AGPRs, so it gives the MFMAs their AGPR-accumulator form (256
    // accumulators live in AGPRs, operands in VGPRs) instead of VGPR-form
    // MFMAs with the AGPRs as spill space.
    asm volatile("" ::: "a0");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mt = blockIdx.x / ntiles_n;
    const int nt = blockIdx.x - mt * ntiles_n;
    int e, p0, rows;
    if (!find_mtile(offsets, E, kTBM, mt, &e, &p0, &rows)) return;
    const int n0 = nt * kTBN;
    const uint16_t* Wexp = W + (int64_t)e * W_stride_elems;

    // This wavefront copies tile rows [64 * wave, 64 * wave + 64) of both tiles,
    // 8 rows per instruction.  Rows past N (weights) or past the tile's
    // dispatch rows (tokens) are clamped to a valid row: they only feed
    // outputs that are never stored.
    const int lseg = (lane & 7) ^ (lane >> 3);
    const char* wbase = reinterpret_cast<const char*>(Wexp);
    const char* xbase = reinterpret_cast<const char*>(A);
    const uint32_t rowbytes = (uint32_t)K * 2;
    uint32_t woff[8], xoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int trow = 64 * wave + 8 * i + (lane >> 3);
        woff[i] = (uint32_t)min(n0 + trow, N - 1) * rowbytes + 16 * lseg;
        const int drow = min(trow, rows - 1);
        const uint32_t arow = (WHICH == 1) ? (uint32_t)a_rows[p0 + drow] : (uint32_t)(p0 + drow);
        xoff[i] = arow * rowbytes + 16 * lseg;
    }
    auto issue = [&](int kt, uint8_t* wt, uint8_t* xt) {
        const uint32_t kb = (uint32_t)kt * (kTBK * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            copy_rows_to_lds(wbase, woff[i] + kb, wt + (64 * wave + 8 * i) * 128);
            copy_rows_to_lds(xbase, xoff[i] + kb, xt + (64 * wave + 8 * i) * 128);
        }
    };

    const int wn = (wave & 1) * 128;   // this wave's weight rows within the tile
    const int wm = (wave >> 1) * 128;  // this wave's dispatch rows within the tile
    const int r = lane & 31;
    const int h = lane >> 5;
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // four k-substeps of 16: lane half h reads logical segment 2 * ks + h
    auto compute = [&](const uint8_t* wt, const uint8_t* xt) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 wf[4], xf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) wf[i] = frag(wt, wn + 32 * i + r, 2 * ks + h);
#pragma unroll
            for (int j = 0; j < 4; ++j) xf[j] = frag(xt, wm + 32 * j + r, 2 * ks + h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(wf[i], xf[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);  // bound the fragments in flight to one substep
        }
    };

    const int nk = K / kTBK;
    issue(0, Wt0, Xt0);
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue(kt + 1, Wt1, Xt1);
        compute(Wt0, Xt0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < nk) issue(kt + 2, Wt0, Xt0);
        compute(Wt1, Xt1);
    }
    if (kt < nk) {  // odd number of K steps: the last one sits in buffer 0
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        compute(Wt0, Xt0);
    }

    // epilogue: element v of acc[i][j] is D[n = wn + 32i + 8(v/4) + 4h + (v%4)][m = wm + 32j + r]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = wm + 32 * j + r;
        if (m >= rows) continue;
        const int64_t orow = (int64_t)(p0 + m) * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn + 32 * i + 8 * q + 4 * h;
                if (n >= N) continue;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if constexpr (WHICH == 1) {
                    uint2 packed;
                    packed.x = float_to_bf16_bits(gelu_erf(v0)) | (float_to_bf16_bits(gelu_erf(v1)) << 16);
                    packed.y = float_to_bf16_bits(gelu_erf(v2)) | (float_to_bf16_bits(gelu_erf(v3)) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + n) = packed;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + n) = make_float4(v0, v1, v2, v3);
                }
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
