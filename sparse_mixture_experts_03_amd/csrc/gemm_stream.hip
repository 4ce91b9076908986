// Weight-streaming grouped expert GEMM for decode-sized token counts.
//
// P2 §2.3: at decode sizes the cost of an expert is moving its weights (the
// MoE layer there spends more time in weight traffic than in GEMM, and the
// weights never stay in cache).  This kernel therefore reads every weight of
// every active expert exactly once per 16 routed tokens and does the
// arithmetic on MFMA so that the matrix cores never limit the stream:
//   workgroup = 32 weight rows x one 16-row tile of the dispatch order;
//   its four wavefronts split K, each streaming 16-byte row segments straight
//   from HBM into MFMA operands (no LDS staging: nothing is reused);
//   the four partial tiles are summed in LDS in a fixed order (deterministic).
// MFMA operand roles are swapped (weights are the 16-row "A" side, tokens the
// "B" side) so each lane ends with four consecutive output features of one
// token and can store them with one vector store.
//
// INT4 experts (P1 §5.4 group-wise INT4 with scales; P2 §2.3 in-kernel
// dequantisation): a 16-byte code segment is 32 weights of one row inside one
// 128-wide scale group.  Codes become bf16 (136 + q) by bit operations alone
// (128 + (q + 8) has a fixed exponent), the MFMA sums (136 + q) x, an MFMA
// against ones sums x, and the group's partial is s * (sum - 136 * sum x), so
// the weights act as exactly q * s.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kStreamRows = 32;  // weight rows per workgroup (two 16-row MFMA tiles)
constexpr int kStreamBM = 16;    // dispatch rows per tile

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Eight signed INT4 codes (one 32-bit word, code i in bits 4i..4i+3) to eight
// bf16 values 136 + q_i, as one MFMA operand.
__device__ __forceinline__ bf16x8 int4x8_to_bf16_offset136(uint32_t w) {
    uint32_t v = w ^ 0x88888888u;                 // q + 8, offset binary
    uint32_t lo = v & 0x0f0f0f0fu;                 // codes 0,2,4,6 in byte 0..3
    uint32_t hi = (v >> 4) & 0x0f0f0f0fu;          // codes 1,3,5,7
    uint4 r;
    // dword p = bf16(128 + c[2p]) | bf16(128 + c[2p+1]) << 16 ; bf16(128 + c) = 0x4300 | c
    r.x = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u) | 0x43004300u;
    r.y = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u) | 0x43004300u;
    r.z = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u) | 0x43004300u;
    r.w = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u) | 0x43004300u;
    return as_bf16x8(r);
}

template <int WHICH>
__device__ __forceinline__ void store_tile(void* out, int64_t N, int p0, int rows, int n0, f32x4 v, int lane) {
    const int m = lane & 15;
    if (m >= rows) return;
    const int n = n0 + 4 * (lane >> 4);
    if constexpr (WHICH == 1) {
        uint2 packed;
        packed.x = float_to_bf16_bits(gelu_erf(v[0])) | (float_to_bf16_bits(gelu_erf(v[1])) << 16);
        packed.y = float_to_bf16_bits(gelu_erf(v[2])) | (float_to_bf16_bits(gelu_erf(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)(p0 + m) * N + n) = packed;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + (int64_t)(p0 + m) * N + n) =
            make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <int WQ, int WHICH>
__global__ void __launch_bounds__(256)
gemm_stream_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                   const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ W,
                   const uint16_t* __restrict__ Wsc, int64_t W_stride, void* __restrict__ out, int N, int K,
                   int ntiles_n) {
    __shared__ f32x4 red[3][2][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int mt = blockIdx.x / ntiles_n;
    const int nt = blockIdx.x - mt * ntiles_n;
    int e, p0, rows;
    if (!find_mtile(offsets, E, kStreamBM, mt, &e, &p0, &rows)) return;

    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = nt * kStreamRows;
    const bool mvalid = r < rows;
    int64_t arow = 0;
    if (mvalid) arow = (WHICH == 1) ? (int64_t)a_rows[p0 + r] : (int64_t)(p0 + r);
    const uint16_t* xrow = A + arow * K;
    const uint8_t* Wexp = W + (int64_t)e * W_stride;
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

    if constexpr (WQ == kBF16) {
        // chunk = 64 columns; lane group g covers columns [16g, 16g+16) of it
        const int nchunks = K / 64;
        const int c0 = wave * nchunks / 4, c1 = (wave + 1) * nchunks / 4;
        const uint16_t* w0 = reinterpret_cast<const uint16_t*>(Wexp) + (int64_t)(n0 + r) * K + 16 * g;
        const uint16_t* w1 = w0 + (int64_t)16 * K;
        const uint16_t* xg = xrow + 16 * g;
        int c = c0;
        for (; c + 4 <= c1; c += 4) {
            uint4 wa[4][2], wb[4][2], xv[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kb = (c + u) * 64;
                wa[u][0] = ld16(w0 + kb);
                wa[u][1] = ld16(w0 + kb + 8);
                wb[u][0] = ld16(w1 + kb);
                wb[u][1] = ld16(w1 + kb + 8);
                xv[u][0] = mvalid ? ld16(xg + kb) : zero4;
                xv[u][1] = mvalid ? ld16(xg + kb + 8) : zero4;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    acc0 = mfma16x16x32(as_bf16x8(wa[u][s]), as_bf16x8(xv[u][s]), acc0);
                    acc1 = mfma16x16x32(as_bf16x8(wb[u][s]), as_bf16x8(xv[u][s]), acc1);
                }
            }
        }
        for (; c < c1; ++c) {
            const int kb = c * 64;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uint4 xa = mvalid ? ld16(xg + kb + 8 * s) : zero4;
                acc0 = mfma16x16x32(as_bf16x8(ld16(w0 + kb + 8 * s)), as_bf16x8(xa), acc0);
                acc1 = mfma16x16x32(as_bf16x8(ld16(w1 + kb + 8 * s)), as_bf16x8(xa), acc1);
            }
        }
    } else {
        // chunk = one 128-column scale group; lane group g covers columns [32g, 32g+32)
        const int nchunks = K / 128;
        const int c0 = wave * nchunks / 4, c1 = (wave + 1) * nchunks / 4;
        const int64_t row_bytes = K / 2;
        const uint8_t* w0 = Wexp + (int64_t)(n0 + r) * row_bytes + 16 * g;
        const uint8_t* w1 = w0 + 16 * row_bytes;
        const uint16_t* xg = xrow + 32 * g;
        // scales of this lane's four output rows (4 * (lane/16) + i) in both tiles
        const int groups = K / 128;
        const uint16_t* sc = Wsc + (int64_t)e * N * groups + (int64_t)(n0 + 4 * g) * groups;
        const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
        for (int c = c0; c < c1; ++c) {
            uint4 q0 = ld16(w0 + (int64_t)c * 64);
            uint4 q1 = ld16(w1 + (int64_t)c * 64);
            uint4 xv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) xv[s] = mvalid ? ld16(xg + c * 128 + 8 * s) : zero4;
            f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0, sx = t0;
            const uint32_t qa[4] = {q0.x, q0.y, q0.z, q0.w};
            const uint32_t qb[4] = {q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 xb = as_bf16x8(xv[s]);
                t0 = mfma16x16x32(int4x8_to_bf16_offset136(qa[s]), xb, t0);
                t1 = mfma16x16x32(int4x8_to_bf16_offset136(qb[s]), xb, t1);
                sx = mfma16x16x32(as_bf16x8(ones), xb, sx);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s0 = bf16_bits_to_float(sc[(int64_t)i * groups + c]);
                float s1 = bf16_bits_to_float(sc[(int64_t)(16 + i) * groups + c]);
                acc0[i] = fmaf(s0, fmaf(-136.0f, sx[i], t0[i]), acc0[i]);
                acc1[i] = fmaf(s1, fmaf(-136.0f, sx[i], t1[i]), acc1[i]);
            }
        }
    }

    // fixed-order reduction of the four K-slices
    if (wave > 0) {
        red[wave - 1][0][lane] = acc0;
        red[wave - 1][1][lane] = acc1;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            acc0 += red[v][0][lane];
            acc1 += red[v][1][lane];
        }
        store_tile<WHICH>(out, N, p0, rows, n0, acc0, lane);
        store_tile<WHICH>(out, N, p0, rows, n0 + 16, acc1, lane);
    }
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
    const int64_t Tk = a.T * a.k;
    const int64_t max_mtiles = Tk / kStreamBM + (Tk < a.E ? Tk : a.E);
    const int ntiles_n = (int)(a.N / kStreamRows);
    const int64_t blocks = max_mtiles * ntiles_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    const uint8_t* W = static_cast<const uint8_t*>(a.W);
    const uint16_t* S = static_cast<const uint16_t*>(a.W_scales);
    dim3 grid((unsigned)blocks), block(256);
    if (a.w_dtype == kBF16) {
        if (a.which == 1)
            hipLaunchKernelGGL((gemm_stream_kernel<kBF16, 1>), grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                               S, a.W_stride, a.out, (int)a.N, (int)a.K, ntiles_n);
        else
            hipLaunchKernelGGL((gemm_stream_kernel<kBF16, 2>), grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                               S, a.W_stride, a.out, (int)a.N, (int)a.K, ntiles_n);
    } else {
        if (a.which == 1)
            hipLaunchKernelGGL((gemm_stream_kernel<kINT4, 1>), grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                               S, a.W_stride, a.out, (int)a.N, (int)a.K, ntiles_n);
        else
            hipLaunchKernelGGL((gemm_stream_kernel<kINT4, 2>), grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W,
                               S, a.W_stride, a.out, (int)a.N, (int)a.K, ntiles_n);
    }
    return hipGetLastError();
}

}  // namespace moe
