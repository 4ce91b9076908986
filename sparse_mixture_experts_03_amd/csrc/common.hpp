// Internal helpers shared by the gfx950 kernels of the MoE-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Storage codes (match moe_dtype in include/moe.h).
constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kINT4 = 2;

// MFMA operand / accumulator vectors.
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two floats -> packed bf16 (lo in the low half), rounded to nearest even by
// gfx950's conversion instruction (v_cvt_pk_bf16_f32: one instruction per
// pair, no branch; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte load through the global address space (global_load_dwordx4, which
// counts only against vmcnt; a generic pointer would give a flat load whose
// completion also gates every LDS wait).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t global_u32x4;
__device__ __forceinline__ uint4 ldg16(const void* p) {
    const u32x4_t v = *(global_u32x4*)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, eight k-values each from k-block
// (l / 16); it receives D[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B, eight k-values each from k-block
// (l / 32); it receives D[8*(v/4) + 4*(l/32) + (v%4)][l % 32] in element v,
// v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Expert ranking of the router and of capacity rerouting: is (za, ea) ranked
// before (zb, eb)?  Larger z first, NaN last, ties to the lower expert index.
__device__ __forceinline__ bool ranks_before(double za, int ea, double zb, int eb) {
    bool na = isnan(za), nb = isnan(zb);
    if (na != nb) return nb;
    if (!na && za != zb) return za > zb;
    return ea < eb;
}

constexpr int kNoExpert = 0x7fffffff;

__device__ __forceinline__ float gelu_erf(float h) {
    return 0.5f * h * (1.0f + erff(h * 0.70710678118654752440f));
}

// GeLU h * Phi(h) for results rounded to bf16: Phi from erf by Abramowitz &
// Stegun's rational approximation 7.1.26, erf(x) = 1 - q(x) for x >= 0 with
// q = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-x^2), t = 1 / (1 + p x),
// |error| <= 1.5e-7, evaluated with the hardware base-2 exponential and
// reciprocal.  With x = |h| / sqrt 2: GeLU(h) = h - h q / 2 for h >= 0 and
// h q / 2 for h < 0 (absolute error below 2e-7 |h|, far under the 2^-9
// relative rounding of bf16).  One branch-free path: no lane divergence.
__device__ __forceinline__ float gelu_bf16(float h) {
    const float x = fabsf(h) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
    float poly = fmaf(t, 1.061405429f, -1.453152027f);
    poly = fmaf(t, poly, 1.421413741f);
    poly = fmaf(t, poly, -0.284496736f);
    poly = fmaf(t, poly, 0.254829592f);
    const float q = t * poly * __builtin_amdgcn_exp2f(-(x * x) * 1.4426950408889634f);
    const float hq = 0.5f * h * q;
    return h >= 0.0f ? h - hq : hq;
}

// SiLU (swish): a * sigmoid(a) = a / (1 + 2^(-a log2 e)), with the hardware
// base-2 exponential and reciprocal (each about 1 ulp; the result is rounded
// to bf16 or enters an fp32 product).  Few live temporaries: it sits in the
// epilogue of kernels whose main loops use nearly every register.
__device__ __forceinline__ float silu_f(float a) {
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}

// Expert activation codes (match moe_expert_act in include/moe.h).  SwiGLU's
// first GEMM has 2 d_ff weight rows interleaved in blocks of 16: rows
// [32 b, 32 b + 16) are the gate rows of hidden units [16 b, 16 b + 16) and
// the next 16 rows their up rows, so a 32-row block of outputs yields 16 units.
constexpr int kActGelu = 0;
constexpr int kActSilu = 1;
constexpr int kActSwiglu = 2;

// The elementwise activation of GEMM1 (GeLU or SiLU) for a bf16 H.
__device__ __forceinline__ float act_f(float v, int act) { return act == kActSilu ? silu_f(v) : gelu_bf16(v); }

// The m-tiles of a grouped GEMM whose experts hold offsets[e+1]-offsets[e]
// rows, cut into tiles of BM rows and numbered expert-major.  Built by one
// whole wavefront (every lane gets the same total); E <= 256, 4 experts per
// lane.
struct MtileScan {
    int tiles[4], begin[4], end[4];  // this lane's experts 4 lane .. 4 lane + 3: tiles, rows [begin, end)
    int excl, incl;                  // m-tiles of the experts before / up to this lane's
    int total;                       // all m-tiles
};

// Only experts whose row count n satisfies rows_lo < n <= rows_hi get tiles.
__device__ __forceinline__ MtileScan scan_mtiles(const int32_t* __restrict__ offsets, int E, int BM, int rows_lo = 0,
                                                 int rows_hi = 0x7fffffff) {
    const int lane = threadIdx.x & 63;
    MtileScan s;
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        int n = 0, b = 0, end = 0;
        if (e < E) {
            b = offsets[e];
            end = offsets[e + 1];
            n = end - b;
            if (n <= rows_lo || n > rows_hi) n = 0;
        }
        s.begin[j] = b;
        s.end[j] = end;
        s.tiles[j] = (n + BM - 1) / BM;
        local += s.tiles[j];
    }
    // inclusive scan of per-lane tile counts across the wavefront
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    s.incl = incl;
    s.excl = incl - local;
    s.total = __shfl(incl, 63, 64);
    return s;
}

// (expert, first dispatch position, rows) of m-tile mt < s.total; called by
// the whole wavefront that built s (no memory access: the scan kept each
// expert's row range).
__device__ __forceinline__ void lookup_mtile(const MtileScan& s, const int32_t* __restrict__ offsets, int BM, int mt,
                                             int* expert, int* pos0, int* rows) {
    (void)offsets;
    const int lane = threadIdx.x & 63;
    const unsigned long long hit = __ballot(mt >= s.excl && mt < s.incl);  // the lane whose range holds mt
    const int src = __ffsll((long long)hit) - 1;
    int e_found = -1, p0 = 0, r = 0;
    if (lane == src) {
        int acc = s.excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (e_found < 0 && mt < acc + s.tiles[j]) {
                e_found = lane * 4 + j;
                p0 = s.begin[j] + (mt - acc) * BM;
                r = min(BM, s.end[j] - p0);
            }
            acc += s.tiles[j];
        }
    }
    *expert = __shfl(e_found, src, 64);
    *pos0 = __shfl(p0, src, 64);
    *rows = __shfl(r, src, 64);
}

// Map a flat m-tile index onto (expert, first dispatch position, rows).
// Returns false when mt lies beyond the last real tile.  Called by one whole
// wavefront.
__device__ __forceinline__ bool find_mtile(const int32_t* __restrict__ offsets, int E, int BM, int mt, int* expert,
                                           int* pos0, int* rows, int rows_lo = 0, int rows_hi = 0x7fffffff) {
    const MtileScan s = scan_mtiles(offsets, E, BM, rows_lo, rows_hi);
    if (mt >= s.total) return false;
    lookup_mtile(s, offsets, BM, mt, expert, pos0, rows);
    return true;
}

}  // namespace moe
