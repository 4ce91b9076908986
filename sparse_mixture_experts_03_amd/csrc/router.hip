// Router: logits l = x . Wg (+ b), optional Gumbel noise, temperature, top-k
// and softmax gates.
//
// P2 §2.2 (single linear layer + softmax, top-2, outputs weighted by their
// confidences), P5 §3.2 (h x W_router with W_router a d x E matrix), P1 §3.1
// (Gumbel noise -ln(-ln u) and temperature tau before the softmax and top-k).
// P4 §4.2 prints a Triton gating kernel that tiles tokens x experts and keeps
// the top-2 per row; here the skinny d x E product is split over the input
// dimension across many workgroups (the decode case has only a handful of
// tokens) and a second kernel finishes each token on one 64-lane wavefront.
//
// Logits accumulate in binary64 from exact products (bf16*bf16 and
// fp32*fp32 are exact in binary64), so expert choices agree with a binary64
// reference except at ties closer than the binary64 rounding of the sums.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kTT = 8;           // tokens per partial-logit workgroup
constexpr int kRowChunk = 128;   // input rows staged in LDS per step
constexpr int kMaxSplits = 64;

// Eight consecutive experts of one Wg row (Wg is d x E row-major), as floats.
// Vector loads when every row holds whole groups of eight (E % 8 == 0).
template <int ACT>
__device__ __forceinline__ void load_wg8(const void* Wg, int64_t row, int E, int e0, bool vec, float w[8]) {
    if constexpr (ACT == kBF16) {
        const uint16_t* p = static_cast<const uint16_t*>(Wg) + row * E + e0;
        if (vec) {
            uint4 v = *reinterpret_cast<const uint4*>(p);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w[2 * j] = __uint_as_float(u[j] << 16);
                w[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = (e0 + j < E) ? bf16_bits_to_float(p[j]) : 0.0f;
        }
    } else {
        const float* p = static_cast<const float*>(Wg) + row * E + e0;
        if (vec) {
            float4 a = *reinterpret_cast<const float4*>(p);
            float4 b = *reinterpret_cast<const float4*>(p + 4);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = (e0 + j < E) ? p[j] : 0.0f;
        }
    }
}

template <int ACT>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
    if constexpr (ACT == kF32) {
        return static_cast<const float*>(p)[i];
    } else {
        return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
    }
}

// Partial logits of an 8-token tile over one slice of the input dimension.
// Thread (eg, rl): expert group eg (8 consecutive experts) and row lane rl;
// it accumulates 8 tokens x 8 experts in binary64 over rows k = rl (mod RL).
// Row lanes are then reduced with a fixed butterfly inside each wavefront and
// a fixed-order sum over the four wavefronts.
// grid = (token tiles, splits); partial is [splits][T][E] binary64.
template <int ACT>
__global__ void __launch_bounds__(kRouterThreads)
router_partial_kernel(const void* __restrict__ x, const void* __restrict__ Wg, int T, int d, int E, int egp,
                      int rows_per_split, double* __restrict__ partial) {
    __shared__ float xs[kRowChunk][kTT];      // staged x slice, token fastest
    __shared__ double red[4][32][kTT * 8];    // per-wave sums, 64 KB
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int eg = tid & (egp - 1);
    const int rl = tid / egp;
    const int RL = kRouterThreads / egp;
    const int e0 = eg * 8;
    const bool active = e0 < E;
    const bool vec = E % 8 == 0;
    const int t0 = blockIdx.x * kTT;
    const int k_begin = blockIdx.y * rows_per_split;
    const int k_end = min(d, k_begin + rows_per_split);

    double acc[kTT][8];
#pragma unroll
    for (int t = 0; t < kTT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = 0.0;

    for (int kc = k_begin; kc < k_end; kc += kRowChunk) {
        const int rows = min(kRowChunk, k_end - kc);
        for (int i = tid; i < kRowChunk * kTT; i += kRouterThreads) {
            const int t = i / kRowChunk, kk = i % kRowChunk;
            xs[kk][t] = (t0 + t < T && kk < rows) ? load_act<ACT>(x, (int64_t)(t0 + t) * d + kc + kk) : 0.0f;
        }
        __syncthreads();
        if (active) {
            for (int kk = rl; kk < rows; kk += RL) {
                float w[8];
                load_wg8<ACT>(Wg, kc + kk, E, e0, vec, w);
                const float4 xa = *reinterpret_cast<const float4*>(&xs[kk][0]);
                const float4 xb = *reinterpret_cast<const float4*>(&xs[kk][4]);
                const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                for (int t = 0; t < kTT; ++t)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[t][j] = fma((double)xv[t], (double)w[j], acc[t][j]);
            }
        }
        __syncthreads();
    }
    // butterfly over the row-lane bits of the lane index
    for (int off = egp; off < 64; off <<= 1) {
#pragma unroll
        for (int t = 0; t < kTT; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[t][j] += __shfl_xor(acc[t][j], off, 64);
    }
    if (lane < egp) {
#pragma unroll
        for (int t = 0; t < kTT; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j) red[wave][lane][t * 8 + j] = acc[t][j];
    }
    __syncthreads();
    for (int i = tid; i < kTT * E; i += kRouterThreads) {
        const int t = i / E, e = i % E;
        if (t0 + t >= T) continue;
        const int g = e / 8, j = e % 8;
        const double v = ((red[0][g][t * 8 + j] + red[1][g][t * 8 + j]) + red[2][g][t * 8 + j]) + red[3][g][t * 8 + j];
        partial[((int64_t)blockIdx.y * T + t0 + t) * E + e] = v;
    }
}

// Partial logits by fp64 MFMA, for bf16 activations at prefill sizes.  Each
// wavefront owns TT x ET tiles of 16 tokens x 16 experts over one slice of
// the input dimension, accumulated by v_mfma_f64_16x16x4 (binary64 products of
// the exact bf16 inputs, binary64 sums).  In each 16x16x4 step lane group g
// (lanes 16 g .. 16 g + 15) supplies input row kb + 8 g + j to both operands
// (A: the lane's token, B: the lane's expert); the sum over k is the same
// whatever row each group takes, and this choice lets a lane fetch its x
// values for 32 rows with one 16-byte load.  Its Wg values are eight 2-byte
// loads of L2-resident rows.  Loads run one 32-row chunk ahead.  Workgroup:
// 4 wavefronts along tokens (TT = 4, ET = 1, E <= 16) or 2 x 2 (TT = 4, ET = 2:
// 64 tokens x 32 experts per wavefront; 2 x 2 tiles measured 10% slower at
// T = 2048, E = 128).
typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
constexpr int kMfmaMinTokens = 64;
constexpr int kMfmaChunk = 32;  // input rows per loop step

template <int TT, int ET>
__global__ void __launch_bounds__(256)
router_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg, int T, int d, int E,
                   int rows_per_split, double* __restrict__ partial) {
    constexpr int WT = (ET == 1) ? 4 : 2;  // wavefronts along tokens
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt = wave % WT, we = wave / WT;
    const int t0 = (blockIdx.x * WT + wt) * (16 * TT);
    const int e0 = (blockIdx.y * (4 / WT) + we) * (16 * ET);
    const int k_begin = blockIdx.z * rows_per_split;
    const int k_end = min(d, k_begin + rows_per_split);
    // rows past T or columns past E read a valid row / column; their outputs are not stored
    const uint16_t* xr[TT];
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) xr[ti] = x + (int64_t)min(t0 + 16 * ti + r, T - 1) * d + 8 * g;
    const uint16_t* wc[ET];
#pragma unroll
    for (int ei = 0; ei < ET; ++ei) wc[ei] = Wg + (int64_t)(8 * g) * E + min(e0 + 16 * ei + r, E - 1);
    f64x4 acc[TT][ET];
#pragma unroll
    for (int ti = 0; ti < TT; ++ti)
#pragma unroll
        for (int ei = 0; ei < ET; ++ei) acc[ti][ei] = (f64x4){0.0, 0.0, 0.0, 0.0};
    uint4 xv[TT], xn[TT];
    uint16_t wv[ET][8], wn[ET][8];
    auto load = [&](int kb, uint4 (&xs)[TT], uint16_t (&ws)[ET][8]) {
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) xs[ti] = *reinterpret_cast<const uint4*>(xr[ti] + kb);
#pragma unroll
        for (int ei = 0; ei < ET; ++ei)
#pragma unroll
            for (int j = 0; j < 8; ++j) ws[ei][j] = wc[ei][(int64_t)(kb + j) * E];
    };
    if (k_begin < k_end) load(k_begin, xv, wv);
    for (int kb = k_begin; kb < k_end; kb += kMfmaChunk) {
        if (kb + kMfmaChunk < k_end) load(kb + kMfmaChunk, xn, wn);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            double a[TT], b[ET];
#pragma unroll
            for (int ti = 0; ti < TT; ++ti) {
                const uint32_t word = (j >> 1) == 0 ? xv[ti].x : (j >> 1) == 1 ? xv[ti].y : (j >> 1) == 2 ? xv[ti].z : xv[ti].w;
                a[ti] = (double)__uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
            }
#pragma unroll
            for (int ei = 0; ei < ET; ++ei) b[ei] = (double)bf16_bits_to_float(wv[ei][j]);
#pragma unroll
            for (int ti = 0; ti < TT; ++ti)
#pragma unroll
                for (int ei = 0; ei < ET; ++ei)
                    acc[ti][ei] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ti], b[ei], acc[ti][ei], 0, 0, 0);
        }
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) xv[ti] = xn[ti];
#pragma unroll
        for (int ei = 0; ei < ET; ++ei)
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[ei][j] = wn[ei][j];
    }
    // result i of lane (r, g) is row g + 4 i, column r of its 16 x 16 tile (the f64
    // layout interleaves rows, unlike the f32 16x16 shapes: measured)
#pragma unroll
    for (int ti = 0; ti < TT; ++ti)
#pragma unroll
        for (int ei = 0; ei < ET; ++ei) {
            const int e = e0 + 16 * ei + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * ti + g + 4 * i;
                if (t < T && e < E) partial[((int64_t)blockIdx.z * T + t) * E + e] = acc[ti][ei][i];
            }
        }
}

// Philox4x64-10 (Salmon et al., SC'11): two 64x64->128 products per round,
// key bumped by the Weyl constants between rounds.  Counter (c0, c1, 0, 0),
// key (k0, k1); all four output words.
struct PhiloxBlock {
    uint64_t w[4];
};
__device__ __forceinline__ PhiloxBlock philox_block(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t k1) {
    uint64_t x0 = c0, x1 = c1, x2 = 0, x3 = 0;
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
        uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
        uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
        x0 = y0;
        x1 = lo1;
        x2 = y2;
        x3 = lo0;
        k0 += 0x9E3779B97F4A7C15ULL;
        k1 += 0xBB67AE8584CAA73BULL;
    }
    PhiloxBlock b;
    b.w[0] = x0;
    b.w[1] = x1;
    b.w[2] = x2;
    b.w[3] = x3;
    return b;
}

// A uniform strictly inside (0, 1) from the top 53 bits of a word plus half an ulp.
__device__ __forceinline__ double open_uniform(uint64_t w) { return ((double)(w >> 11) + 0.5) * 0x1.0p-53; }

// Router noise of one (token, expert) key, before the temperature: the Gumbel
// draw -ln(-ln u) from word 0 (P1 §3.1) and sigma times a standard normal by
// Box-Muller, sqrt(-2 ln u1) cos(2 pi u2), from words 2 and 3 (P5 §3.3).
__device__ __forceinline__ double router_noise(double l, int use_gumbel, double noise_std, uint64_t seed,
                                               uint64_t token, uint64_t expert) {
    const PhiloxBlock b = philox_block(token, expert, seed, 0);
    double v = l + (use_gumbel ? -log(-log(open_uniform(b.w[0]))) : 0.0);
    if (noise_std > 0.0) {
        const double two_pi = 6.283185307179586;  // 2 pi rounded to binary64
        v += noise_std * (sqrt(-2.0 * log(open_uniform(b.w[2]))) * cos(two_pi * open_uniform(b.w[3])));
    }
    return v;
}

// One token per workgroup (E > 64) or per wavefront (E <= 64, four tokens per
// workgroup).  Thread e of the token sums the split partials of expert e (all
// loads issued before the adds, summed in split order), adds bias and noise
// and applies the temperature; the token's first wavefront then picks the
// top-k and forms the softmax gates from the E values in LDS.  The values and
// the order of every operation are the same in both arrangements.
template <bool kWavePerToken>
__global__ void __launch_bounds__(256)
router_finalize_kernel(const double* __restrict__ partial, int nsplit, int T, int E, int k,
                       const float* __restrict__ bias, double tau, int use_gumbel, double noise_std,
                       int gate_norm, uint64_t seed, uint64_t token_offset, int32_t* __restrict__ ids,
                       float* __restrict__ gates,
                       double* __restrict__ prob_rows, double* __restrict__ entropy_rows,
                       double* __restrict__ z_rows) {
    __shared__ double zs_all[256];
    __shared__ int sel_all[4][8];  // the chosen experts, best first
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int t = kWavePerToken ? blockIdx.x * 4 + wave : blockIdx.x;
    const int e_own = kWavePerToken ? (tid & 63) : tid;  // the expert this thread sums
    double* const zs = kWavePerToken ? zs_all + 64 * wave : zs_all;
    int* const sel = sel_all[kWavePerToken ? wave : 0];
    if (kWavePerToken && t >= T) return;  // whole wavefronts
    if (e_own < E) {
        const double* src = partial + (int64_t)t * E + e_own;
        const int64_t step = (int64_t)T * E;
        double v[kMaxSplits];
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < nsplit) v[s] = src[s * step];
        double l = 0.0;
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < nsplit) l += v[s];
        if (bias) l += (double)bias[e_own];
        if (use_gumbel || noise_std > 0.0)
            l = router_noise(l, use_gumbel, noise_std, seed, token_offset + (uint64_t)t, (uint64_t)e_own);
        zs[e_own] = l / tau;
    }
    // one wavefront per token reads back only its own LDS writes, which complete in order
    if constexpr (!kWavePerToken) {
        __syncthreads();
        if (tid >= 64) return;
    }
    const int lane = tid & 63;
    double z[4];
    bool live[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        live[j] = e < E;
        z[j] = live[j] ? zs[e] : 0.0;
    }
    // softmax denominator over all experts (max-subtracted)
    double m = -INFINITY;
    bool any_nan = false;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (live[j]) {
            if (isnan(z[j])) any_nan = true;
            else m = fmax(m, z[j]);
        }
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
    any_nan = __any(any_nan);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (live[j]) s += exp(z[j] - m);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (z_rows) {  // capacity-limited dispatch reranks overflowing tokens
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (live[j]) z_rows[(int64_t)t * E + lane + 64 * j] = z[j];
    }
    if (prob_rows) {
        // this token's full softmax row, and (router statistics) its entropy -sum p ln p (0 ln 0 = 0)
        double h = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (live[j]) {
                const double p = any_nan ? (double)NAN : exp(z[j] - m) / s;
                prob_rows[(int64_t)t * E + lane + 64 * j] = p;
                if (!(p == 0.0)) h -= p * log(p);
            }
        for (int off = 32; off >= 1; off >>= 1) h += __shfl_xor(h, off, 64);
        if (lane == 0 && entropy_rows) entropy_rows[t] = h;
    }
    // top-k by repeated wavefront argmax
    bool taken[4] = {false, false, false, false};
    for (int r = 0; r < k; ++r) {
        double bz = 0.0;
        int be = kNoExpert;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            if (live[j] && !taken[j] && (be == kNoExpert || ranks_before(z[j], e, bz, be))) {
                bz = z[j];
                be = e;
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const double oz = __shfl_xor(bz, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oe != kNoExpert && (be == kNoExpert || ranks_before(oz, oe, bz, be))) {
                bz = oz;
                be = oe;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane + 64 * j == be) taken[j] = true;
        if (lane == 0) {
            ids[(int64_t)t * k + r] = be;
            sel[r] = be;
            const double p = any_nan ? (double)NAN : exp(bz - m) / s;
            gates[(int64_t)t * k + r] = (float)p;
        }
    }
    if (gate_norm && lane == 0) {
        // softmax over the chosen z (P4 §4.3), max-subtracted at the best, summed in slot order
        const double top = zs[sel[0]];
        double den = 0.0;
        for (int r = 0; r < k; ++r) den += exp(zs[sel[r]] - top);
        for (int r = 0; r < k; ++r) gates[(int64_t)t * k + r] = (float)(exp(zs[sel[r]] - top) / den);
    }
}

}  // namespace

RouterPlan router_plan(int64_t T, int64_t d, int E) {
    RouterPlan p;
    p.tokens_per_tile = kTT;
    p.tiles = (int)((T + kTT - 1) / kTT);
    int egp = 1;
    while (egp * 8 < E) egp <<= 1;
    p.expert_groups = egp;
    // Enough workgroups to spread the d x E gating matrix over the chip
    // (~256), each split at least one 256-row chunk, at most 64 splits.
    const int nchunks = (int)((d + kRowChunk - 1) / kRowChunk);
    int want = p.tiles > 0 ? (256 + p.tiles - 1) / p.tiles : 1;
    if (want > nchunks) want = nchunks;
    if (want > kMaxSplits) want = kMaxSplits;
    if (want < 1) want = 1;
    const int chunks_per_split = (nchunks + want - 1) / want;
    p.rows_per_split = chunks_per_split * kRowChunk;
    p.splits = (nchunks + chunks_per_split - 1) / chunks_per_split;
    // fp64-MFMA kernel: about 512 workgroups, at least 128 input rows per split
    const int64_t tok_wg = E <= 16 ? 256 : 128, exp_wg = E <= 16 ? 16 : 64;
    const int64_t wgs = ((T + tok_wg - 1) / tok_wg) * ((E + exp_wg - 1) / exp_wg);
    int64_t ms = wgs > 0 ? (512 + wgs - 1) / wgs : 1;
    ms = std::min<int64_t>(ms, std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, d / 128)));
    const int64_t chunks = (d + kMfmaChunk - 1) / kMfmaChunk;
    const int64_t cps = (chunks + ms - 1) / ms;
    p.mfma_rows_per_split = (int)(cps * kMfmaChunk);
    p.mfma_splits = (int)((chunks + cps - 1) / cps);
    p.partial_bytes = (size_t)std::max(p.splits, p.mfma_splits) * (size_t)T * (size_t)E * sizeof(double);
    return p;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const RouterPlan p = router_plan(a.T, a.d, a.E);
    int nsplit = p.splits;
    if (a.act_dtype == kBF16 && a.T >= kMfmaMinTokens) {
        nsplit = p.mfma_splits;
        const uint16_t* xb = static_cast<const uint16_t*>(a.x);
        const uint16_t* wb = static_cast<const uint16_t*>(a.Wg);
        if (a.E <= 16) {
            dim3 grid((unsigned)((a.T + 255) / 256), 1, (unsigned)p.mfma_splits);
            hipLaunchKernelGGL((router_mfma_kernel<4, 1>), grid, dim3(256), 0, stream, xb, wb, (int)a.T, (int)a.d, a.E,
                               p.mfma_rows_per_split, a.partial);
        } else {
            dim3 grid((unsigned)((a.T + 127) / 128), (unsigned)((a.E + 63) / 64), (unsigned)p.mfma_splits);
            hipLaunchKernelGGL((router_mfma_kernel<4, 2>), grid, dim3(256), 0, stream, xb, wb, (int)a.T, (int)a.d, a.E,
                               p.mfma_rows_per_split, a.partial);
        }
    } else if (a.act_dtype == kF32) {
        dim3 grid1(p.tiles, p.splits);
        hipLaunchKernelGGL(router_partial_kernel<kF32>, grid1, dim3(kRouterThreads), 0, stream, a.x, a.Wg, (int)a.T,
                           (int)a.d, a.E, p.expert_groups, p.rows_per_split, a.partial);
    } else {
        dim3 grid1(p.tiles, p.splits);
        hipLaunchKernelGGL(router_partial_kernel<kBF16>, grid1, dim3(kRouterThreads), 0, stream, a.x, a.Wg,
                           (int)a.T, (int)a.d, a.E, p.expert_groups, p.rows_per_split, a.partial);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.E <= 64)
        hipLaunchKernelGGL(router_finalize_kernel<true>, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, stream,
                           a.partial, nsplit, (int)a.T, a.E, a.k, a.bias, (double)a.tau, a.use_gumbel,
                           (double)a.noise_std, a.gate_norm, a.seed, a.token_offset, a.ids, a.gates, a.prob_rows,
                           a.entropy_rows, a.z_rows);
    else
        hipLaunchKernelGGL(router_finalize_kernel<false>, dim3((unsigned)a.T), dim3(256), 0, stream, a.partial,
                           nsplit, (int)a.T, a.E, a.k, a.bias, (double)a.tau, a.use_gumbel, (double)a.noise_std,
                           a.gate_norm, a.seed, a.token_offset, a.ids, a.gates, a.prob_rows, a.entropy_rows,
                           a.z_rows);
    return hipGetLastError();
}

}  // namespace moe
