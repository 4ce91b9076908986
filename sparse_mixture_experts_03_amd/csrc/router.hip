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
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterKC = 32;          // input columns staged per step (LDS <= 33 KB at E = 256)
constexpr int kRouterPairsPerThread = 4;  // (token, expert) pairs per thread: TT*E <= 1024

template <int ACT>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
    if constexpr (ACT == kF32) {
        return static_cast<const float*>(p)[i];
    } else {
        return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
    }
}

// Partial logits over one slice of the input dimension.
// grid = (token tiles, splits); partial is [splits][T][E] binary64.
template <int ACT>
__global__ void __launch_bounds__(kRouterThreads)
router_partial_kernel(const void* __restrict__ x, const void* __restrict__ Wg, int T, int d, int E,
                      int TT, int chunks_per_split, double* __restrict__ partial) {
    extern __shared__ float smem[];
    const int xs_stride = kRouterKC + 1;
    float* xs = smem;                      // [TT][KC+1]
    float* ws = smem + TT * xs_stride;     // [KC][E]
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * TT;
    const int split = blockIdx.y;
    const int k_begin = split * chunks_per_split * kRouterKC;
    const int k_end = min(d, k_begin + chunks_per_split * kRouterKC);
    const int npairs = TT * E;

    double acc[kRouterPairsPerThread];
#pragma unroll
    for (int j = 0; j < kRouterPairsPerThread; ++j) acc[j] = 0.0;

    for (int kc = k_begin; kc < k_end; kc += kRouterKC) {
        for (int i = tid; i < TT * kRouterKC; i += kRouterThreads) {
            int tt = i / kRouterKC, kk = i % kRouterKC;
            int t = t0 + tt, kx = kc + kk;
            xs[tt * xs_stride + kk] = (t < T && kx < k_end) ? load_act<ACT>(x, (int64_t)t * d + kx) : 0.0f;
        }
        for (int i = tid; i < kRouterKC * E; i += kRouterThreads) {
            int kk = i / E, e = i % E;
            int kx = kc + kk;
            ws[i] = (kx < k_end) ? load_act<ACT>(Wg, (int64_t)kx * E + e) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRouterPairsPerThread; ++j) {
            int p = tid + j * kRouterThreads;
            if (p < npairs) {
                int tt = p / E, e = p % E;
                const float* xr = xs + tt * xs_stride;
                double a = acc[j];
                for (int kk = 0; kk < kRouterKC; ++kk)
                    a = fma((double)xr[kk], (double)ws[kk * E + e], a);
                acc[j] = a;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kRouterPairsPerThread; ++j) {
        int p = tid + j * kRouterThreads;
        if (p < npairs) {
            int tt = p / E, e = p % E;
            int t = t0 + tt;
            if (t < T) partial[((int64_t)split * T + t) * E + e] = acc[j];
        }
    }
}

// Philox4x64-10 (Salmon et al., SC'11): two 64x64->128 products per round,
// key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t k1) {
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
    return x0;
}

__device__ __forceinline__ double gumbel_draw(uint64_t seed, uint64_t token, uint64_t expert) {
    uint64_t r0 = philox_word0(token, expert, seed, 0);
    double u = ((double)(r0 >> 11) + 0.5) * 0x1.0p-53;
    return -log(-log(u));
}

// Is (za, ea) ranked before (zb, eb)?  Larger z first, NaN last, ties to the
// lower expert index.  Invalid slots carry e = INT_MAX and never win.
__device__ __forceinline__ bool ranks_before(double za, int ea, double zb, int eb) {
    bool na = isnan(za), nb = isnan(zb);
    if (na != nb) return nb;
    if (!na && za != zb) return za > zb;
    return ea < eb;
}

constexpr int kNoExpert = 0x7fffffff;

// One wavefront per token: sum the partial logits in split order, add bias
// and noise, apply the temperature, pick the top-k, and form the softmax gates.
__global__ void __launch_bounds__(256)
router_finalize_kernel(const double* __restrict__ partial, int nsplit, int T, int E, int k,
                       const float* __restrict__ bias, double tau, int use_gumbel, uint64_t seed,
                       uint64_t token_offset, int32_t* __restrict__ ids, float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    double z[4];
    bool live[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int e = lane + 64 * j;
        live[j] = e < E;
        z[j] = 0.0;
        if (live[j]) {
            double l = 0.0;
            for (int s = 0; s < nsplit; ++s) l += partial[((int64_t)s * T + t) * E + e];
            if (bias) l += (double)bias[e];
            double g = use_gumbel ? gumbel_draw(seed, token_offset + (uint64_t)t, (uint64_t)e) : 0.0;
            z[j] = (l + g) / tau;
        }
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
    // top-k by repeated wavefront argmax
    bool taken[4] = {false, false, false, false};
    for (int r = 0; r < k; ++r) {
        double bz = 0.0;
        int be = kNoExpert;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = lane + 64 * j;
            if (live[j] && !taken[j] && (be == kNoExpert || ranks_before(z[j], e, bz, be))) {
                bz = z[j];
                be = e;
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            double oz = __shfl_xor(bz, off, 64);
            int oe = __shfl_xor(be, off, 64);
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
            double p = any_nan ? (double)NAN : exp(bz - m) / s;
            gates[(int64_t)t * k + r] = (float)p;
        }
    }
}

}  // namespace

RouterPlan router_plan(int64_t T, int64_t d, int E) {
    RouterPlan p;
    int tt = 1024 / E;
    if (tt > 64) tt = 64;
    if (tt < 1) tt = 1;
    p.tokens_per_tile = tt;
    p.tiles = (int)((T + tt - 1) / tt);
    int nchunks = (int)((d + kRouterKC - 1) / kRouterKC);
    int want = p.tiles > 0 ? (512 + p.tiles - 1) / p.tiles : 1;
    if (want < 1) want = 1;
    if (want > nchunks) want = nchunks;
    p.chunks_per_split = (nchunks + want - 1) / want;
    p.splits = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
    p.partial_bytes = (size_t)p.splits * (size_t)T * (size_t)E * sizeof(double);
    return p;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    RouterPlan p = router_plan(a.T, a.d, a.E);
    dim3 grid1(p.tiles, p.splits);
    size_t lds = sizeof(float) * ((size_t)p.tokens_per_tile * (kRouterKC + 1) + (size_t)kRouterKC * a.E);
    if (a.act_dtype == kF32) {
        hipLaunchKernelGGL(router_partial_kernel<kF32>, grid1, dim3(kRouterThreads), lds, stream, a.x, a.Wg,
                           (int)a.T, (int)a.d, a.E, p.tokens_per_tile, p.chunks_per_split, a.partial);
    } else {
        hipLaunchKernelGGL(router_partial_kernel<kBF16>, grid1, dim3(kRouterThreads), lds, stream, a.x, a.Wg,
                           (int)a.T, (int)a.d, a.E, p.tokens_per_tile, p.chunks_per_split, a.partial);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    dim3 grid2((unsigned)((a.T + 3) / 4));
    hipLaunchKernelGGL(router_finalize_kernel, grid2, dim3(256), 0, stream, a.partial, p.splits, (int)a.T, a.E,
                       a.k, a.bias, (double)a.tau, a.use_gumbel, a.seed, a.token_offset, a.ids, a.gates);
    return hipGetLastError();
}

}  // namespace moe
