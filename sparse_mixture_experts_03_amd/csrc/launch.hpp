// Host-side launchers of the library's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
struct RouterPlan {
    int tokens_per_tile;   // tokens per partial-logit workgroup
    int tiles;             // token tiles
    int expert_groups;     // power of two >= E / 8: 8-expert groups per Wg row
    int rows_per_split;    // input rows (of d) per split
    int splits;            // workgroups along the input dimension (<= 64)
    // bf16 activations with T >= 64: the fp64-MFMA partial kernel and its split
    int mfma_rows_per_split, mfma_splits;
    size_t partial_bytes;  // binary64 partial logits [splits][T][E], enough for either kernel
};
RouterPlan router_plan(int64_t T, int64_t d, int E);

struct RouterArgs {
    const void* x;
    const void* Wg;
    const float* bias;
    int64_t T, d;
    int E, k, act_dtype;
    float tau;
    int use_gumbel;
    float noise_std;     // Gaussian logit noise sigma (0: none)
    int gate_norm;       // 1: gates renormalised over the k chosen
    uint64_t seed, token_offset;
    double* partial;  // workspace, >= router_plan().partial_bytes
    int32_t* ids;
    float* gates;
    double* prob_rows = nullptr;     // optional [T][E]: every token's softmax row (router statistics)
    double* entropy_rows = nullptr;  // optional [T]: every token's -sum p ln p
    double* z_rows = nullptr;        // optional [T][E]: every token's (l + g) / tau
};
hipError_t launch_router(const RouterArgs& a, hipStream_t stream);

// ------------------------------------------------------ router statistics
// From prob_rows [T][E], entropy_rows [T] and ids [T][k]: fraction[E] =
// count_e / (T k), mean_prob[E] = sum_t p[t][e] / T and scalars[4] = { mean
// entropy, sum_e (fraction_e - 1/E)^2, sum_e (mean_prob_e - 1/E)^2, std of
// fraction }.  scratch: >= stats_scratch_bytes(E).  T >= 1.
size_t stats_scratch_bytes(int E);
hipError_t launch_router_stats(const double* prob_rows, const double* entropy_rows, const int32_t* ids, int64_t T,
                               int E, int k, void* scratch, double* fraction, double* mean_prob, double* scalars,
                               hipStream_t stream);
// ------------------------------------------------ capacity-limited dispatch
// In place on ids/gates [T][k] (the top-k routing), given the stable
// permutation of that routing (pos, offsets, counts from launch_permute), the
// [T][E] rows z (ranking) and p (gates), the capacity 1 <= cap <= T and the
// policy (0 drop, 1 reroute).  Overflowing assignments end with id -1 and
// gate 0, or with their rerouted expert and its probability.
hipError_t launch_capacity(int32_t* ids, float* gates, const int32_t* pos, const int32_t* offsets,
                           const int32_t* counts, const double* z_rows, const double* prob_rows, int64_t T, int E,
                           int k, int cap, int policy, hipStream_t stream);

// fraction[E] = mean_prob[E] = scalars[4] = 0 (empty batch)
hipError_t launch_zero_stats(int E, double* fraction, double* mean_prob, double* scalars, hipStream_t stream);

// --------------------------------------------------------------- permute
hipError_t launch_permute(const int32_t* ids, int64_t T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_token, int32_t* pos, hipStream_t stream);
// counts[0..E) = 0 (T == 0)
hipError_t launch_zero_counts(int32_t* counts, int E, int32_t* offsets, hipStream_t stream);

// ---------------------------------------------------------- grouped GEMM
struct GemmArgs {
    int which;              // 1: out = act(W1 . A[a_rows]) ; 2: out = W2 . A
    const void* A;          // activations: x [T][K] (which 1) or H [T*k][K] (which 2)
    const int32_t* a_rows;  // which 1: dispatch position -> token row of A
    const int32_t* offsets; // [E+1]
    const void* W;          // expert 0's [N][K] matrix
    const void* W_scales;   // INT4: bf16 [E][N][K/128]
    int64_t W_stride;       // bytes between experts
    void* out;              // [T*k][N] ([T*k][N/2] for SwiGLU)
    int64_t T, N, K;        // T: tokens (rows = T * k)
    int E, k, w_dtype, act_dtype;
    int path;               // 1 streaming, 2 tiled
    int rows_lo, rows_hi;   // only experts holding n rows, rows_lo < n <= rows_hi
    int stream_mt;          // streaming kernel: 16-row dispatch tiles per workgroup (1, 2 or 4)
    int act = 0;            // which 1: kActGelu, kActSilu or kActSwiglu (N = 2 d_ff weight rows)
    int ksplit = 1;         // K halves written to out and out + T*k*N as fp32 partials (which 2: tiled bf16 and
                            // streaming; which 1: streaming, no activation)
};
hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream);  // BF16 / INT4 weights
// H = bf16(act(P + P[stride])) for the two fp32 K-half partials of GEMM1 ([rows][N] each; N = dff, or 2 dff
// interleaved gate/up rows for SwiGLU); dff a multiple of 4
hipError_t launch_act_halves(const float* P, int64_t stride, void* H, int64_t rows, int N, int dff, int act,
                             hipStream_t stream);
hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream);   // BF16 weights
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t stream);     // F32 weights

// --------------------------------------------------------- router encoder
// offsets = {0, T} (one expert holding every row), by a kernel
hipError_t launch_encoder_offsets(int32_t* offsets, int64_t T, hipStream_t stream);
// h[T][d_r] (act dtype) = GeLU(pre + b_in), pre fp32 [T][d_r]; b_in may be null; d_r % 64 == 0
hipError_t launch_encoder_act(const float* pre, const float* b_in, void* h, int64_t T, int d_r, int act_dtype,
                              hipStream_t stream);

// --------------------------------------------------------------- combine
// Y2: null, or the second K half of Y (added to Y before the gate weighting)
hipError_t launch_combine(const float* Y, const int32_t* pos, const float* gates, void* y, int64_t T, int64_t d,
                          int k, int act_dtype, hipStream_t stream, const float* Y2 = nullptr);

}  // namespace moe
