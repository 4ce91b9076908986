// Router statistics over one batch: the monitoring and balance quantities
// the pages attach to the router.
//   P1 §3.2 router entropy: mean over tokens of -sum_e p ln p;
//   P3 §4.2 (the expert_load buffer): mean selection probability
//     P_e = sum_t p[t][e] / T over the full softmax rows;
//   P5 §3.2 balance loss: sum_e (f_e - 1/E)^2 with f_e the fraction of the
//     T k assignments routed to e; P3 §3.2 writes the same sum over P_e;
//   P5 §4 monitoring: the spread (standard deviation) of f_e across experts;
//   the product form E sum_e f_e P_e of the balance term (1 when uniform).
// The router's finalize step writes each token's softmax row and entropy;
// here one workgroup per expert sums its column (and counts its assignments)
// in a fixed order, and one workgroup forms the per-expert and scalar
// results, so the statistics are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

// Fixed-order block sum: thread i's value at slot i, then a halving tree.
__device__ __forceinline__ double block_sum(double v, double* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int w = kThreads / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// Block e < E: colsum[e] = sum_t prob_rows[t][e], count[e] = #{(t, j): ids = e}.
// Block E: colsum[E] = sum_t entropy_rows[t].  Each thread sums one contiguous
// range of tokens in ascending order.
__global__ void __launch_bounds__(kThreads)
stats_columns_kernel(const double* __restrict__ prob_rows, const double* __restrict__ entropy_rows,
                     const int32_t* __restrict__ ids, int64_t T, int E, int k, double* __restrict__ colsum,
                     int64_t* __restrict__ count) {
    __shared__ double red[kThreads];
    const int e = blockIdx.x;
    const int64_t per = (T + kThreads - 1) / kThreads;
    const int64_t t0 = (int64_t)threadIdx.x * per;
    const int64_t t1 = t0 + per < T ? t0 + per : T;
    double acc = 0.0;
    double n = 0.0;
    if (e < E) {
        for (int64_t t = t0; t < t1; ++t) {
            acc += prob_rows[t * E + e];
            for (int j = 0; j < k; ++j) n += ids[t * k + j] == e ? 1.0 : 0.0;
        }
    } else {
        for (int64_t t = t0; t < t1; ++t) acc += entropy_rows[t];
    }
    const double total = block_sum(acc, red);
    const double cnt = block_sum(n, red);  // exact: integers below 2^53
    if (threadIdx.x == 0) {
        colsum[e] = total;
        if (e < E) count[e] = (int64_t)cnt;
    }
}

__global__ void __launch_bounds__(kThreads)
stats_final_kernel(const double* __restrict__ colsum, const int64_t* __restrict__ count, int64_t T, int E, int k,
                   double* __restrict__ fraction, double* __restrict__ mean_prob, double* __restrict__ scalars) {
    __shared__ double red[kThreads];
    const int e = threadIdx.x;
    const double inv_e = 1.0 / (double)E;
    double df2 = 0.0, dp2 = 0.0, fp = 0.0;
    if (e < E) {
        const double f = (double)count[e] / ((double)T * (double)k);
        const double pm = colsum[e] / (double)T;
        fraction[e] = f;
        mean_prob[e] = pm;
        df2 = (f - inv_e) * (f - inv_e);
        dp2 = (pm - inv_e) * (pm - inv_e);
        fp = f * pm;
    }
    const double sf = block_sum(df2, red);
    const double sp = block_sum(dp2, red);
    const double sfp = block_sum(fp, red);
    if (e == 0) {
        scalars[0] = colsum[E] / (double)T;
        scalars[1] = sf;
        scalars[2] = sp;
        scalars[3] = sqrt(sf / (double)E);
        scalars[4] = (double)E * sfp;
    }
}

__global__ void zero_stats_kernel(int E, double* fraction, double* mean_prob, double* scalars) {
    const int i = threadIdx.x;
    if (i < E) {
        fraction[i] = 0.0;
        mean_prob[i] = 0.0;
    }
    if (i < 5) scalars[i] = 0.0;
}

}  // namespace

hipError_t launch_zero_stats(int E, double* fraction, double* mean_prob, double* scalars, hipStream_t stream) {
    hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(256), 0, stream, E, fraction, mean_prob, scalars);
    return hipGetLastError();
}

size_t stats_scratch_bytes(int E) { return (size_t)(E + 1) * sizeof(double) + (size_t)E * sizeof(int64_t); }

hipError_t launch_router_stats(const double* prob_rows, const double* entropy_rows, const int32_t* ids, int64_t T,
                               int E, int k, void* scratch, double* fraction, double* mean_prob, double* scalars,
                               hipStream_t stream) {
    double* colsum = static_cast<double*>(scratch);
    int64_t* count = reinterpret_cast<int64_t*>(colsum + E + 1);
    hipLaunchKernelGGL(stats_columns_kernel, dim3((unsigned)E + 1), dim3(kThreads), 0, stream, prob_rows,
                       entropy_rows, ids, T, E, k, colsum, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kThreads), 0, stream, colsum, count, T, E, k, fraction,
                       mean_prob, scalars);
    return hipGetLastError();
}

}  // namespace moe
