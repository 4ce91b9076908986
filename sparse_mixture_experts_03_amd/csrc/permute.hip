// Dispatch bookkeeping: per-expert counts, exclusive offsets, and the stable
// expert-major order of the T*k (token, slot) assignments.
//
// P3 §4.2 keeps a per-expert load vector and notes that tokens are really
// scattered to their experts (a grouped GEMM then runs per expert).  The order
// here is a stable counting sort, so it is unique and deterministic:
//   sorted_token[offsets[e] + r] = token of the r-th assignment to e in
//   row-major (token, slot) order;  pos[t*k + j] = position of (t, j).
//
// One 1024-thread workgroup: each of the 16 wavefronts owns a contiguous
// segment of the assignments, builds a per-wave histogram in LDS, the
// per-(wave, expert) bases come from one exclusive scan, and each wavefront
// then walks its segment 64 assignments at a time, ranking equal experts
// among its lanes with ballots (no float or order-dependent atomics).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = 256;

__global__ void __launch_bounds__(1024)
permute_kernel(const int32_t* __restrict__ ids, int Tk, int E, int k, int32_t* __restrict__ counts,
               int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token, int32_t* __restrict__ pos) {
    __shared__ int hist[kWaves][kMaxE];
    __shared__ int offs[kMaxE + 1];
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    for (int i = tid; i < kWaves * kMaxE; i += 1024) (&hist[0][0])[i] = 0;
    __syncthreads();

    const int seg = (Tk + kWaves - 1) / kWaves;
    const int a0 = min(Tk, w * seg);
    const int a1 = min(Tk, a0 + seg);
    for (int a = a0 + lane; a < a1; a += 64) {
        int e = ids[a];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[w][e], 1);
    }
    __syncthreads();

    // counts, then the exclusive scan of counts on wavefront 0 (4 experts per lane)
    if (w == 0) {
        int c[4], local = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = lane * 4 + j;
            int s = 0;
            if (e < E)
                for (int v = 0; v < kWaves; ++v) s += hist[v][e];
            c[j] = s;
            local += s;
        }
        int incl = local;
        for (int off = 1; off < 64; off <<= 1) {
            int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        int run = incl - local;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = lane * 4 + j;
            if (e < E) {
                counts[e] = c[j];
                offs[e] = run;
                offsets[e] = run;
            }
            run += c[j];
        }
        if (lane == 63) {
            offs[E] = incl;
            offsets[E] = incl;
        }
    }
    __syncthreads();
    // hist[v][e] becomes the first position wavefront v writes for expert e
    if (tid < E) {
        int run = offs[tid];
        for (int v = 0; v < kWaves; ++v) {
            int n = hist[v][tid];
            hist[v][tid] = run;
            run += n;
        }
    }
    __syncthreads();

    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = a0; base < a1; base += 64) {
        int a = base + lane;
        int e = (a < a1) ? ids[a] : -1;
        bool valid = (unsigned)e < (unsigned)E;
        unsigned long long same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            bool bit = valid && ((e >> b) & 1);
            unsigned long long bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        if (!valid) same = 0;
        int rank = __popcll(same & below);
        int leader = valid ? (__ffsll((long long)same) - 1) : lane;
        int first = 0;
        if (valid && lane == leader) first = atomicAdd(&hist[w][e], __popcll(same));
        first = __shfl(first, leader, 64);
        if (valid) {
            int slot = first + rank;
            sorted_token[slot] = a / k;
            pos[a] = slot;
        } else if (a < a1) {
            pos[a] = -1;
        }
    }
}

__global__ void zero_counts_kernel(int32_t* counts, int E, int32_t* offsets) {
    int i = threadIdx.x;
    if (i < E && counts) counts[i] = 0;
    if (i <= E && offsets) offsets[i] = 0;
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int64_t T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_token, int32_t* pos, hipStream_t stream) {
    if (T == 0) return launch_zero_counts(counts, E, offsets, stream);
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, stream, ids, (int)(T * k), E, k, counts, offsets,
                       sorted_token, pos);
    return hipGetLastError();
}

hipError_t launch_zero_counts(int32_t* counts, int E, int32_t* offsets, hipStream_t stream) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kMaxE + 64), 0, stream, counts, E, offsets);
    return hipGetLastError();
}

}  // namespace moe
