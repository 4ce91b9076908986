// Capacity-limited dispatch of a top-k routing.
//
// Switch-style capacity (P5 §3.2: each expert takes at most
// cap = ceil(T k / E * capacity_factor) assignments; a full expert passes
// further tokens to their next-best expert) and the capacity-factor trade-off
// of P2 §3.2 (overflow is dropped, or retried at the next-best expert).  The
// assignments queue in row-major (token, slot) order:
//   pass 1: an assignment keeps its expert iff it is among the first cap
//           assignments of that expert's queue, i.e. iff its rank
//           pos - offsets[e] in the stable dispatch order is below cap;
//   pass 2: (reroute) the overflowing assignments, in the same order, each
//           move to the best-ranked expert (z order of the router) that the
//           token does not use at that moment and that still holds fewer
//           than cap assignments; with none, or under the drop policy, the
//           assignment is dropped (id -1, gate 0).  A rerouted assignment's
//           gate is p of its new expert (not renormalised).
//
// Pass 1 is parallel over the assignments.  Pass 2 is a sequential greedy
// fill (each choice depends on every earlier one through the expert counts),
// so it runs on one workgroup: the assignments stream through in chunks of
// whole tokens, the chunk's overflowing assignments are listed in order with
// a block scan, every wavefront stages their tokens' z rows in LDS, and one
// wavefront then walks the list, each step a 64-lane argmax over the experts
// with the per-expert counts and the chunk's current ids in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;  // assignments per chunk (rounded down to whole tokens)
constexpr int kMaxE = 256;
constexpr int kStageDoubles = 8192;            // 64 KB of staged z rows
constexpr int kMaxK = 8;

__global__ void __launch_bounds__(kThreads)
capacity_kernel(int32_t* __restrict__ ids, float* __restrict__ gates, const int32_t* __restrict__ pos,
                const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
                const double* __restrict__ z_rows, const double* __restrict__ prob_rows, int64_t Tk, int E, int k,
                int cap, int reroute) {
    __shared__ int cnt[kMaxE];        // assignments each expert holds
    __shared__ int offs[kMaxE];       // first dispatch position of each expert in the top-k routing
    __shared__ int cur[kChunk];       // the chunk's current expert per assignment (-1: none)
    __shared__ int list[kChunk];      // the chunk's overflowing assignments, row-major
    __shared__ int wsum[kWaves];
    __shared__ double zs[kStageDoubles];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    if (tid < E) {
        cnt[tid] = min(counts[tid], cap);  // what pass 1 keeps
        offs[tid] = offsets[tid];
    }
    __syncthreads();
    const int chunk = (kChunk / k) * k;
    const int rows = min(256, kStageDoubles / E);

    for (int64_t base = 0; base < Tk; base += chunk) {
        const int n_here = (int)min((int64_t)chunk, Tk - base);
        // pass 1 on assignments 4 tid .. 4 tid + 3 of the chunk
        int over = 0;  // bit r: assignment 4 tid + r overflows
#pragma unroll
        for (int r = 0; r < kPerThread; ++r) {
            const int i = kPerThread * tid + r;
            if (i < n_here) {
                const int64_t a = base + i;
                const int e = ids[a];
                const bool keep = (unsigned)e >= (unsigned)E || pos[a] - offs[e] < cap;
                cur[i] = keep ? e : -1;
                if (!keep) over |= 1 << r;
            }
        }
        // row-major list of the overflowing assignments (block exclusive scan of per-thread counts)
        const int c = __popc(over);
        int incl = c;
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const int s = wsum[v];
            if (v < w) before += s;
            total += s;
        }
        int at = before + incl - c;
#pragma unroll
        for (int r = 0; r < kPerThread; ++r)
            if ((over >> r) & 1) list[at++] = kPerThread * tid + r;
        __syncthreads();

        // pass 2 (reroute), in batches of staged z rows
        if (reroute) {
            for (int q0 = 0; q0 < total; q0 += rows) {
                const int nr = min(rows, total - q0);
                for (int idx = tid; idx < nr * E; idx += kThreads) {
                    const int r = idx / E;
                    const int e = idx - r * E;
                    const int64_t t = (base + list[q0 + r]) / k;
                    zs[idx] = z_rows[t * E + e];
                }
                __syncthreads();
                if (w == 0) {
                    for (int r = 0; r < nr; ++r) {
                        const int i = list[q0 + r];
                        const int first = i - i % k;  // the token's slot 0 (chunks hold whole tokens)
                        int tok[kMaxK];
#pragma unroll
                        for (int jj = 0; jj < kMaxK; ++jj) tok[jj] = jj < k ? cur[first + jj] : -1;
                        double bz = 0.0;
                        int be = kNoExpert;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int e = lane + 64 * j;
                            if (e < E && cnt[e] < cap) {
                                bool used = false;
#pragma unroll
                                for (int jj = 0; jj < kMaxK; ++jj) used |= tok[jj] == e;
                                const double z = zs[r * E + e];
                                if (!used && (be == kNoExpert || ranks_before(z, e, bz, be))) {
                                    bz = z;
                                    be = e;
                                }
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
                        // every lane holds the same be; LDS operations of one wavefront complete in order
                        if (be != kNoExpert && lane == 0) {
                            cur[i] = be;
                            cnt[be] += 1;
                        }
                    }
                }
                __syncthreads();
            }
        }

        // the overflowing assignments' final ids and gates
        for (int q = tid; q < total; q += kThreads) {
            const int i = list[q];
            const int64_t a = base + i;
            const int e = cur[i];
            ids[a] = e;
            gates[a] = e >= 0 ? (float)prob_rows[(a / k) * E + e] : 0.0f;
        }
        __syncthreads();  // cur, list and wsum are reused by the next chunk
    }
}

}  // namespace

hipError_t launch_capacity(int32_t* ids, float* gates, const int32_t* pos, const int32_t* offsets,
                           const int32_t* counts, const double* z_rows, const double* prob_rows, int64_t T, int E,
                           int k, int cap, int policy, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    if (E < 1 || E > kMaxE || k < 1 || k > kMaxK || cap < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(capacity_kernel, dim3(1), dim3(kThreads), 0, stream, ids, gates, pos, offsets, counts, z_rows,
                       prob_rows, T * k, E, k, cap, policy == 1 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace moe
