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
// whole tokens and the chunk's overflowing assignments are listed in order
// with a block scan.  Wavefront 0 then walks the list while the other
// fifteen stage, one batch ahead in a double-buffered LDS ring, each listed
// token's experts as 64-bit keys that order like z (the token's kept experts
// get the lowest key).  Wavefront 0 holds every expert's count in registers
// (lane l owns experts l, l + 64, ...), so one step is: mask full experts and
// those the token took earlier in the walk, take each lane's best key, one
// DPP max-reduction of the keys' high halves and a ballot of the lanes that
// hold it.  When exactly one lane does, its key is the unique maximum and the
// lane and its slot give the expert; otherwise (equal high halves, or only
// NaN or no candidates) the low halves are reduced among the tied lanes and
// then the expert index among the lanes holding the full maximum (ties go to
// the lower index).  The owning lane increments the expert's count.  The next
// step's keys and token are read from LDS under the current step's
// reductions.
#include "common.hpp"
#include "launch.hpp"

// Wavefront reductions of ROCm's device library (DPP based).
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;  // assignments per chunk (rounded down to whole tokens)
constexpr int kMaxE = 256;
constexpr int kRingKeys = 4096;                // keys per ring buffer (32 KB)
constexpr int kMaxK = 8;

// A 64-bit key that orders like the router's ranking: larger z larger key,
// any NaN below every number, and 0 reserved for "not a candidate".  -0 is
// folded into +0 (they compare equal, so the lower index must decide).
__device__ __forceinline__ uint64_t rank_key(double z) {
    if (isnan(z)) return 1;
    const uint64_t b = (uint64_t)__double_as_longlong(z + 0.0);
    return (b >> 63) ? ~b : (b | (1ull << 63));
}

// JN = ceil(E / 64): experts per lane of wavefront 0.
template <int JN>
__global__ void __launch_bounds__(kThreads)
capacity_kernel(int32_t* __restrict__ ids, float* __restrict__ gates, const int32_t* __restrict__ pos,
                const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
                const double* __restrict__ z_rows, const double* __restrict__ prob_rows, int64_t Tk, int E, int k,
                int cap, int reroute) {
    __shared__ int offs[kMaxE];       // first dispatch position of each expert in the top-k routing
    __shared__ int cur[kChunk];       // the chunk's expert per assignment after pass 1 (-1: overflow)
    __shared__ int list[kChunk];      // the chunk's overflowing assignments, row-major
    __shared__ int res[kChunk];       // their final experts (-1: dropped)
    __shared__ int ltok[kChunk];      // their tokens (chunk-local)
    __shared__ int wsum[kWaves];
    __shared__ uint64_t ring[2][kRingKeys];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    if (tid < E) offs[tid] = offsets[tid];
    // wavefront 0: the count of expert lane + 64 j after pass 1, then after each reroute
    int held[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
        const int e = lane + 64 * j;
        held[j] = (w == 0 && e < E) ? min(counts[e], cap) : cap;  // absent experts count as full
    }
    __syncthreads();
    const int chunk = (kChunk / k) * k;
    const int rows = min(256, kRingKeys / E);  // listed assignments per ring buffer

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
            if ((over >> r) & 1) {
                const int i = kPerThread * tid + r;
                res[at] = -1;
                ltok[at] = i / k;
                list[at++] = i;
            }
        __syncthreads();

        // pass 2 (reroute)
        if (reroute && total > 0) {
            const int nb = (total + rows - 1) / rows;
            // keys of listed assignments [q0, q0 + nr) into ring[buf], by threads t0, t0 + stride, ...
            auto stage = [&](int q0, int nr, uint64_t* buf, int t0, int stride) {
                for (int idx = t0; idx < nr * E; idx += stride) {
                    const int r = idx / E;
                    const int e = idx - r * E;
                    const int i = list[q0 + r];
                    const int first = i - i % k;  // the token's slot 0 (chunks hold whole tokens)
                    bool kept = false;
                    for (int jj = 0; jj < k; ++jj) kept |= cur[first + jj] == e;
                    buf[idx] = kept ? 0ull : rank_key(z_rows[((base + i) / k) * E + e]);
                }
            };
            stage(0, min(rows, total), ring[0], tid, kThreads);
            __syncthreads();
            int tok = -1;  // wavefront 0: the token being rerouted, and the experts it took so far
            int took = 0;
            for (int b = 0; b < nb; ++b) {
                const int q0 = b * rows;
                const int nr = min(rows, total - q0);
                if (w == 0) {
                    const uint64_t* buf = ring[b & 1];
                    uint64_t key[JN];
#pragma unroll
                    for (int j = 0; j < JN; ++j) key[j] = lane + 64 * j < E ? buf[lane + 64 * j] : 0ull;
                    int tnext = ltok[q0];
                    for (int r = 0; r < nr; ++r) {
                        const int t = tnext;
                        if (t != tok) {
                            tok = t;
                            took = 0;
                        }
                        uint64_t bk = 0;
                        int bj = 0;
#pragma unroll
                        for (int j = 0; j < JN; ++j) {
                            uint64_t kj = key[j];
                            if (held[j] >= cap || ((took >> j) & 1)) kj = 0;
                            if (kj > bk) {  // strict: the lower index keeps a tie
                                bk = kj;
                                bj = j;
                            }
                        }
                        const int rn = min(r + 1, nr - 1);
#pragma unroll
                        for (int j = 0; j < JN; ++j) key[j] = lane + 64 * j < E ? buf[rn * E + lane + 64 * j] : 0ull;
                        tnext = ltok[q0 + rn];
                        const uint32_t hi = (uint32_t)(bk >> 32);
                        const uint32_t mhi = __ockl_wfred_max_u32(hi);
                        const uint64_t at_max = __ballot(hi == mhi);
                        int be = -1;
                        if (mhi != 0 && __popcll(at_max) == 1) {
                            const int wl = __ffsll((unsigned long long)at_max) - 1;
                            be = wl + 64 * __builtin_amdgcn_readlane(bj, wl);
                        } else {
                            // low halves among the lanes at the maximum high half, then the lowest index
                            const uint32_t mlo = __ockl_wfred_max_u32(hi == mhi ? (uint32_t)bk : 0u);
                            if (mhi != 0 || mlo != 0) {
                                const bool top = hi == mhi && (uint32_t)bk == mlo;
                                be = (int)__ockl_wfred_min_u32(top ? (uint32_t)(lane + 64 * bj) : 0xffffffffu);
                            }
                        }
                        if (be >= 0) {
                            const bool own = lane == (be & 63);
#pragma unroll
                            for (int j = 0; j < JN; ++j)
                                if (j == (be >> 6)) {
                                    held[j] += own ? 1 : 0;
                                    took |= own ? 1 << j : 0;
                                }
                            if (lane == 0) res[q0 + r] = be;
                        }
                    }
                } else if (b + 1 < nb) {
                    stage(q0 + rows, min(rows, total - q0 - rows), ring[(b + 1) & 1], tid - 64, kThreads - 64);
                }
                __syncthreads();
            }
        }

        // the overflowing assignments' final ids and gates
        for (int q = tid; q < total; q += kThreads) {
            const int64_t a = base + list[q];
            const int e = res[q];
            ids[a] = e;
            gates[a] = e >= 0 ? (float)prob_rows[(a / k) * E + e] : 0.0f;
        }
        __syncthreads();  // cur, list, res and wsum are reused by the next chunk
    }
}

}  // namespace

hipError_t launch_capacity(int32_t* ids, float* gates, const int32_t* pos, const int32_t* offsets,
                           const int32_t* counts, const double* z_rows, const double* prob_rows, int64_t T, int E,
                           int k, int cap, int policy, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    if (E < 1 || E > kMaxE || k < 1 || k > kMaxK || cap < 1) return hipErrorInvalidValue;
#define MOE_CAPACITY_LAUNCH(JN_)                                                                               \
    hipLaunchKernelGGL((capacity_kernel<JN_>), dim3(1), dim3(kThreads), 0, stream, ids, gates, pos, offsets, counts, \
                       z_rows, prob_rows, T * k, E, k, cap, policy == 1 ? 1 : 0)
    const int jn = (E + 63) / 64;
    if (jn == 1) MOE_CAPACITY_LAUNCH(1);
    else if (jn == 2) MOE_CAPACITY_LAUNCH(2);
    else if (jn == 3) MOE_CAPACITY_LAUNCH(3);
    else MOE_CAPACITY_LAUNCH(4);
#undef MOE_CAPACITY_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
