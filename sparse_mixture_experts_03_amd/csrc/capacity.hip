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
// with a block scan.  The list is cut into batches of at most 60 rows;
// wavefront 0 walks a batch while the other fifteen rank the next one into a
// double-buffered LDS array: a row's candidates are its kCand best experts in
// z order (the token's kept experts excluded) among those not at capacity in
// a snapshot wavefront 0 published two batches earlier (experts only fill up,
// so a stale snapshot merely leaves in experts that the walk then finds full).
// A token's rows in one batch share their candidates, so each token's run is
// ranked once.
//
// The walk takes up to 64 rows at a time, one per lane.  A lane proposes the
// first of its ranked candidates that is below capacity and not taken by its
// token, skipping as many further live candidates as its token has earlier
// rows in the group (those rows take them).  A bit-sliced ballot match counts
// the lower lanes proposing the same expert, and the rows before the first
// proposal that would push its expert past capacity are committed at once:
// each of them is exactly the sequential greedy choice at its row.  The walk
// resumes at the conflicting row, or, when a row has used up all kCand ranked
// candidates, takes that row alone with an exact wavefront reduction over its
// keys rebuilt from z (masked by the current counts and the token's picks;
// ties go to the lower expert index).  Expert counts live in LDS.
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
constexpr int kMaxK = 8;
constexpr int kCand = 4;                       // ranked candidates staged per listed assignment (16 bits each)
constexpr int kStagers = kWaves - 1;           // wavefronts that stage while wavefront 0 walks

// A 64-bit key that orders like the router's ranking: larger z larger key,
// any NaN below every number, and 0 reserved for "not a candidate".  -0 is
// folded into +0 (they compare equal, so the lower index must decide).
__device__ __forceinline__ uint64_t rank_key(double z) {
    const int64_t b = __double_as_longlong(z + 0.0);
    const uint64_t key = (uint64_t)b ^ ((uint64_t)(b >> 63) | (1ull << 63));  // negative: all bits flipped
    return isnan(z) ? 1ull : key;
}

// The maxima of a and of b (of a, b, c and d) over the wavefront, left in lane 63: a prefix max
// within each row of 16 lanes (row_shr 1, 2, 4, 8), then row 0's and row 2's
// maxima into rows 1 and 3 (row_bcast 15) and row 1's into rows 2 and 3
// (row_bcast 31).  The chains are interleaved so that each one's DPP
// operand waits are the others' issue slots.
__device__ __forceinline__ void wave_max_lane63_x2(uint32_t& a, uint32_t& b) {
#define MOE_DPP_MAX_STEP(CTRL, ROWS)                                                                    \
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, ROWS, 0xf, false));               \
    b = max(b, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROWS, 0xf, false));
    MOE_DPP_MAX_STEP(0x111, 0xf)
    MOE_DPP_MAX_STEP(0x112, 0xf)
    MOE_DPP_MAX_STEP(0x114, 0xf)
    MOE_DPP_MAX_STEP(0x118, 0xf)
    MOE_DPP_MAX_STEP(0x142, 0xa)
    MOE_DPP_MAX_STEP(0x143, 0xc)
#undef MOE_DPP_MAX_STEP
}
__device__ __forceinline__ void wave_max_lane63_x4(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& d) {
#define MOE_DPP_MAX_STEP(CTRL, ROWS)                                                                    \
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, ROWS, 0xf, false));               \
    b = max(b, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROWS, 0xf, false));               \
    c = max(c, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, CTRL, ROWS, 0xf, false));               \
    d = max(d, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d, CTRL, ROWS, 0xf, false));
    MOE_DPP_MAX_STEP(0x111, 0xf)
    MOE_DPP_MAX_STEP(0x112, 0xf)
    MOE_DPP_MAX_STEP(0x114, 0xf)
    MOE_DPP_MAX_STEP(0x118, 0xf)
    MOE_DPP_MAX_STEP(0x142, 0xa)
    MOE_DPP_MAX_STEP(0x143, 0xc)
#undef MOE_DPP_MAX_STEP
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
    __shared__ uint64_t cand[2][64];        // per listed assignment of a batch: its kCand best candidates, 0xffff past the last
    __shared__ uint64_t snap[2][4];         // experts at capacity (bit e % 64 of word e / 64), published per batch
    __shared__ int hcnt[kMaxE];             // each expert's count after pass 1, then after each reroute
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform, so wavefront 0's walk is scalar code
    if (tid < E) {
        offs[tid] = offsets[tid];
        hcnt[tid] = min(counts[tid], cap);
    }
    __syncthreads();
    const int chunk = (kChunk / k) * k;
    // listed assignments per batch: kG per staging wavefront, whose z is requested a batch ahead
    constexpr int kG = JN <= 2 ? 4 : 2;
    constexpr int rows = kStagers * kG;
    static_assert(rows <= 64, "a batch is walked by one wavefront");

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
            const int64_t tok0 = base / k;  // the chunk's first token (chunks hold whole tokens)
            // wavefront 0: the experts at capacity as bit words (bit l of word j is expert 64 j + l)
            auto publish = [&](int sn) {
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int e = lane + 64 * j;
                    const uint64_t f = __ballot(e >= E || hcnt[e] >= cap);
                    if (lane == 0) snap[sn][j] = f;
                }
            };
            // best key of a wavefront's JN keys per lane (expert lane + 64 j): one DPP max over the high halves and a
            // ballot; equal high halves (or only NaN keys) fall back to the low halves and then the lowest index.
            // -1 when every key is 0.  The result is wavefront-uniform.
            auto wave_argmax = [&](const uint64_t (&kv)[JN]) -> int {
                uint64_t bk = 0;
                int bj = 0;
#pragma unroll
                for (int j = 0; j < JN; ++j)
                    if (kv[j] > bk) {  // strict: the lower index keeps a tie
                        bk = kv[j];
                        bj = j;
                    }
                const uint32_t hi = (uint32_t)(bk >> 32);
                const uint32_t mhi = __ockl_wfred_max_u32(hi);
                const uint64_t at_max = __ballot(hi == mhi);
                if (mhi != 0 && __popcll(at_max) == 1) {
                    const int wl = __ffsll((unsigned long long)at_max) - 1;
                    return wl + 64 * __builtin_amdgcn_readlane(bj, wl);
                }
                const uint32_t mlo = __ockl_wfred_max_u32(hi == mhi ? (uint32_t)bk : 0u);
                if (mhi == 0 && mlo == 0) return -1;
                const bool top = hi == mhi && (uint32_t)bk == mlo;
                return __builtin_amdgcn_readfirstlane(
                    (int)__ockl_wfred_min_u32(top ? (uint32_t)(lane + 64 * bj) : 0xffffffffu));
            };
            // a listed row's keys: z order, 0 for the token's kept experts and where out[j] is set
            auto row_keys = [&](int q, const double (&zv)[JN], uint64_t (&kv)[JN], const bool (&out)[JN]) {
                const int first = ltok[q] * k;  // the token's slot 0
                bool kept[JN];
#pragma unroll
                for (int j = 0; j < JN; ++j) kept[j] = out[j];
                for (int jj = 0; jj < k; ++jj) {
                    const int ce = cur[first + jj];
#pragma unroll
                    for (int j = 0; j < JN; ++j) kept[j] |= ce == lane + 64 * j;
                }
#pragma unroll
                for (int j = 0; j < JN; ++j) kv[j] = kept[j] ? 0ull : rank_key(zv[j]);
            };
            auto zload = [&](int q, double (&dst)[JN]) {
                const double* zr = z_rows + (tok0 + ltok[min(q, total - 1)]) * E;
#pragma unroll
                for (int j = 0; j < JN; ++j) dst[j] = lane + 64 * j < E ? zr[lane + 64 * j] : 0.0;
            };

            // ---- staging (wavefronts 1 .. kStagers).  Rows of one token in a batch share their candidates (the same
            // kept experts and the same snapshot), so only the first row of each token's run in the batch is ranked
            // and its candidates are written for the whole run.  Those run starts are dealt out in order: the kG
            // starts sw, sw + kStagers, ... belong to staging wavefront sw.  A row's candidates are its kCand best
            // keys among the experts that are not at capacity in the snapshot published two batches earlier
            // (experts only fill up, so the snapshot leaves out only experts that are still full when the row is
            // walked).  A wavefront's rows are ranked side by side: each lane sorts its JN keys (stable odd-even
            // transposition, so equal keys keep the lower expert first), and every round reduces the lanes'
            // leading keys (one DPP max of the high halves and a ballot; the low halves and the expert index only on
            // a tie or NaN) and shifts the winning lane's list up by one.
            const int sw = w - 1;
            // this wavefront's rows of batch b (-1: none)
            auto assign = [&](int b, int (&rr)[kG]) {
                const int q0 = b * rows;
                const int nr = min(rows, total - q0);
                const bool start = lane < nr && (lane == 0 || ltok[q0 + lane] != ltok[q0 + lane - 1]);
                const int idx = __popcll(__ballot(start) & ((1ull << lane) - 1));
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    const uint64_t m = __ballot(start && idx == sw + kStagers * g);
                    rr[g] = m ? (int)__builtin_ctzll(m) : -1;
                }
            };
            auto prefetch = [&](int b, const int (&rr)[kG], double (&dst)[kG][JN]) {
#pragma unroll
                for (int g = 0; g < kG; ++g) zload(b * rows + max(rr[g], 0), dst[g]);
            };
            auto rank_rows = [&](int q0, int nr, int slot, const int (&rr)[kG], const double (&zc)[kG][JN],
                                 const bool (&fx)[JN]) {
                constexpr int P = kG;
                uint64_t kv[P][JN];
                int ix[P][JN];
                bool fin[P];
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    fin[p] = rr[p] < 0;
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        ix[p][j] = lane + 64 * j;
                        kv[p][j] = 0;
                    }
                    if (fin[p]) continue;
                    row_keys(q0 + rr[p], zc[p], kv[p], fx);
#pragma unroll
                    for (int pass = 0; pass < JN; ++pass)
#pragma unroll
                        for (int j = pass & 1; j + 1 < JN; j += 2)
                            if (kv[p][j + 1] > kv[p][j]) {
                                const uint64_t tk = kv[p][j];
                                kv[p][j] = kv[p][j + 1];
                                kv[p][j + 1] = tk;
                                const int ti = ix[p][j];
                                ix[p][j] = ix[p][j + 1];
                                ix[p][j + 1] = ti;
                            }
                }
                // starts are dealt in order (a third row only if there is a second), so with two rows or fewer only
                // the first two chains are reduced
                const bool two = P == 2 || fin[2 % P];
                uint64_t cw[P];
#pragma unroll
                for (int p = 0; p < P; ++p) cw[p] = ~0ull;
#pragma unroll
                for (int c = 0; c < kCand; ++c) {
                    uint32_t hi[P], mx[P];
#pragma unroll
                    for (int p = 0; p < P; ++p) mx[p] = hi[p] = (uint32_t)(kv[p][0] >> 32);
                    if (P == 4 && !two)
                        wave_max_lane63_x4(mx[0], mx[1], mx[2 % P], mx[3 % P]);
                    else
                        wave_max_lane63_x2(mx[0], mx[1 % P]);
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        if (fin[p]) continue;
                        const uint32_t mhi = __builtin_amdgcn_readlane(mx[p], 63);
                        const uint64_t am = __ballot(hi[p] == mhi);
                        int be;
                        if (mhi != 0 && __popcll(am) == 1) {
                            be = __builtin_amdgcn_readlane(ix[p][0], __builtin_ctzll(am));
                        } else {  // equal high halves, only NaN keys, or none left
                            const uint64_t hk = kv[p][0];
                            const uint32_t mlo = __ockl_wfred_max_u32(hi[p] == mhi ? (uint32_t)hk : 0u);
                            const bool top = hi[p] == mhi && (uint32_t)hk == mlo;
                            be = (mhi == 0 && mlo == 0)
                                     ? -1
                                     : __builtin_amdgcn_readfirstlane(
                                           (int)__ockl_wfred_min_u32(top ? (uint32_t)ix[p][0] : 0xffffffffu));
                        }
                        if (be < 0) {
                            fin[p] = true;
                            continue;
                        }
                        cw[p] ^= (uint64_t)(be ^ 0xffff) << (16 * c);
                        const bool win = ix[p][0] == be;
#pragma unroll
                        for (int j = 0; j + 1 < JN; ++j) {
                            kv[p][j] = win ? kv[p][j + 1] : kv[p][j];
                            ix[p][j] = win ? ix[p][j + 1] : ix[p][j];
                        }
                        kv[p][JN - 1] = win ? 0ull : kv[p][JN - 1];
                    }
                }
                if (lane == 0) {
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        if (rr[p] < 0) continue;
                        const int tk = ltok[q0 + rr[p]];
                        for (int r2 = rr[p]; r2 < nr && ltok[q0 + r2] == tk; ++r2) cand[slot][r2] = cw[p];
                    }
                }
            };
            // batch b's rows are ranked from z requested during the previous batch; batch b + 1's z is requested
            // afterwards (the compiler waits for every outstanding load before the first use of batch b's z, so
            // requests made before the ranking would be waited for there)
            auto stage = [&](int b, const int (&rc)[kG], const double (&zc)[kG][JN], int (&rn)[kG],
                             double (&zn)[kG][JN]) {
                const int q0 = b * rows;
                const int nr = min(rows, total - q0);
                const int slot = b & 1;
                bool fx[JN];  // expert lane + 64 j is past E or at capacity in the snapshot
#pragma unroll
                for (int j = 0; j < JN; ++j) fx[j] = lane + 64 * j >= E || ((snap[slot][j] >> lane) & 1);
                rank_rows(q0, nr, slot, rc, zc, fx);
                if (b + 1 < nb) {
                    assign(b + 1, rn);
                    prefetch(b + 1, rn, zn);
                }
            };

            // ---- walk (wavefront 0): a batch in one pass, lane l taking row g0 + l.  A lane proposes the m-th of
            // its ranked candidates that is below capacity now and not taken by its token before row g0, m being
            // the number of rows of its token among rows g0 .. g0 + l - 1 (those rows take the candidates ranked
            // before it).  A bit-sliced ballot match counts the lower lanes proposing the same expert; the rows
            // before the first proposal that would exceed capacity (or that needs the exact pick: all kCand
            // candidates gone) are committed, and the walk resumes at that row.  Experts only fill up, so each
            // committed proposal is the best expert left at its row in the sequential order.
            constexpr int kBits = JN == 1 ? 6 : JN == 2 ? 7 : 8;
            auto walk = [&](int b) {
                const int q0 = b * rows;
                const int nr = min(rows, total - q0);
                const int slot = b & 1;
                const uint64_t lt = (1ull << lane) - 1;
                int g0 = 0;
                for (int pass = 0; g0 < nr && pass < nr; ++pass) {  // every pass commits at least row g0
                    const int r = g0 + lane;
                    const bool in = r < nr;
                    const int qr = q0 + r;
                    // one round of LDS reads: the row's candidates and token, the token of the row before it, and
                    // (lane d - 1) the token and pick of row g0 - d for d < k
                    const uint64_t cw = in ? cand[slot][r] : ~0ull;
                    const int tk = in ? ltok[qr] : -1;
                    const int tpv = in && qr >= 1 ? ltok[qr - 1] : -2;
                    const int qd = q0 + g0 - 1 - lane;
                    const bool dl = lane < k - 1 && qd >= 0;
                    const int td = dl ? ltok[qd] : -3;
                    const int pd = dl ? res[qd] : -1;
                    // the experts row g0's token took before row g0
                    const int t0 = __builtin_amdgcn_readfirstlane(tk);
                    uint64_t pm[JN];
#pragma unroll
                    for (int j = 0; j < JN; ++j) pm[j] = 0;
                    for (uint64_t mb = __ballot(dl && td == t0 && pd >= 0); mb; mb &= mb - 1) {
                        const int pe = __builtin_amdgcn_readlane(pd, __builtin_ctzll(mb));
#pragma unroll
                        for (int j = 0; j < JN; ++j)
                            if ((pe >> 6) == j) pm[j] |= 1ull << (pe & 63);
                    }
                    // rank among the pass's rows of the same token; lanes of the first run continue row g0 - 1's token
                    const uint64_t starts = __ballot(tk != tpv);
                    const uint64_t le = starts & (lt | (1ull << lane));
                    const int run0 = le ? 63 - __clzll((long long)le) : 0;
                    const bool cont = (starts & 1) == 0 && le == 0;
                    const int m = lane - run0;
                    // the proposal: m-th live candidate; -1 drop (the ranking ran out), -3 exact pick needed
                    int hc[kCand];
#pragma unroll
                    for (int c = 0; c < kCand; ++c) hc[c] = hcnt[min((int)((cw >> (16 * c)) & 0xffff), E - 1)];
                    int pe = -3, ph = 0, v = 0;
                    bool done = !in;
#pragma unroll
                    for (int c = 0; c < kCand; ++c) {
                        const int ce = (int)((cw >> (16 * c)) & 0xffff);
                        if (!done && ce == 0xffff) {
                            pe = -1;
                            done = true;
                        }
                        if (!done) {
                            uint64_t pw = pm[0];
#pragma unroll
                            for (int j = 1; j < JN; ++j)
                                if ((ce >> 6) == j) pw = pm[j];
                            const bool live = hc[c] < cap && !(cont && ((pw >> (ce & 63)) & 1));
                            if (live && v == m) {
                                pe = ce;
                                ph = hc[c];
                                done = true;
                            }
                            v += live ? 1 : 0;
                        }
                    }
                    // lower lanes proposing the same expert
                    const bool has = in && pe >= 0;
                    uint64_t eq = __ballot(has);
#pragma unroll
                    for (int bit = 0; bit < kBits; ++bit) {
                        const bool set = (pe >> bit) & 1;
                        const uint64_t bm = __ballot(has && set);
                        eq &= set ? bm : ~bm;
                    }
                    const bool ok = !in || pe == -1 || (pe >= 0 && ph + __popcll(eq & lt) < cap);
                    const uint64_t bad = __ballot(!ok);
                    const int n_in = nr - g0;
                    const int f = bad ? (int)__builtin_ctzll(bad) : n_in;
                    const uint64_t cm = f >= 64 ? ~0ull : (1ull << f) - 1;
                    if (lane < f) res[qr] = pe;
                    if (has && lane < f && (eq & cm & ~(lt | (1ull << lane))) == 0) hcnt[pe] = ph + __popcll(eq & cm);
                    if (f == n_in) break;
                    if (__builtin_amdgcn_readlane(pe, f) != -3) {  // over capacity: propose again from row g0 + f
                        g0 += f;
                        continue;
                    }
                    // the exact pick for row g0 + f: its keys from z, without the experts at capacity and those its
                    // token took at earlier rows
                    const int q = q0 + g0 + f;
                    const int tq = __builtin_amdgcn_readfirstlane(ltok[q]);
                    uint64_t tm[JN];
#pragma unroll
                    for (int j = 0; j < JN; ++j) tm[j] = 0;
                    for (int d = 1; d < k && q - d >= 0; ++d) {
                        if (__builtin_amdgcn_readfirstlane(ltok[q - d]) != tq) break;
                        const int te = __builtin_amdgcn_readfirstlane(res[q - d]);
                        if (te >= 0) {
#pragma unroll
                            for (int j = 0; j < JN; ++j)
                                if ((te >> 6) == j) tm[j] |= 1ull << (te & 63);
                        }
                    }
                    double zv[JN];
                    zload(q, zv);
                    bool out[JN];
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        const int e = lane + 64 * j;
                        out[j] = e >= E || hcnt[min(e, E - 1)] >= cap || ((tm[j] >> lane) & 1);
                    }
                    uint64_t kv[JN];
                    row_keys(q, zv, kv, out);
                    const int be = wave_argmax(kv);
                    if (lane == 0) {
                        res[q] = be;
                        if (be >= 0) hcnt[be] += 1;
                    }
                    g0 += f + 1;
                }
            };

            double za[kG][JN], zb[kG][JN];
            int ra[kG], rb[kG];
            if (w == 0) {
                publish(0);
                publish(1);
            } else {
                assign(0, ra);
                prefetch(0, ra, za);
            }
            __syncthreads();
            if (w != 0) stage(0, ra, za, rb, zb);
            __syncthreads();
            for (int b = 0; b < nb; ++b) {
                if (w == 0) {
                    walk(b);
                    publish(b & 1);  // read when batch b + 2 is staged
                } else if (b + 1 < nb) {
                    if ((b + 1) & 1)
                        stage(b + 1, rb, zb, ra, za);
                    else
                        stage(b + 1, ra, za, rb, zb);
                }
                __syncthreads();
            }
        }

        // the overflowing assignments' final ids and gates
        for (int q = tid; q < total; q += kThreads) {
            const int64_t a = base + list[q];
            const int e = res[q];
            ids[a] = e;
            gates[a] = e >= 0 ? (float)prob_rows[(base / k + ltok[q]) * E + e] : 0.0f;
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
