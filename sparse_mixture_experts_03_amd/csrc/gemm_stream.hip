// Weight-streaming grouped expert GEMM for decode-sized token counts.
//
// P2 §2.3: at decode sizes the cost of an expert is moving its weights (the
// MoE layer there spends more time in weight traffic than in GEMM, and the
// weights never stay in cache).  This kernel therefore reads every weight of
// every active expert exactly once per 16*MT routed tokens (MT = 1, 2 or 4)
// and does the arithmetic on MFMA so that the matrix cores never limit the
// stream:
//   workgroup = 16*NB weight rows x one 16*MT-row tile of the dispatch order;
//   its four wavefronts split K; each streams its rows in stages of 256 or 512
//   bytes per row with fully coalesced non-temporal 16-byte loads (a wavefront
//   instruction reads whole 128-byte lines), parks the stage in a private
//   padded LDS buffer while the next stage is in flight, and reads it back in
//   MFMA operand layout (the MFMA row layout would otherwise split every line
//   over two instructions);
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

constexpr int kStreamBM = 16;  // dispatch rows per tile
// Tile shapes (measured per weight type and dispatch-tile height): 16-row weight tiles per workgroup and bytes
// of each weight row per pipeline stage.
constexpr int kNbBf16 = 1, kStageBf16 = 256;          // bf16 experts, 16-row dispatch tiles
constexpr int kNbInt4x16 = 4, kStageInt4x16 = 128;    // INT4 experts, 16-row dispatch tiles
constexpr int kNbInt4 = 4, kStageInt4 = 256;          // INT4 experts, 32- and 64-row dispatch tiles

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Weight loads: read once, never reused (non-temporal).
__device__ __forceinline__ uint4 ldw16(const void* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Eight signed INT4 codes (one 32-bit word, code i in bits 4i..4i+3) to eight
// bf16 values 136 + q_i, as one MFMA operand.  bf16(128 + c) = 0x4300 | c for
// c < 16, and c = q + 8 is the code with bit 3 flipped.  Output dword p holds
// codes 2p (low nibble of byte p of w) and 2p + 1 (low nibble of byte p of
// w >> 4): one byte permute places them in the two halves with zero bytes
// above them, and one three-input bit operation keeps bits 0-2, flips bit 3
// (a zero becomes one in the 0x43 byte as well) and clears the rest.
__device__ __forceinline__ uint32_t nibble_pair_to_bf16(uint32_t x) {
    return (x & 0x00070007u) | (~x & 0x43084308u);
}
__device__ __forceinline__ bf16x8 int4x8_to_bf16_offset136(uint32_t w) {
    const uint32_t w4 = w >> 4;
    uint4 r;
    r.x = nibble_pair_to_bf16(__builtin_amdgcn_perm(w4, w, 0x0c040c00u));
    r.y = nibble_pair_to_bf16(__builtin_amdgcn_perm(w4, w, 0x0c050c01u));
    r.z = nibble_pair_to_bf16(__builtin_amdgcn_perm(w4, w, 0x0c060c02u));
    r.w = nibble_pair_to_bf16(__builtin_amdgcn_perm(w4, w, 0x0c070c03u));
    return as_bf16x8(r);
}

// The same eight codes in a permuted K order that needs no byte permute:
// output dword j holds codes j (bits 4j..4j+3 of w, low half) and j + 4 (bits
// 16+4j.., high half), i.e. K slots (0,4,1,5,2,6,3,7); the activation operand
// is permuted to match (kperm_x).  One shift and one three-input bit operation
// ((w >> 4j) & 0x000f000f) ^ 0x43084308 per dword: the xor flips bit 3 of each
// code and sets the 0x43 exponent bytes.
__device__ __forceinline__ bf16x8 int4x8_to_bf16_offset136_kperm(uint32_t w) {
    constexpr uint32_t kNib = 0x000f000fu, kMagic = 0x43084308u;
    constexpr uint32_t kAndXor = (0xf0 & 0xcc) ^ 0xaa;  // truth table of (src0 & src1) ^ src2
    uint4 r;
    r.x = __builtin_amdgcn_bitop3_b32(w, kNib, kMagic, kAndXor);
    r.y = __builtin_amdgcn_bitop3_b32(w >> 4, kNib, kMagic, kAndXor);
    r.z = __builtin_amdgcn_bitop3_b32(w >> 8, kNib, kMagic, kAndXor);
    r.w = __builtin_amdgcn_bitop3_b32(w >> 12, kNib, kMagic, kAndXor);
    return as_bf16x8(r);
}
// Eight bf16 activations (x0..x7) reordered to the K slots above: (x0,x4),
// (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ uint4 kperm_x(uint4 v) {
    uint4 r;
    r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    return r;
}

template <int WHICH>
__device__ __forceinline__ void store_tile(void* out, int64_t N, int p0, int rows, int n0, f32x4 v, int lane,
                                           int act) {
    const int m = lane & 15;
    if (m >= rows) return;
    const int n = n0 + 4 * (lane >> 4);
    if constexpr (WHICH == 1) {
        uint2 packed;
        packed.x = pack_bf16x2(act_f(v[0], act), act_f(v[1], act));
        packed.y = pack_bf16x2(act_f(v[2], act), act_f(v[3], act));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)(p0 + m) * N + n) = packed;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + (int64_t)(p0 + m) * N + n) =
            make_float4(v[0], v[1], v[2], v[3]);
    }
}

// SwiGLU: a gate block g and its up block u (16 weight rows each) give 16
// hidden units starting at u0 of H (row stride Nh).
__device__ __forceinline__ void store_swiglu(void* out, int64_t Nh, int p0, int rows, int u0, f32x4 g, f32x4 u,
                                             int lane) {
    const int m = lane & 15;
    if (m >= rows) return;
    uint2 packed;
    packed.x = pack_bf16x2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
    packed.y = pack_bf16x2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)(p0 + m) * Nh + u0 + 4 * (lane >> 4)) = packed;
}

// Only experts holding n rows with rows_lo < n <= rows_hi are multiplied here.
template <int WQ, int WHICH, int NB, int MT, int kStageBytes, bool SCV = false>
__global__ void __launch_bounds__(256)
gemm_stream_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                   const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ W,
                   const uint16_t* __restrict__ Wsc, int64_t W_stride, void* __restrict__ out, int N, int K,
                   int ntiles_n, int rows_lo, int rows_hi, int act, int ksplit, int64_t split_stride) {
    constexpr int ROWS = 16 * NB;              // weight rows per workgroup
    constexpr int SEGS = kStageBytes / 16;     // 16-byte segments per row per stage
    constexpr int LROW = kStageBytes + 16;     // padded LDS row (conflict-free 16-row column reads)
    constexpr int LOADS = ROWS * SEGS / 64;    // 16-byte loads per lane per stage
    constexpr int GPS = kStageBytes / 64;      // INT4: 128-column scale groups per stage
    // per-wavefront stage buffers (INT4: followed by the stage's scales, ROWS x GPS bf16);
    // after the K loop the same LDS holds the partial tiles
    constexpr int kWaveLds = ROWS * LROW + (WQ == kINT4 ? ROWS * GPS * 2 : 0);
    constexpr int kStageLds = 4 * kWaveLds;
    constexpr int kRedBytes = 3 * NB * MT * 64 * 16;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStageLds > kRedBytes ? kStageLds : kRedBytes];
    uint8_t (*stage_lds)[kWaveLds] = reinterpret_cast<uint8_t (*)[kWaveLds]>(smem);
    f32x4 (*red)[NB * MT][64] = reinterpret_cast<f32x4 (*)[NB * MT][64]>(smem);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // ksplit = 2: workgroups 2 b and 2 b + 1 take the two halves of tile b's K stages and write them to out and
    // out + split_stride as fp32 partials without the activation (GEMM2: added in a fixed order by the combine;
    // GEMM1: by act_halves_kernel, which applies the activation)
    const int ks = blockIdx.x % ksplit;
    const int b_tile = blockIdx.x / ksplit;
    const int mt = b_tile / ntiles_n;
    const int nt = b_tile - mt * ntiles_n;
    if (WHICH == 2 || ksplit == 2) out = static_cast<float*>(out) + ks * split_stride;
    int e, p0, rows;
    if (!find_mtile(offsets, E, kStreamBM * MT, mt, &e, &p0, &rows, rows_lo, rows_hi)) return;

    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = nt * ROWS;
    // dispatch row 16 c + r of the tile feeds MFMA column tile c; lanes past
    // the tile's rows load nothing (at decode sizes most of them); with INT4
    // experts they read the tile's first row instead of branching around
    // their loads (rows >= 1 in every tile; those output columns are never stored)
    bool mvalid[MT];
    const uint16_t* xrow[MT];
#pragma unroll
    for (int c = 0; c < MT; ++c) {
        const int m = 16 * c + r;
        mvalid[c] = m < rows;
        int64_t arow = 0;
        if (mvalid[c]) arow = (WHICH == 1) ? (int64_t)a_rows[p0 + m] : (int64_t)(p0 + m);
        else if (WQ == kINT4) arow = (WHICH == 1) ? (int64_t)a_rows[p0] : (int64_t)p0;
        xrow[c] = A + arow * K;
    }
    const bool xall = WQ == kINT4;
    const int64_t row_bytes = (WQ == kBF16) ? (int64_t)K * 2 : (int64_t)K / 2;
    const uint8_t* Wblk = W + (int64_t)e * W_stride + (int64_t)n0 * row_bytes;
    uint8_t* lds = stage_lds[wave];
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    // This wavefront's stages (kStageBytes of every row each) of the workgroup's K range.
    const int nstages = (int)((row_bytes + kStageBytes - 1) / kStageBytes);
    const int lo = ks * nstages / ksplit, span = (ks + 1) * nstages / ksplit - lo;
    const int st0 = lo + wave * span / 4, st1 = lo + (wave + 1) * span / 4;

    // coalesced loads: instruction i, lane L -> row (64i + L) / SEGS, segment (64i + L) % SEGS
    auto gload = [&](int st, uint4 (&buf)[LOADS]) {
        const int64_t s0 = (int64_t)st * kStageBytes;
        const int64_t valid = min((int64_t)kStageBytes, row_bytes - s0);
        if constexpr (WQ == kINT4) {
            // no guards: segments past a K tail re-read the row's last 16 bytes
            // (never used), so every stage issues the same loads unconditionally
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int flat = 64 * i + lane;
                const int row = flat / SEGS, seg = flat % SEGS;
                buf[i] = ldw16(Wblk + (int64_t)row * row_bytes + min(s0 + seg * 16, row_bytes - 16));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int flat = 64 * i + lane;
            const int row = flat / SEGS, seg = flat % SEGS;
            buf[i] = (seg * 16 < valid) ? ldw16(Wblk + (int64_t)row * row_bytes + s0 + seg * 16) : zero4;
        }
    };
    auto lstore = [&](const uint4 (&buf)[LOADS]) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int flat = 64 * i + lane;
            const int row = flat / SEGS, seg = flat % SEGS;
            *reinterpret_cast<uint4*>(lds + row * LROW + seg * 16) = buf[i];
        }
    };

    f32x4 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < MT; ++c) acc[b][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // INT4 scales: each stage's GPS scales of row `srow` of the block are
    // loaded by lane srow (one vector load when aligned) with the stage's
    // codes, parked next to them in LDS, and read back per output row.
    const int groups = K / 128;
    const int srow = lane % ROWS;
    const uint16_t* sc_row = (WQ == kINT4) ? Wsc + (int64_t)e * N * groups + (int64_t)(n0 + srow) * groups : nullptr;
    uint16_t* sc_lds = reinterpret_cast<uint16_t*>(lds + ROWS * LROW);  // [ROWS][GPS]
    typedef uint16_t scales_t __attribute__((ext_vector_type(GPS)));
    auto sload = [&](int st, scales_t& v) {
        const int gb = st * GPS;
        if constexpr (SCV) {
            v = *reinterpret_cast<const scales_t*>(sc_row + gb);
        } else {
#pragma unroll
            for (int j = 0; j < GPS; ++j) {  // unconditional loads (clamped), then zero past the last group
                const uint16_t t = sc_row[min(gb + j, groups - 1)];
                v[j] = gb + j < groups ? t : (uint16_t)0;
            }
        }
    };
    const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);

    // Two register buffers: stage st + 1 is in flight while stage st is parked
    // in LDS and multiplied.
    constexpr bool XP = WQ == kINT4 && MT == 1;
    constexpr int XG = XP ? GPS : 1;
    uint4 xs[XG][MT][4];
    auto xload = [&](int st) {
        if constexpr (XP) {
            // groups past a K tail are never used: their loads repeat the last group
            const int gbase = st * GPS;
#pragma unroll
            for (int cc = 0; cc < GPS; ++cc) {
                const int grp = min(gbase + cc, groups - 1);
#pragma unroll
                for (int c = 0; c < MT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s) xs[cc][c][s] = ld16(xrow[c] + grp * 128 + 32 * g + 8 * s);
            }
        }
    };
    auto process = [&](int st, const uint4 (&buf)[LOADS], const scales_t& sbuf) {
        lstore(buf);
        if constexpr (WQ == kINT4) {
            if (lane < ROWS) *reinterpret_cast<scales_t*>(sc_lds + srow * GPS) = sbuf;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const int64_t s0 = (int64_t)st * kStageBytes;
        const int valid = (int)min((int64_t)kStageBytes, row_bytes - s0);
        if constexpr (WQ == kBF16) {
            // 64-column chunks (128 bytes per row); lane group g takes segments 2g, 2g+1
            const int kbase = (int)(s0 / 2);
            for (int cc = 0; cc < valid / 128; ++cc) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int koff = cc * 64 + (2 * g + s) * 8;
                    uint4 xa[MT];
#pragma unroll
                    for (int c = 0; c < MT; ++c) xa[c] = mvalid[c] ? ld16(xrow[c] + kbase + koff) : zero4;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const uint4 wa =
                            *reinterpret_cast<const uint4*>(lds + (16 * b + r) * LROW + cc * 128 + (2 * g + s) * 16);
#pragma unroll
                        for (int c = 0; c < MT; ++c) acc[b][c] = mfma16x16x32(as_bf16x8(wa), as_bf16x8(xa[c]), acc[b][c]);
                    }
                }
            }
        } else {
            // one 128-column scale group per 64 bytes of each row; lane group g takes columns [32g, 32g+32)
            const int gbase = (int)(s0 / 64);
            // the permuted-K dequantisation where registers allow it (16-row dispatch
            // tiles; with 32 or 64 rows its activation copies would spill)
            constexpr bool KPERM = MT == 1;
            scales_t sv[NB][4];  // this lane's output rows 16 b + 4 g + i
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[b][i] = *reinterpret_cast<const scales_t*>(sc_lds + (16 * b + 4 * g + i) * GPS);
            const int nch = SCV ? GPS : valid / 64;  // SCV: K is a multiple of the stage
#pragma unroll
            for (int cc = 0; cc < GPS; ++cc) {
                if (cc >= nch) break;
                const int grp = gbase + cc;
                uint4 xv[MT][4];
#pragma unroll
                for (int c = 0; c < MT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        xv[c][s] = XP ? xs[XP ? cc : 0][c][s]
                                 : (xall || mvalid[c]) ? ld16(xrow[c] + grp * 128 + 32 * g + 8 * s) : zero4;
                f32x4 t[NB][MT], sx[MT];
                uint4 q[NB];
#pragma unroll
                for (int c = 0; c < MT; ++c) sx[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < NB; ++b) {
#pragma unroll
                    for (int c = 0; c < MT; ++c) t[b][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
                    q[b] = *reinterpret_cast<const uint4*>(lds + (16 * b + r) * LROW + cc * 64 + 16 * g);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    uint4 xo[MT];
#pragma unroll
                    for (int c = 0; c < MT; ++c) xo[c] = KPERM ? kperm_x(xv[c][s]) : xv[c][s];
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const uint32_t word = s == 0 ? q[b].x : s == 1 ? q[b].y : s == 2 ? q[b].z : q[b].w;
                        const bf16x8 wq = KPERM ? int4x8_to_bf16_offset136_kperm(word) : int4x8_to_bf16_offset136(word);
#pragma unroll
                        for (int c = 0; c < MT; ++c) t[b][c] = mfma16x16x32(wq, as_bf16x8(xo[c]), t[b][c]);
                    }
#pragma unroll
                    for (int c = 0; c < MT; ++c) sx[c] = mfma16x16x32(as_bf16x8(ones), as_bf16x8(xo[c]), sx[c]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float scale = bf16_bits_to_float(sv[b][i][cc]);
#pragma unroll
                        for (int c = 0; c < MT; ++c)
                            acc[b][c][i] = fmaf(scale, fmaf(-136.0f, sx[c][i], t[b][c][i]), acc[b][c][i]);
                    }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    };
    uint4 bufa[LOADS], bufb[LOADS];
    scales_t sa = {}, sb = {};
    auto fetch = [&](int st, uint4 (&buf)[LOADS], scales_t& sbuf) {
        gload(st, buf);
        if constexpr (WQ == kINT4) sload(st, sbuf);
    };
    if (st0 < st1) fetch(st0, bufa, sa);
    // (using the two buffers in turn instead of copying needs two copies of the
    // stage code and more registers; measured slower at decode sizes)
    if constexpr (WQ == kINT4) {
        // the last stage is peeled so that the loop's loads are unconditional
        int st = st0;
        for (; st + 1 < st1; ++st) {
            if constexpr (XP) {
                xload(st);  // issued before the next stage's weights, so its waits never include them
                __builtin_amdgcn_sched_barrier(0);
            }
            fetch(st + 1, bufb, sb);
            process(st, bufa, sa);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) bufa[i] = bufb[i];
            sa = sb;
        }
        if (st < st1) {
            if constexpr (XP) xload(st);
            process(st, bufa, sa);
        }
    } else {
        for (int st = st0; st < st1; ++st) {
            if (st + 1 < st1) fetch(st + 1, bufb, sb);
            process(st, bufa, sa);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) bufa[i] = bufb[i];
            sa = sb;
        }
    }

    // fixed-order reduction of the four K-slices (in the stage buffers, once every wavefront is done with them)
    __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int c = 0; c < MT; ++c) red[wave - 1][b * MT + c][lane] = acc[b][c];
    }
    __syncthreads();
    if (wave == 0) {
        if (WHICH == 1 && ksplit == 2) {  // fp32 partial of every weight row, the activation comes later
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int c = 0; c < MT; ++c) {
                    f32x4 v = acc[b][c];
#pragma unroll
                    for (int w = 0; w < 3; ++w) v += red[w][b * MT + c][lane];
                    store_tile<2>(out, N, p0 + 16 * c, rows - 16 * c, n0 + 16 * b, v, lane, act);
                }
            return;
        }
        if constexpr (WHICH == 1 && NB % 2 == 0) {
            if (act == kActSwiglu) {  // blocks 2 b' (gate) and 2 b' + 1 (up) of 32 aligned rows
#pragma unroll
                for (int b = 0; b < NB; b += 2)
#pragma unroll
                    for (int c = 0; c < MT; ++c) {
                        f32x4 g = acc[b][c], u = acc[b + 1][c];
#pragma unroll
                        for (int w = 0; w < 3; ++w) {
                            g += red[w][b * MT + c][lane];
                            u += red[w][(b + 1) * MT + c][lane];
                        }
                        store_swiglu(out, N >> 1, p0 + 16 * c, rows - 16 * c, (n0 + 16 * b) >> 1, g, u, lane);
                    }
                return;
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int c = 0; c < MT; ++c) {
                f32x4 v = acc[b][c];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += red[w][b * MT + c][lane];
                store_tile<WHICH>(out, N, p0 + 16 * c, rows - 16 * c, n0 + 16 * b, v, lane, act);
            }
    }
}

template <int WQ, int NB, int MT, int SB>
hipError_t launch_stream_nb(const GemmArgs& a, hipStream_t stream) {
    const int64_t Tk = a.T * a.k;
    const int64_t max_mtiles = Tk / (kStreamBM * MT) + (Tk < a.E ? Tk : a.E);
    const int ntiles_n = (int)(a.N / (16 * NB));
    const int64_t blocks = max_mtiles * ntiles_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    const uint8_t* W = static_cast<const uint8_t*>(a.W);
    const uint16_t* S = static_cast<const uint16_t*>(a.W_scales);
    const int ksplit = a.ksplit == 2 ? 2 : 1;
    if (blocks * ksplit > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t split_stride = a.T * a.k * a.N;
    dim3 grid((unsigned)(blocks * ksplit)), block(256);
    // INT4: each stage's group scales are one vector load when every row's
    // scales start on a stage boundary of an aligned array
    const bool scv = WQ == kINT4 && (a.K / 128) % (SB / 64) == 0 && ((uintptr_t)S % 16) == 0;
#define MOE_STREAM_LAUNCH(WHICH_, SCV_)                                                                            \
    hipLaunchKernelGGL((gemm_stream_kernel<WQ, WHICH_, NB, MT, SB, SCV_>), grid, block, 0, stream, A, a.a_rows,     \
                       a.offsets, a.E, W, S, a.W_stride, a.out, (int)a.N, (int)a.K, ntiles_n, a.rows_lo, a.rows_hi, \
                       a.act, ksplit, split_stride)
    if constexpr (WQ == kINT4) {
        if (a.which == 1) {
            if (scv) MOE_STREAM_LAUNCH(1, true); else MOE_STREAM_LAUNCH(1, false);
        } else {
            if (scv) MOE_STREAM_LAUNCH(2, true); else MOE_STREAM_LAUNCH(2, false);
        }
    } else {
        if (a.which == 1) MOE_STREAM_LAUNCH(1, false); else MOE_STREAM_LAUNCH(2, false);
    }
#undef MOE_STREAM_LAUNCH
    return hipGetLastError();
}

// bf16 weights: 16 MT weight rows per workgroup for 16 MT dispatch rows, so
// the activation rows (re-read by every workgroup from L2) never outweigh the
// weights streamed from HBM; the wider tiles stage 128 bytes of each row (the
// register double buffer stays at 8 loads per lane).  INT4: 64 weight rows.
hipError_t launch_stream_bf16(const GemmArgs& a, hipStream_t stream) {
    // SwiGLU pairs a gate and an up block of 16 rows inside one workgroup: NB even
    if constexpr (kNbBf16 % 2 != 0) {
        if (a.stream_mt == 1 && a.which == 1 && a.act == kActSwiglu) return launch_stream_nb<kBF16, 2, 1, 128>(a, stream);
    }
    if (a.stream_mt == 1) return launch_stream_nb<kBF16, kNbBf16, 1, kStageBf16>(a, stream);
    if (a.stream_mt == 2) return launch_stream_nb<kBF16, 2, 2, 128>(a, stream);
    return launch_stream_nb<kBF16, 4, 4, 128>(a, stream);
}
hipError_t launch_stream_int4(const GemmArgs& a, hipStream_t stream) {
    if (a.stream_mt == 1) return launch_stream_nb<kINT4, kNbInt4x16, 1, kStageInt4x16>(a, stream);
    if (a.stream_mt == 2) return launch_stream_nb<kINT4, kNbInt4, 2, kStageInt4>(a, stream);
    return launch_stream_nb<kINT4, kNbInt4, 4, kStageInt4>(a, stream);
}

// GEMM1 in two K halves: H = bf16(act(P0 + P1)) from the fp32 partials P0 = P, P1 = P + stride ([rows][N]
// each, the halves added in that order).  SwiGLU: N = 2 dff weight rows, 32-row blocks of 16 gate rows then
// their 16 up rows; hidden unit 16 b + j is silu(gate row 32 b + j) * (up row 32 b + 16 + j).  Four units per
// thread.
__global__ void __launch_bounds__(256)
act_halves_kernel(const float* __restrict__ P, int64_t stride, uint16_t* __restrict__ H, int64_t rows, int N, int dff,
                  int act) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // first of this thread's four units
    if (i >= rows * dff) return;
    const int64_t r = i / dff;
    const int u = (int)(i - r * dff);
    const float* p0 = P + r * N;
    const float* p1 = p0 + stride;
    float h[4];
    if (act == kActSwiglu) {
        const int g = 32 * (u >> 4) + (u & 15);  // four units inside one block of 16 (dff is a multiple of 64)
        const float4 ga = *reinterpret_cast<const float4*>(p0 + g), gb = *reinterpret_cast<const float4*>(p1 + g);
        const float4 ua = *reinterpret_cast<const float4*>(p0 + g + 16);
        const float4 ub = *reinterpret_cast<const float4*>(p1 + g + 16);
        h[0] = silu_f(ga.x + gb.x) * (ua.x + ub.x);
        h[1] = silu_f(ga.y + gb.y) * (ua.y + ub.y);
        h[2] = silu_f(ga.z + gb.z) * (ua.z + ub.z);
        h[3] = silu_f(ga.w + gb.w) * (ua.w + ub.w);
    } else {
        const float4 a = *reinterpret_cast<const float4*>(p0 + u), b = *reinterpret_cast<const float4*>(p1 + u);
        h[0] = act_f(a.x + b.x, act);
        h[1] = act_f(a.y + b.y, act);
        h[2] = act_f(a.z + b.z, act);
        h[3] = act_f(a.w + b.w, act);
    }
    uint2 packed;
    packed.x = pack_bf16x2(h[0], h[1]);
    packed.y = pack_bf16x2(h[2], h[3]);
    *reinterpret_cast<uint2*>(H + i) = packed;
}

}  // namespace

hipError_t launch_act_halves(const float* P, int64_t stride, void* H, int64_t rows, int N, int dff, int act,
                             hipStream_t stream) {
    const int64_t quads = rows * dff / 4;
    if (quads == 0) return hipSuccess;
    hipLaunchKernelGGL(act_halves_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, P, stride,
                       static_cast<uint16_t*>(H), rows, N, dff, act);
    return hipGetLastError();
}

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
    // N is a multiple of 64, so any NB in {1, 2, 4} tiles it exactly.
    if (a.w_dtype == kBF16) return launch_stream_bf16(a, stream);
    return launch_stream_int4(a, stream);
}

}  // namespace moe
