// LDS-tiled MFMA grouped expert GEMM for prefill-sized token counts.
//
// P3 §3.2: every expert is the same d -> 4d -> d GELU MLP with its own W1 and
// W2, so one kernel serves all experts; P3 §4.2 notes the per-expert work is
// really a grouped GEMM over the tokens scattered to each expert, and P2 §3.3
// credits fusing the activation into the expert GEMM.  Here:
//   workgroup tile = 256 weight rows x 256 dispatch rows (one expert), one
//   workgroup per CU; an expert's last, partial tile uses a 128- or 64-row
//   variant so padding stays small.  Tiles go straight from HBM/L2 into LDS
//   with gfx950's global_load_lds (16 bytes per lane, no register staging),
//   and tile rows keep their 16-byte segments in XOR-permuted slots, so the
//   copies, the dequantised stores and the 32-row MFMA fragment reads are
//   free of LDS bank conflicts.  MFMA 32x32x16 bf16 with fp32 accumulators in
//   AGPRs throughout.
//   bf16 weights: K-stages of 64 (every tile row of a stage is one whole
//   128-byte line), two weight and three dispatch-row slots of 32 KB (all
//   160 KB of LDS), eight wavefronts (two per SIMD) of 128 x 64 outputs.
//   GEMM1 runs them in lockstep, one barrier per stage; GEMM2's 256-row
//   tiles run two groups of four in ping-pong (one multiplies while the other
//   reads fragments and copies).
//   INT4 weights (P1 §5.4, P2 §2.3): K-stages of 32 in a ring of four, the
//   dispatch rows three stages ahead and the codes four; the workgroup turns
//   each stage's codes into bf16(q * s) in LDS, in the layout the bf16 tiles
//   use, so the MFMA step is the same; four wavefronts of 128 x 128 outputs
//   (256 accumulators each), one barrier per stage.
//   GEMM1's epilogue applies the activation and stores bf16 H, GEMM2's
//   stores fp32 Y; both are staged through LDS so every store writes whole
//   lines (SwiGLU, which pairs gate and up rows, stores from registers).
// The m-tiles of all experts are numbered expert-major and located from the
// offsets on the device, so skewed loads (0 .. thousands of rows per expert)
// need no host round trip; tiles past the last real one exit at once.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"


namespace moe {

namespace {

constexpr int kTBN = 256;   // weight rows per tile
constexpr int kTBM = 256;   // dispatch rows per tile
constexpr int kTBK = 32;    // K per stage (64 bytes of every tile row)
constexpr int kStages = 4;  // LDS ring: stage k+3 streams in while stage k is multiplied
constexpr int kTileBytes = 256 * kTBK * 2;  // 16 KB per operand per stage
// INT4 kernel: 4 + 4 stages of 16 KB, the code ring (4 x 4 KB) and the scale ring (2 x 4 KB).  Both
// kernels stage their epilogues through the same LDS, over the rings: safe only once the last stage has
// waited for every copy (vmcnt 0), which both do before their epilogues.
constexpr int kInt4LdsBytes = 2 * kStages * kTileBytes + kStages * 4096 + 2 * 4096;
// bf16 kernel: 2 weight + 3 dispatch-row stages of 32 KB, all of a CU's LDS.
constexpr int kBf16LdsBytes = 5 * 32768;
// INT4: VALU operations of the next stage's code expansion placed after each MFMA of this stage
// (other group sizes spill).
constexpr int kInt4MixValu = 6;

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// One wavefront copies 16 tile rows x 64 bytes (1 KB) of one stage into LDS:
// lane L fetches logical segment (L & 3) ^ ((L >> 4) & 3) of row L >> 2, which
// lands at LDS byte 16 * L of the 1 KB block, i.e. physical slot L & 3 of that
// row.  `base` is wave-uniform and `off` a 32-bit byte offset (one expert's
// weights and every activation array stay below 4 GiB), so the load takes the
// scalar-base + vector-offset form.
__device__ __forceinline__ void copy_rows_to_lds(const char* base, uint32_t off, uint8_t* lds_block) {
    __builtin_amdgcn_global_load_lds((gvoid*)(base + off), (lvoid*)lds_block, 16, 0, 0);
}
// The same with the non-temporal hint (data read once).
__device__ __forceinline__ void copy_rows_to_lds_nt(const char* base, uint32_t off, uint8_t* lds_block) {
    __builtin_amdgcn_global_load_lds((gvoid*)(base + off), (lvoid*)lds_block, 16, 0, 2);
}

// LDS byte offset of logical segment `seg` (0..3) of tile row `row`.
// Physical slot = seg ^ ((row >> 2) & 3): any 8 consecutive rows read at one
// logical segment touch 8 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t frag_offset(int row, int seg) {
    return (uint32_t)(row * 64 + 16 * (seg ^ ((row >> 2) & 3)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lvoid*)p;
}

// The fragment reads are issued as inline asm: the compiler cannot tell LDS
// reads of one ring slot from the direct-to-LDS loads still filling the
// others and would otherwise wait for every load in flight before each read.
// Their completion is awaited explicitly (lgkmcnt) before the MFMAs use them.
__device__ __forceinline__ bf16x8 ds_read16(uint32_t addr) {
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the compiler's release/acquire fence (which would
// also wait for the direct-to-LDS loads of the stages still in flight); the
// explicit vmcnt waits before it publish exactly the stage that is due.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---- INT4 weight rows -------------------------------------------------
// Four code words (8 INT4 codes each) of this thread, one from each of four
// code rows (word addresses c0 + 256 j), read from LDS where the wavefront's
// own direct-to-LDS loads put them.  The outputs are early-clobber: a load's
// result may land before the next load of the group has read the address.
__device__ __forceinline__ void ds_read_codes(uint32_t c0, uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t& w3) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:256\n\t"
        "ds_read_b32 %2, %4 offset:512\n\tds_read_b32 %3, %4 offset:768\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
        : "v"(c0));
}
// The matching four bf16 group scales (256 bytes apart in the scale ring),
// zero-extended.
__device__ __forceinline__ void ds_read_scales(uint32_t s0, uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& d) {
    asm volatile(
        "ds_read_u16 %0, %4\n\tds_read_u16 %1, %4 offset:256\n\t"
        "ds_read_u16 %2, %4 offset:512\n\tds_read_u16 %3, %4 offset:768\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
        : "v"(s0));
}

__device__ __forceinline__ void ds_write16(uint32_t addr, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// One code word (8 INT4 codes: byte j holds k = 2j in its low nibble and
// k = 2j + 1 in its high nibble) with its group's bf16 scale -> one 16-byte
// tile segment of 8 bf16 values bf16(q * s), written to LDS at `addr`.
// q * s is formed exactly as fma(q + 8, s, -8 s) ((q + 8) * s has at most 12
// significant bits) and rounded once, to nearest even.
__device__ __forceinline__ uint4 dequant_word(uint32_t word, uint32_t sbits) {
    const float s = bf16_bits_to_float(sbits);
    const float m8s = -8.0f * s;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t lo = (word & 0x0f0f0f0fu) ^ 0x08080808u;
    const uint32_t hi = ((word >> 4) & 0x0f0f0f0fu) ^ 0x08080808u;
    uint32_t packed[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a = __builtin_fmaf((float)((lo >> (8 * j)) & 0xffu), s, m8s);
        const float b = __builtin_fmaf((float)((hi >> (8 * j)) & 0xffu), s, m8s);
        const bf16x2_t v = {(__bf16)a, (__bf16)b};
        packed[j] = __builtin_bit_cast(uint32_t, v);
    }
    return make_uint4(packed[0], packed[1], packed[2], packed[3]);
}
__device__ __forceinline__ void dequant_word_to_lds(uint32_t word, uint32_t sbits, uint32_t addr) {
    const float s = bf16_bits_to_float(sbits);
    const float m8s = -8.0f * s;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t lo = (word & 0x0f0f0f0fu) ^ 0x08080808u;         // q + 8 of even k
    const uint32_t hi = ((word >> 4) & 0x0f0f0f0fu) ^ 0x08080808u;  // q + 8 of odd k
    uint32_t packed[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a = __builtin_fmaf((float)((lo >> (8 * j)) & 0xffu), s, m8s);
        const float b = __builtin_fmaf((float)((hi >> (8 * j)) & 0xffu), s, m8s);
        const bf16x2_t v = {(__bf16)a, (__bf16)b};
        packed[j] = __builtin_bit_cast(uint32_t, v);
    }
    ds_write16(addr, packed[0], packed[1], packed[2], packed[3]);
}

// Epilogue: element v of acc[i][j] is D[n = wn + 32i + 8(v/4) + 4h + (v%4)][m = wm + 32j + r];
// GEMM1 stores bf16 GeLU(D), GEMM2 stores fp32 D, for rows below `rows` and n below N.
// GEMM1 epilogue of both tiled kernels, staged through LDS (free once the K
// loop is done): each wavefront writes its activated bf16 tile into a private
// padded region laid out [dispatch row][weight row], then reads it back in
// 16-byte chunks, so every store instruction writes whole 128-byte lines of H
// instead of 16-byte pieces of 32 rows.  Not for SwiGLU (two rows per unit).
template <int TI, int TJ, int ACT, int NWAVE, int LDS_BYTES>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[TI][TJ], uint8_t* lds, void* __restrict__ out,
                                               int N, int n0, int p0, int rows, int wn, int wm, int r, int h,
                                               bool math) {
    constexpr int NW = 32 * TI, MW = 32 * TJ;  // this wavefront's weight rows x dispatch rows
    constexpr int STRIDE = NW * 2 + 16;        // padded LDS row in bytes (16-byte aligned)
    static_assert(NWAVE * MW * STRIDE <= LDS_BYTES, "epilogue staging exceeds the kernel's LDS");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint8_t* wl = lds + wave * (MW * STRIDE);
    barrier();  // every wavefront has finished reading the last stage
    if (!math) return;
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            // one 32 x 32 block at a time: the empty statement pins the block to the accumulator registers
            // until here, so the compiler does not copy every block out of them at once (more registers
            // than are left beside the accumulators)
            f32x16 blk = acc[i][j];
            asm volatile("" : "+a"(blk));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint2 packed;
                packed.x = pack_bf16x2(act_f(blk[4 * q], ACT), act_f(blk[4 * q + 1], ACT));
                packed.y = pack_bf16x2(act_f(blk[4 * q + 2], ACT), act_f(blk[4 * q + 3], ACT));
                *reinterpret_cast<uint2*>(wl + (32 * j + r) * STRIDE + (32 * i + 8 * q + 4 * h) * 2) = packed;
            }
        }
    constexpr int CH = NW * 2 / 16, RPI = 64 / CH;  // chunks per row, rows per instruction
    const int cr = lane / CH, cc = lane % CH;
    const int n = n0 + wn + cc * 8;  // N is a multiple of 8
#pragma unroll
    for (int k = 0; k < MW / RPI; ++k) {
        const int ml = k * RPI + cr;
        const uint4 v = *reinterpret_cast<const uint4*>(wl + ml * STRIDE + cc * 16);
        if (wm + ml < rows && n < N)
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (int64_t)(p0 + wm + ml) * N + n) = v;
    }
}

// GEMM2 epilogue of both tiled kernels (fp32 Y), staged through LDS like GEMM1's
// in passes of 32 dispatch rows (a wavefront's whole fp32 tile would not fit):
// every store instruction writes whole rows of Y.  Each wavefront reuses only
// its own region and its LDS operations execute in order, so one barrier (the
// last stage is no longer read) is enough.
template <int TI, int TJ, int NWAVE, int LDS_BYTES>
__device__ __forceinline__ void store_tile_lds_f32(const f32x16 (&acc)[TI][TJ], uint8_t* lds, float* __restrict__ out,
                                                   int N, int n0, int p0, int rows, int wn, int wm, int r, int h,
                                                   bool math) {
    constexpr int NW = 32 * TI;         // this wavefront's weight rows (columns of Y)
    constexpr int STRIDE = NW * 4 + 16;  // padded LDS row in bytes
    static_assert(NWAVE * 32 * STRIDE <= LDS_BYTES, "epilogue staging exceeds the kernel's LDS");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint8_t* wl = lds + wave * (32 * STRIDE);
    constexpr int CH = NW * 4 / 16, RPI = 64 / CH;  // 16-byte chunks per row, rows per instruction
    const int cr = lane / CH, cc = lane % CH;
    const int n = n0 + wn + cc * 4;  // N is a multiple of 4
    barrier();
    if (!math) return;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(wl + r * STRIDE + (32 * i + 8 * q + 4 * h) * 4) =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int ml = k * RPI + cr;
            const float4 v = *reinterpret_cast<const float4*>(wl + ml * STRIDE + cc * 16);
            const int m = wm + 32 * j + ml;
            if (m < rows && n < N) *reinterpret_cast<float4*>(out + (int64_t)(p0 + m) * N + n) = v;
        }
    }
}

template <int WHICH, int TI, int TJ, int ACT>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TI][TJ], void* __restrict__ out, int N, int n0, int p0,
                                           int rows, int wn, int wm, int r, int h) {
    if constexpr (WHICH == 1 && ACT == kActSwiglu) {
        // accumulators 0..7 of a 32-row block hold gate rows 8 q + 4 h + c (q < 2), 8..15 the up rows 16 below
        const int Nh = N >> 1;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int m = wm + 32 * j + r;
            if (m >= rows) continue;
            const int64_t orow = (int64_t)(p0 + m) * Nh;
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int nb = n0 + wn + 32 * i;
                if (nb >= N) continue;
                f32x16 blk = acc[i][j];
                asm volatile("" : "+a"(blk));  // one block out of the accumulator registers at a time
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float hv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) hv[c] = silu_f(blk[4 * q + c]) * blk[4 * q + 8 + c];
                    uint2 packed;
                    packed.x = pack_bf16x2(hv[0], hv[1]);
                    packed.y = pack_bf16x2(hv[2], hv[3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + (nb >> 1) + 8 * q + 4 * h) =
                        packed;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int m = wm + 32 * j + r;
        if (m >= rows) continue;
        const int64_t orow = (int64_t)(p0 + m) * N;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn + 32 * i + 8 * q + 4 * h;
                if (n >= N) continue;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if constexpr (WHICH == 1) {
                    uint2 packed;
                    packed.x = pack_bf16x2(act_f(v0, ACT), act_f(v1, ACT));
                    packed.y = pack_bf16x2(act_f(v2, ACT), act_f(v3, ACT));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + n) = packed;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + n) = make_float4(v0, v1, v2, v3);
                }
            }
        }
    }
}

// One workgroup tile: 256 weight rows x XROWS dispatch rows, wavefront w
// owning TI 32-row weight tiles x TJ 32-row dispatch tiles.  XROWS = 256: 2 x 2
// wavefronts of 128 x 128; XROWS = 128: 4 x 1 of 64 x 128; XROWS = 64: 4 x 1
// of 64 x 64.  The smaller shapes serve the last, partial tile of an expert
// so that a remainder of 40 rows costs a quarter tile, not a full one.
// Wexp is the expert's packed INT4 codes [N][K/2], Wsc its bf16 scales
// [N][K/128] (bf16 experts use tile_gemm_bf16 and tile_gemm2_bf16_pp).
template <int WQ, int WHICH, int TI, int TJ, int XROWS, int ACT>
__device__ __forceinline__ void tile_gemm(uint8_t (*Wt)[kTileBytes], uint8_t (*Xt)[kTileBytes], uint8_t (*Ct)[4096],
                                          uint8_t (*St)[4096],
                                          const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                                          const void* Wexp, const void* Wsc, void* __restrict__ out, int N, int K,
                                          int n0, int p0, int rows) {
    constexpr int WN_WAVES = 256 / (32 * TI);  // wavefronts along the weight rows
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar

    const int lseg = (lane & 3) ^ ((lane >> 4) & 3);  // logical segment this lane copies
    const char* xbase = reinterpret_cast<const char*>(A);
    const uint32_t xrowbytes = (uint32_t)K * 2;

    const int wn = (wave % WN_WAVES) * (32 * TI);  // this wave's weight rows within the tile
    const int wm = (wave / WN_WAVES) * (32 * TJ);  // this wave's dispatch rows within the tile
    const int r = lane & 31;
    const int h = lane >> 5;
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // two k-substeps of 16: lane half h reads logical segment 2 * ks + h.
    // Substep 1's fragments are read while substep 0's MFMAs run.
    uint32_t wrow_off[TI], xrow_off[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) wrow_off[i] = frag_offset(wn + 32 * i + r, 0);  // XOR 16*seg selects segment seg
#pragma unroll
    for (int j = 0; j < TJ; ++j) xrow_off[j] = frag_offset(wm + 32 * j + r, 0);
    auto compute = [&](int buf, auto mid) {
        const uint32_t wb = lds_addr(Wt[buf]), xb = lds_addr(Xt[buf]);
        bf16x8 wf[2][TI], xf[2][TJ];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i) wf[ks][i] = ds_read16(wb + (wrow_off[i] ^ (16 * (2 * ks + h))));
#pragma unroll
            for (int j = 0; j < TJ; ++j) xf[ks][j] = ds_read16(xb + (xrow_off[j] ^ (16 * (2 * ks + h))));
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks == 0) {
                if constexpr (TI + TJ == 8) {
                    asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(wf[0][0]), "+v"(wf[0][1]), "+v"(wf[0][2]),
                                 "+v"(wf[0][3]), "+v"(xf[0][0]), "+v"(xf[0][1]), "+v"(xf[0][2]), "+v"(xf[0][3]));
                } else if constexpr (TI + TJ == 6) {
                    asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(wf[0][0]), "+v"(wf[0][1]), "+v"(xf[0][0]),
                                 "+v"(xf[0][1]), "+v"(xf[0][2]), "+v"(xf[0][3]));
                } else {
                    asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(wf[0][0]), "+v"(wf[0][1]), "+v"(xf[0][0]),
                                 "+v"(xf[0][1]));
                }
            } else {
                if constexpr (TI + TJ == 8) {
                    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(wf[1][0]), "+v"(wf[1][1]), "+v"(wf[1][2]),
                                 "+v"(wf[1][3]), "+v"(xf[1][0]), "+v"(xf[1][1]), "+v"(xf[1][2]), "+v"(xf[1][3]));
                } else if constexpr (TI + TJ == 6) {
                    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(wf[1][0]), "+v"(wf[1][1]), "+v"(xf[1][0]),
                                 "+v"(xf[1][1]), "+v"(xf[1][2]), "+v"(xf[1][3]));
                } else {
                    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(wf[1][0]), "+v"(wf[1][1]), "+v"(xf[1][0]),
                                 "+v"(xf[1][1]));
                }
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32x32x16(wf[ks][i], xf[ks][j], acc[i][j]);
            if (ks == 0) mid();
        }
    };
    auto no_mid = [] {};

    const int nk = K / kTBK;
    static_assert(WQ == kINT4, "bf16 experts use tile_gemm_bf16 and tile_gemm2_bf16_pp");
    // The 16 code bytes per weight-tile row for stage j, C(j), are
    // copied at step j-4 into code slot j % 4 (one direct-to-LDS load per
    // wavefront: lane L's bytes land at 16 L of the wavefront's 1 KB, and
    // each wavefront dequantises only the rows it copied itself, so its own
    // vmcnt guards them),
    // and the dispatch rows X(j) at step j-3, spread evenly over the four
    // wavefronts (XROWS / 64 loads each).  A wavefront's loads thus go out
    // in the order
    //   C(0) X(0) C(1) X(1) C(2) X(2) C(3) | X(3) C(4) | X(4) C(5) | ...
    // (prologue | step 0 | step 1 ...), and a wait for one of them counts
    // the loads issued after it.  The scales of the row's next 8 groups
    // (16 bytes, 32 stages) follow the same route every 32 stages, issued
    // before the codes of the first stage that needs them; being extra
    // loads that the counts leave out, they can only lengthen a wait.
    // Step s:
    //   wait for X(s) and for this thread's LDS stores (W(s), written at
    //   step s-1); barrier (publishes stage s, frees the slot of s-1);
    //   issue X(s+3) into that slot and C(s+4); wait for C(s+1) and read
    //   its codes; multiply stage s, expanding those codes to bf16 in
    //   registers between the MFMAs of its first substep (one wavefront
    //   per SIMD: VALU work placed between MFMAs runs while they execute,
    //   6 operations after each MFMA measured best); then store them to
    //   LDS slot (s+1) % 4 (last read at step s-3, before the barrier of
    //   step s-2).
    // K is a multiple of 1024: the stages come in whole blocks of 32.
    constexpr int XL = XROWS / 64;  // dispatch-row loads per wavefront per stage
    const char* cbase = reinterpret_cast<const char*>(Wexp);
    const char* sbase = reinterpret_cast<const char*>(Wsc);
    // lane L of wavefront w copies the codes (and scales) of weight-tile
    // row 64 (L / 16) + 16 w + L % 16: the rows this wavefront dequantises
    const uint32_t wrow = (uint32_t)min(n0 + 64 * (lane >> 4) + 16 * wave + (lane & 15), N - 1);
    const uint32_t coff = wrow * ((uint32_t)K / 2);
    const uint32_t soff = wrow * ((uint32_t)K / 128) * 2;
    // rows past the tile's dispatch rows (and weight rows past N) are clamped to a valid row: they
    // only feed outputs that are never stored
    uint32_t xoff_e[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int trow = wave * (XROWS / 4) + 16 * i + (lane >> 2);
        const int drow = min(trow, rows - 1);
        const uint32_t arow = (WHICH == 1) ? (uint32_t)a_rows[p0 + drow] : (uint32_t)(p0 + drow);
        xoff_e[i] = arow * xrowbytes + 16 * lseg;
    }
    auto issue_xe = [&](int kt, int buf) {
        const uint32_t kb = (uint32_t)kt * (kTBK * 2);
#pragma unroll
        for (int i = 0; i < XL; ++i)
            copy_rows_to_lds(xbase, xoff_e[i] + kb, &Xt[buf][(wave * (XROWS / 4) + 16 * i) * 64]);
    };
    auto issue_c = [&](int kt) { copy_rows_to_lds(cbase, coff + (uint32_t)kt * 16, &Ct[kt % kStages][wave * 1024]); };
    auto issue_scales = [&](int blk) {  // groups 8 blk .. 8 blk + 7 (stages 32 blk .. 32 blk + 31)
        copy_rows_to_lds(sbase, soff + (uint32_t)blk * 16, &St[blk & 1][wave * 1024]);
    };
    // Dequantisation: thread (wavefront w, lane l) writes 16-byte physical
    // slot l & 3 of weight-tile rows 64 j + 16 w + l / 4, j = 0..3, so each
    // of its LDS stores covers 1 KB contiguously (free of bank conflicts);
    // that slot holds logical segment lseg of every one of those rows.  Row
    // 64 j + 16 w + r was copied by lane 16 j + r of this wavefront: its
    // codes sit at 1024 w + 256 j + 16 r of the code slot.
    const uint32_t cread = lds_addr(Ct[0]) + 1024 * wave + 16 * (lane >> 2) + 4 * lseg;
    const uint32_t sread = lds_addr(St[0]) + 1024 * wave + 16 * (lane >> 2);
    const uint32_t wdst = 1024 * wave + 16 * lane;
    uint32_t sc0, sc1, sc2, sc3;  // group scales of this thread's four rows
    auto read_scales = [&](int g) {
        ds_read_scales(sread + (uint32_t)((g >> 3) & 1) * 4096 + (uint32_t)(g & 7) * 2, sc0, sc1, sc2, sc3);
    };
    // rem = stages after s (>= 0); the counts follow the issue order above
    auto wait_x = [&](int rem) {
        if (rem >= 3) wait_vmcnt<3 + 2 * XL>();
        else if (rem == 2) wait_vmcnt<2 + 2 * XL>();
        else if (rem == 1) wait_vmcnt<1 + XL>();
        else wait_vmcnt<0>();
    };
    // C(s+1) landed; rem = stages after s (>= 1)
    auto wait_c = [&](int rem) {
        if (rem >= 4) wait_vmcnt<3 + 3 * XL>();
        else if (rem == 3) wait_vmcnt<2 + 3 * XL>();
        else if (rem == 2) wait_vmcnt<1 + 2 * XL>();
        else wait_vmcnt<XL>();
    };
    auto dequant = [&](int j) {  // stage j's codes -> LDS slot j % 4 (scales of group j / 4 loaded)
        uint32_t w0, w1, w2, w3;
        ds_read_codes(cread + (uint32_t)(j % kStages) * 4096, w0, w1, w2, w3);
        const uint32_t wb = lds_addr(Wt[j % kStages]) + wdst;
        dequant_word_to_lds(w0, sc0, wb);
        dequant_word_to_lds(w1, sc1, wb + 4096);
        dequant_word_to_lds(w2, sc2, wb + 8192);
        dequant_word_to_lds(w3, sc3, wb + 12288);
    };
    // prologue
    issue_scales(0);
    issue_c(0);
    issue_xe(0, 0);
    issue_c(1);
    issue_xe(1, 1);
    issue_c(2);
    issue_xe(2, 2);
    issue_c(3);
    wait_c(4);
    read_scales(0);
    dequant(0);

    // one step; J = s % 4 (static), rem = nk - 1 - s (static in each call below)
    auto step = [&](int s, const int J, const int rem) {
        wait_x(rem);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier();
        if (rem >= 3) issue_xe(s + 3, (J + 3) % kStages);
        if (rem >= 4) issue_c(s + 4);
        if (rem >= 1) {
            // stage s + 1's codes are expanded between the MFMAs of stage s's
            // first substep and written to their (free) slot after stage s
            wait_c(rem);
            if (J == 3) read_scales((s + 1) >> 2);
            uint32_t w0, w1, w2, w3;
            ds_read_codes(cread + (uint32_t)((s + 1) % kStages) * 4096, w0, w1, w2, w3);
            uint4 d0, d1, d2, d3;
            compute(J, [&] {
                d0 = dequant_word(w0, sc0);
                d1 = dequant_word(w1, sc1);
                d2 = dequant_word(w2, sc2);
                d3 = dequant_word(w3, sc3);
                // one MFMA, then a share of the expansion's VALU operations, in turn
#pragma unroll
                for (int m = 0; m < TI * TJ; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kInt4MixValu, 0);
                }
            });
            const uint32_t wb = lds_addr(Wt[(s + 1) % kStages]) + wdst;
            ds_write16(wb, d0.x, d0.y, d0.z, d0.w);
            ds_write16(wb + 4096, d1.x, d1.y, d1.z, d1.w);
            ds_write16(wb + 8192, d2.x, d2.y, d2.z, d2.w);
            ds_write16(wb + 12288, d3.x, d3.y, d3.z, d3.w);
            return;
        }
        if (rem >= 1) {
            wait_c(rem);
            if (J == 3) read_scales((s + 1) >> 2);  // stage s + 1 opens a new group
            dequant(s + 1);
        }
        compute(J, no_mid);
    };
    int s0 = 0;
    for (; s0 + 8 <= nk; s0 += 4) {  // steady state: every step has 4 or more stages after it
        if ((s0 & 31) == 0 && s0 + 32 < nk) issue_scales((s0 >> 5) + 1);
        step(s0, 0, 4);
        step(s0 + 1, 1, 4);
        step(s0 + 2, 2, 4);
        step(s0 + 3, 3, 4);
    }
    step(s0, 0, 3);  // the last four stages
    step(s0 + 1, 1, 2);
    step(s0 + 2, 2, 1);
    step(s0 + 3, 3, 0);

    // the last stage waited for every load (vmcnt 0), so nothing lands in the staging area
    if constexpr (WHICH == 1 && ACT != kActSwiglu) {
        store_tile_lds<TI, TJ, ACT, 4, kInt4LdsBytes>(acc, &Wt[0][0], out, N, n0, p0, rows, wn, wm, r, h, true);
    } else if constexpr (WHICH == 2) {
        store_tile_lds_f32<TI, TJ, 4, kInt4LdsBytes>(acc, &Wt[0][0], static_cast<float*>(out), N, n0, p0, rows, wn, wm, r, h, true);
    } else {
        store_tile<WHICH, TI, TJ, ACT>(acc, out, N, n0, p0, rows, wn, wm, r, h);
    }
}

// bf16 weights, K-stages of 64: each stage holds 128 bytes (one whole
// 128-byte line) of every tile row, 32 KB per operand.  Copying whole lines runs the direct-to-LDS loads
// about 1.5x faster than half lines (measured on L2-resident data: 16 rows x
// 64 B per instruction reach 21-24 TB/s, 8 rows x 128 B 33 TB/s).  The
// eight 16-byte segments of a row sit in slots permuted by (row >> 1) & 7,
// so 16 consecutive rows read at one logical segment hit 16 distinct bank
// groups.  Stage k is multiplied in four k-substeps of 16.  Logical segment seg of tile row
// `row` sits at byte row * 128 + 16 * (seg ^ ((row >> 1) & 7)) of a stage.
//
// Eight wavefronts per workgroup, two per SIMD, so one wavefront's MFMAs run
// while the other waits on fragment reads, copies or the barrier (measured
// 7-15% faster per 256-row tile than four wavefronts of 128 x 128).  With 256
// dispatch rows each of the 8 computes 128 weight rows x 64 dispatch rows
// (128 accumulators, about 220 registers in all); with 128 rows 64 x 64; with
// 64 rows (weight-streaming tiles) only wavefronts 0-3 compute 64 x 64, which
// measured faster than spreading such a tile over all 8.  All 8 copy: wavefront
// w moves tile rows [32 w, 32 w + 32) of each operand.
//
// Schedule (measured faster than copying right after the barrier):
// * weights (two slots) are copied one stage ahead, dispatch rows (three
//   slots, each stage's rows are new data for the XCD's L2) two ahead;
// * a step's copies are issued while its first fragment reads are in
//   flight (weights) or after its first half of MFMAs (dispatch rows), so
//   they do not delay the reads that start the step;
// * the last substep's MFMAs are held over the next barrier and issued
//   under the next stage's first reads, so the matrix pipe has queued
//   work across the stage boundary;
// * a scheduling fence after each first half stops the compiler from
//   hoisting the second fragment wait above those MFMAs.
// Issue order W(k+1) | X(k+2): at step k only X(k+1) (4 loads of the
// wavefronts that copy dispatch rows) may still be in flight.  The barrier
// publishes stage k and frees the slots of stage k-1 (W) and k-1 (X), which
// the step's copies reuse.
template <int WHICH, int TI, int TJ, int XROWS, int ACT, int MWAVE = 8>
__device__ __forceinline__ void tile_gemm_bf16(uint8_t* lds, const uint16_t* __restrict__ A,
                                               const int32_t* __restrict__ a_rows, const void* Wexp,
                                               void* __restrict__ out, int N, int K, int n0, int p0, int rows,
                                               int kt0, int nk) {
    constexpr int NWAVE = 8;
    constexpr int WN_WAVES = 256 / (32 * TI);
    static_assert(WN_WAVES * (XROWS / (32 * TJ)) == MWAVE, "wave grid");
    const bool math = (threadIdx.x >> 6) < MWAVE;
    constexpr uint32_t kStage = 256 * 128;
    // A tile of at most 128 dispatch rows is an expert's only m-tile or its last, so no later tile re-reads its
    // weights: they are copied with the non-temporal hint (each instruction moves whole 128-byte lines).  On
    // the balanced 128-expert prefill, where nearly every tile streams its weights, W1 3.18 -> 2.89 ms.
    constexpr bool kWeightsOnce = XROWS <= 128;
    uint8_t* const Wr = lds;
    uint8_t* const Xr = lds + 2 * kStage;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // wavefront w copies tile rows [32 w, 32 w + 32): 4 instructions of 8 rows x 128 bytes per operand
    const bool xload = 32 * wave < XROWS;
    const char* wbase = reinterpret_cast<const char*>(Wexp);
    const char* xbase = reinterpret_cast<const char*>(A);
    const uint32_t rowbytes = (uint32_t)K * 2;
    uint32_t woff[4], xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int trow = 32 * wave + 8 * i + (lane >> 3);
        const uint32_t seg = (uint32_t)((lane & 7) ^ ((trow >> 1) & 7));
        woff[i] = (uint32_t)min(n0 + trow, N - 1) * rowbytes + 16 * seg;
        const int drow = min(trow, rows - 1);
        const uint32_t arow = (WHICH == 1) ? (uint32_t)a_rows[p0 + drow] : (uint32_t)(p0 + drow);
        xoff[i] = arow * rowbytes + 16 * seg;
    }
    // stages kt0 .. kt0 + nk - 1 of the K dimension (kt counts from 0 within them)
    auto issue_w = [&](int kt) {
        const uint32_t kb = (uint32_t)(kt0 + kt) * 128;
        uint8_t* slot = Wr + (kt & 1) * kStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (kWeightsOnce)
                copy_rows_to_lds_nt(wbase, woff[i] + kb, slot + (32 * wave + 8 * i) * 128);
            else
                copy_rows_to_lds(wbase, woff[i] + kb, slot + (32 * wave + 8 * i) * 128);
        }
    };
    auto issue_x = [&](int kt) {
        const uint32_t kb = (uint32_t)(kt0 + kt) * 128;
        uint8_t* slot = Xr + (kt % 3) * kStage;
        if (xload) {
#pragma unroll
            for (int i = 0; i < 4; ++i) copy_rows_to_lds(xbase, xoff[i] + kb, slot + (32 * wave + 8 * i) * 128);
        }
    };
    const int wn = (wave % WN_WAVES) * (32 * TI);
    const int wm = (wave / WN_WAVES) * (32 * TJ);
    const int r = lane & 31;
    const int h = lane >> 5;
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    uint32_t wrow_off[TI], xrow_off[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) wrow_off[i] = (uint32_t)(wn + 32 * i + r) * 128;
#pragma unroll
    for (int j = 0; j < TJ; ++j) xrow_off[j] = (uint32_t)(wm + 32 * j + r) * 128;
    const uint32_t swz = (uint32_t)((r >> 1) & 7);
    auto read_sub = [&](uint32_t wb, uint32_t xb, int ks, bf16x8 (&wf)[TI], bf16x8 (&xf)[TJ]) {
        if (MWAVE < 8 && !math) return;
        const uint32_t so = 16 * ((uint32_t)(2 * ks + h) ^ swz);
#pragma unroll
        for (int i = 0; i < TI; ++i) wf[i] = ds_read16(wb + wrow_off[i] + so);
#pragma unroll
        for (int j = 0; j < TJ; ++j) xf[j] = ds_read16(xb + xrow_off[j] + so);
    };
    auto mma_sub = [&](const bf16x8 (&wf)[TI], const bf16x8 (&xf)[TJ]) {
        if (MWAVE < 8 && !math) return;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32x32x16(wf[i], xf[j], acc[i][j]);
    };
    // wait until at most N fragment reads are outstanding, then tie the fragments to the wait
    auto wait_frags = [&](auto nc, bf16x8 (&wf)[TI], bf16x8 (&xf)[TJ]) {
        constexpr int NN = decltype(nc)::value;
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NN) : "memory");
#pragma unroll
        for (int i = 0; i < TI; ++i) asm volatile("" : "+v"(wf[i]));
#pragma unroll
        for (int j = 0; j < TJ; ++j) asm volatile("" : "+v"(xf[j]));
    };
    using NF = std::integral_constant<int, TI + TJ>;
    using N0 = std::integral_constant<int, 0>;
    issue_w(0);
    issue_x(0);
    if (nk > 1) issue_x(1);
    bf16x8 dw[TI], dx[TJ];
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk && xload) wait_vmcnt<4>(); else wait_vmcnt<0>();
        barrier();
        const uint32_t wb = lds_addr(Wr + (kt & 1) * kStage), xb = lds_addr(Xr + (kt % 3) * kStage);
        bf16x8 w0[TI], x0[TJ], w1[TI], x1[TJ];
        read_sub(wb, xb, 0, w0, x0);
        read_sub(wb, xb, 1, w1, x1);
        if (kt > 0) mma_sub(dw, dx);
        if (kt + 1 < nk) issue_w(kt + 1);
        wait_frags(NF{}, w0, x0);
        mma_sub(w0, x0);
        __builtin_amdgcn_sched_barrier(0);
        wait_frags(N0{}, w1, x1);
        mma_sub(w1, x1);
        if (kt + 2 < nk) issue_x(kt + 2);
        read_sub(wb, xb, 2, w0, x0);
        read_sub(wb, xb, 3, dw, dx);
        wait_frags(NF{}, w0, x0);
        mma_sub(w0, x0);
        __builtin_amdgcn_sched_barrier(0);
        wait_frags(N0{}, dw, dx);
    }
    mma_sub(dw, dx);
    if constexpr (WHICH == 1 && ACT != kActSwiglu) {
        store_tile_lds<TI, TJ, ACT, NWAVE, kBf16LdsBytes>(acc, lds, out, N, n0, p0, rows, wn, wm, r, h, math);
    } else if constexpr (WHICH == 2) {
        store_tile_lds_f32<TI, TJ, NWAVE, kBf16LdsBytes>(acc, lds, static_cast<float*>(out), N, n0, p0, rows, wn, wm, r, h, math);
    } else {
        if (math) store_tile<WHICH, TI, TJ, ACT>(acc, out, N, n0, p0, rows, wn, wm, r, h);
    }
}


// ---- bf16 GEMM2, 256 dispatch rows: two wavefront groups in ping-pong ----
// The K-stages of 64 and the LDS layout of tile_gemm_bf16 (whole 128-byte
// lines per tile row, 32 KB per operand and stage): kPpW weight slots and
// kPpX dispatch-row slots, 160 KB in all.  Whole-line copies matter here:
// with K-stages of 32 (half lines) the copies alone took longer than the
// MFMAs (dense 4096 x 16384 x 4096: 0.37 ms of copies against 0.33 ms of
// MFMAs and fragment reads), twice as long again with 32 KB rows.
//
// Group 0 (wavefronts 0-3, one per SIMD) and group 1 (wavefronts 4-7, the
// other wavefront of each SIMD) take turns: time is cut into phases ended
// by a workgroup barrier, and in every phase one group multiplies one half
// of a stage (16 MFMAs per wavefront, K = 32, from fragments already in
// registers) while the other reads its fragments of the next half from LDS
// and issues copies.  Each SIMD's matrix pipe is then fed by one wavefront
// while the other's LDS reads and copies run beside it, and no wavefront
// waits on its own reads.  Half-stage h (stage h / 2) is multiplied by
// group 0 in phase 2h and by group 1 in phase 2h + 1; group 0 reads its
// fragments in phase 2h - 1, group 1 in phase 2h.
//
// Copies: group 0 copies the weight tile, group 1 the dispatch rows, each
// wavefront 64 tile rows (8 loads of 8 rows x 128 bytes) per stage, issued
// as two halves of 4 loads in two phases (all 8 at once stalled the
// issuing wavefronts: GEMM2 5% slower).  Stage s is last read in phase
// 4s + 2 (group 1, half-stage 2s + 1), and stage s + 1 must be published
// by the barrier ending phase 4s + 2.  Group 1 issues the first half of
// dispatch-row stage s + kPpX right after its own reads of phase 4s + 2
// have returned (group 0 read that half-stage a phase earlier) and the
// second half in phase 4s + 4; it waits for its loads of stage s + 1 in
// phase 4s + 2.  Group 0 issues the halves of weight stage s + kPpW in
// phases 4s + 3 and 4s + 5 and waits for its loads of stage s + 1 after its
// MFMAs of phase 4s + 2.  Fragment reads are waited for before the barrier
// that ends their phase, so no slot is refilled under a read.
//
// Measured against tile_gemm_bf16 on 256-row tiles (same box, round-robin):
// GEMM2 3-5% faster on the skewed 16- and 128-expert prefills, GEMM1 2-4%
// slower on the 16-expert one, so GEMM1 keeps tile_gemm_bf16.
constexpr int kPpW = 3, kPpX = 2;

template <int OFF>
__device__ __forceinline__ bf16x8 ds_read16_at(uint32_t addr) {
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}

// GEMM2 (A = H, rows p0 .. p0 + rows - 1; fp32 Y), stages kt0 .. kt0 + ns - 1 of 64 along K
__device__ __forceinline__ void tile_gemm2_bf16_pp(uint8_t* lds, const uint16_t* __restrict__ A, const void* Wexp,
                                                   float* __restrict__ out, int N, int K, int n0, int p0, int rows,
                                                   int kt0, int ns) {
    constexpr int TI = 4, TJ = 2;
    constexpr uint32_t kSlot = 256 * 128;
    static_assert((kPpW + kPpX) * kSlot <= kBf16LdsBytes, "rings exceed the kernel's LDS");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int v = wave & 3;
    const int R = grp == 0 ? kPpW : kPpX;  // this group's ring
    const uint32_t wring = lds_addr(lds), xring = lds_addr(lds + kPpW * kSlot);

    // this wavefront's copies: tile rows [64 v, 64 v + 64) of its group's operand, 8 rows x 128 bytes per
    // load; lane L moves logical segment (L & 7) ^ ((row >> 1) & 7) of row L >> 3 of its block, which lands
    // at LDS byte 16 L of the block.  Rows past N (weights) or past the tile's rows (dispatch rows) are
    // clamped: they only feed outputs that are never stored.
    const uint32_t rowbytes = (uint32_t)K * 2;
    const char* src = grp == 0 ? reinterpret_cast<const char*>(Wexp) : reinterpret_cast<const char*>(A);
    uint32_t goff[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int trow = 64 * v + 8 * q + (lane >> 3);
        const uint32_t seg = (uint32_t)((lane & 7) ^ ((trow >> 1) & 7));
        const uint32_t grow = grp == 0 ? (uint32_t)min(n0 + trow, N - 1) : (uint32_t)(p0 + min(trow, rows - 1));
        goff[q] = grow * rowbytes + 16 * seg;
    }
    uint8_t* const ring = lds + grp * (kPpW * kSlot) + 8192 * v;
    // half hf of this wavefront's loads of stage st: tile rows 64 v + 32 hf .. + 32
    auto issue_half = [&](int st, int hf) {
        if (st >= ns) return;
        const uint32_t kb = (uint32_t)(kt0 + st) * 128;
        uint8_t* slot = ring + (st % R) * kSlot;
        if (hf == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) copy_rows_to_lds(src, goff[q] + kb, slot + 1024 * q);
        } else {
#pragma unroll
            for (int q = 4; q < 8; ++q) copy_rows_to_lds(src, goff[q] + kb, slot + 1024 * q);
        }
    };
    // wait until at most n of this wavefront's loads are in flight (n a multiple of 4, at most 16)
    auto wait_loads = [&](int n) {
        if (n >= 16) wait_vmcnt<16>();
        else if (n >= 12) wait_vmcnt<12>();
        else if (n >= 8) wait_vmcnt<8>();
        else if (n >= 4) wait_vmcnt<4>();
        else wait_vmcnt<0>();
    };

    // fragments of half-stage hs: weight rows wn + 32 i + r and dispatch rows wm + 32 j + r, k-substep
    // 2 (hs & 1) + ks; lane half h reads logical segment 2 (2 (hs & 1) + ks) + h; tiles i and j sit 4 KB apart
    // with the same permutation
    const int wn = (wave & 1) * 128;
    const int wm = (wave >> 1) * 64;
    const int r = lane & 31;
    const int h = lane >> 5;
    const uint32_t swz = (uint32_t)((r >> 1) & 7);
    uint32_t lw[4], lx[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const uint32_t so = 16 * ((uint32_t)(2 * s4 + h) ^ swz);
        lw[s4] = (uint32_t)(wn + r) * 128 + so;
        lx[s4] = (uint32_t)(wm + r) * 128 + so;
    }
    bf16x8 wf[2][TI], xf[2][TJ];
    auto read_frags = [&](int hs, auto hi) {  // hi = hs & 1, a compile-time constant
        const int st = hs >> 1;
        const uint32_t wb = wring + (st % kPpW) * kSlot, xb = xring + (st % kPpX) * kSlot;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint32_t aw = wb + lw[2 * decltype(hi)::value + ks], ax = xb + lx[2 * decltype(hi)::value + ks];
            wf[ks][0] = ds_read16_at<0>(aw);
            wf[ks][1] = ds_read16_at<4096>(aw);
            wf[ks][2] = ds_read16_at<8192>(aw);
            wf[ks][3] = ds_read16_at<12288>(aw);
            xf[ks][0] = ds_read16_at<0>(ax);
            xf[ks][1] = ds_read16_at<4096>(ax);
        }
    };
    auto wait_frags = [&] {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i) asm volatile("" : "+v"(wf[ks][i]));
#pragma unroll
            for (int j = 0; j < TJ; ++j) asm volatile("" : "+v"(xf[ks][j]));
        }
    };
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto mma = [&] {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32x32x16(wf[ks][i], xf[ks][j], acc[i][j]);
    };
    const int nh = 2 * ns;
    // a wavefront's step outside its multiply phases: the fragments of half-stage m, and the copies and
    // waits that fall in that phase
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    auto fetch = [&](int m, auto odd) {  // odd = m & 1
        if (m >= nh) return;
        read_frags(m, odd);
        if (grp == 0) {
            // weight stage m / 2 - 1 + kPpW into the slot of stage m / 2 - 1, no longer read
            if (m >= 2) issue_half(m / 2 - 1 + kPpW, decltype(odd)::value);
            wait_frags();
        } else {
            wait_frags();
            if (decltype(odd)::value) {  // that was the last read of stage st: its slot takes stage st + kPpX
                const int st = m / 2;
                issue_half(st + kPpX, 0);
                if (st + 1 < ns) wait_loads(st + 2 < ns ? 4 : 0);  // stage st + 1 in, half of st + 2 in flight
            } else if (m >= 2) {
                issue_half(m / 2 - 1 + kPpX, 1);
            }
        }
    };
    // Both groups run the same loop, multiply | barrier | fetch | barrier; group 1 enters it one phase
    // later (one more barrier before it, one fewer after the epilogue), so its multiply phases are group 0's
    // fetch phases.  The multiplies stay in straight-line code, which keeps the accumulators in AGPRs.  The
    // scheduling fences keep each phase's instructions on its side of the barrier (MFMAs are not memory
    // operations, so the barrier alone would not hold them).
    auto phase_end = [] {
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int st = 0; st < R; ++st) {
        issue_half(st, 0);
        issue_half(st, 1);
    }
    wait_loads(8 * (min(R, ns) - 1));  // stage 0 in
    barrier();
    fetch(0, Even{});
    if (grp == 1) phase_end();
    for (int st = 0; st < ns; ++st) {  // half-stages 2 st and 2 st + 1
        mma();
        phase_end();
        fetch(2 * st + 1, Odd{});
        phase_end();
        mma();
        if (grp == 0 && st + 1 < ns) wait_loads(st + 2 < ns ? 8 : 0);  // weights: st + 1 in, st + 2 in flight
        phase_end();
        fetch(2 * st + 2, Even{});
        phase_end();
    }
    // every load has landed and every fragment read has returned: the epilogue may stage through the rings
    store_tile_lds_f32<TI, TJ, 8, kBf16LdsBytes>(acc, lds, out, N, n0, p0, rows, wn, wm, r, h, true);
    // group 0 has passed one barrier fewer; it takes it here, where the accumulators are no longer live (a
    // conditional barrier while they are makes the compiler copy them all out of the AGPRs)
    if (grp == 0) barrier();
}


// W: the experts' weights, W_stride bytes apart (bf16 [N][K] or INT4 codes
// [N][K/2]); Wsc: INT4 scales bf16 [E][N][K/128] (unused for bf16).  Only
// experts holding more than rows_lo rows are multiplied here.
template <int WQ, int WHICH, int ACT>
__global__ void __launch_bounds__(256, 1)
gemm_tiled_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                  const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ W, int64_t W_stride,
                  const uint16_t* __restrict__ Wsc, void* __restrict__ out, int N, int K, int ntiles_n, int rows_lo) {
    static_assert(WQ == kINT4, "bf16 experts use gemm_tiled_bf16_kernel");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kInt4LdsBytes];
    uint8_t (*Wt)[kTileBytes] = reinterpret_cast<uint8_t (*)[kTileBytes]>(smem);
    uint8_t (*Xt)[kTileBytes] = reinterpret_cast<uint8_t (*)[kTileBytes]>(smem + kStages * kTileBytes);
    uint8_t (*Ct)[4096] = reinterpret_cast<uint8_t (*)[4096]>(smem + 2 * kStages * kTileBytes);     // INT4 code ring
    uint8_t (*St)[4096] = reinterpret_cast<uint8_t (*)[4096]>(smem + 2 * kStages * kTileBytes + kStages * 4096);  // scales

    // An (empty) statement that clobbers an AGPR tells the backend this kernel
    // uses AGPRs, so it gives the MFMAs their AGPR-accumulator form (the
    // accumulators live in AGPRs, operands in VGPRs).
    asm volatile("" ::: "a0");
    // Tiles in m-major order: the workgroups running at one time (one per CU,
    // handed to the XCDs in turn) share the dispatch-row tiles of one or two
    // m-tiles and stream different weight tiles.  (Grouping 4-16 m-tiles per
    // XCD to share weight tiles in L2 measured no faster.)
    const MtileScan scan = scan_mtiles(offsets, E, kTBM, rows_lo, 0x7fffffff);
    const int mt = blockIdx.x / ntiles_n;
    const int nt = blockIdx.x - mt * ntiles_n;
    if (mt >= scan.total) return;
    int e, p0, rows;
    lookup_mtile(scan, offsets, kTBM, mt, &e, &p0, &rows);
    e = __builtin_amdgcn_readfirstlane(e);  // uniform across the workgroup: keep the bases scalar
    p0 = __builtin_amdgcn_readfirstlane(p0);
    rows = __builtin_amdgcn_readfirstlane(rows);
    const int n0 = nt * kTBN;
    const void* Wexp = W + (int64_t)e * W_stride;
    const void* Wsc_e = (WQ == kINT4) ? (const void*)(Wsc + (int64_t)e * N * (K / 128)) : nullptr;
    if (rows > 128)
        tile_gemm<WQ, WHICH, 4, 4, 256, ACT>(Wt, Xt, Ct, St, A, a_rows, Wexp, Wsc_e, out, N, K, n0, p0, rows);
    else if (rows > 64)
        tile_gemm<WQ, WHICH, 2, 4, 128, ACT>(Wt, Xt, Ct, St, A, a_rows, Wexp, Wsc_e, out, N, K, n0, p0, rows);
    else
        tile_gemm<WQ, WHICH, 2, 2, 64, ACT>(Wt, Xt, Ct, St, A, a_rows, Wexp, Wsc_e, out, N, K, n0, p0, rows);
}

// bf16 experts: 2 weight + 3 dispatch-row stages of 32 KB (160 KB, all of a
// CU's LDS), 8 wavefronts.
template <int WHICH, int ACT>
__global__ void __launch_bounds__(512, 1)
gemm_tiled_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
                       const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ W, int64_t W_stride,
                       void* __restrict__ out, int N, int K, int ntiles_n, int rows_lo, int ksplit,
                       int64_t split_stride) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kBf16LdsBytes];
    asm volatile("" ::: "a0");  // accumulators in AGPRs (see gemm_tiled_kernel)
    const MtileScan scan = scan_mtiles(offsets, E, kTBM, rows_lo, 0x7fffffff);
    // ksplit = 2 (GEMM2 only): workgroups 2 b and 2 b + 1 take the two K halves
    // of tile b and write them to out and out + split_stride (fp32 partials)
    const int ks = blockIdx.x % ksplit;
    const int b = blockIdx.x / ksplit;
    const int mt = b / ntiles_n;
    const int nt = b - mt * ntiles_n;
    const int nk = K / 64 / ksplit, kt0 = ks * nk;
    if (WHICH == 2) out = static_cast<float*>(out) + ks * split_stride;
    if (mt >= scan.total) return;
    int e, p0, rows;
    lookup_mtile(scan, offsets, kTBM, mt, &e, &p0, &rows);
    e = __builtin_amdgcn_readfirstlane(e);
    p0 = __builtin_amdgcn_readfirstlane(p0);
    rows = __builtin_amdgcn_readfirstlane(rows);
    const int n0 = nt * kTBN;
    const void* Wexp = W + (int64_t)e * W_stride;
    if (rows > 128) {
        if constexpr (WHICH == 2)
            tile_gemm2_bf16_pp(smem, A, Wexp, static_cast<float*>(out), N, K, n0, p0, rows, kt0, nk);
        else
            tile_gemm_bf16<WHICH, 4, 2, 256, ACT>(smem, A, a_rows, Wexp, out, N, K, n0, p0, rows, kt0, nk);
    } else if (rows > 64) {
        tile_gemm_bf16<WHICH, 2, 2, 128, ACT>(smem, A, a_rows, Wexp, out, N, K, n0, p0, rows, kt0, nk);
    } else {
        tile_gemm_bf16<WHICH, 2, 2, 64, ACT, 4>(smem, A, a_rows, Wexp, out, N, K, n0, p0, rows, kt0, nk);
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
    const int64_t Tk = a.T * a.k;
    const int64_t max_mtiles = Tk / kTBM + (Tk < a.E ? Tk : a.E);
    const int ntiles_n = (int)((a.N + kTBN - 1) / kTBN);
    const int64_t blocks = max_mtiles * ntiles_n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    const uint8_t* W = static_cast<const uint8_t*>(a.W);
    const uint16_t* S = static_cast<const uint16_t*>(a.W_scales);
    dim3 grid((unsigned)blocks), block(256);
    const int N = (int)a.N, K = (int)a.K;
#define MOE_TILED_LAUNCH(WQ_, WHICH_, ACT_)                                                                        \
    hipLaunchKernelGGL((gemm_tiled_kernel<WQ_, WHICH_, ACT_>), grid, block, 0, stream, A, a.a_rows, a.offsets, a.E, W, \
                       a.W_stride, S, a.out, N, K, ntiles_n, a.rows_lo)
    if (a.w_dtype == kINT4) {
        if (a.which == 2) MOE_TILED_LAUNCH(kINT4, 2, kActGelu);
        else if (a.act == kActSilu) MOE_TILED_LAUNCH(kINT4, 1, kActSilu);
        else if (a.act == kActSwiglu) MOE_TILED_LAUNCH(kINT4, 1, kActSwiglu);
        else MOE_TILED_LAUNCH(kINT4, 1, kActGelu);
    } else {
        const int ksplit = (a.which == 2 && a.ksplit == 2 && K % 128 == 0) ? 2 : 1;
        if ((int64_t)blocks * ksplit > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 grid_k((unsigned)(blocks * ksplit));
        const int64_t split_stride = a.T * a.k * a.N;
#define MOE_TILED_BF16_LAUNCH(WHICH_, ACT_)                                                                        \
    hipLaunchKernelGGL((gemm_tiled_bf16_kernel<WHICH_, ACT_>), grid_k, dim3(512), 0, stream, A, a.a_rows,            \
                       a.offsets, a.E, W, a.W_stride, a.out, N, K, ntiles_n, a.rows_lo, ksplit, split_stride)
        if (a.which == 2) MOE_TILED_BF16_LAUNCH(2, kActGelu);
        else if (a.act == kActSilu) MOE_TILED_BF16_LAUNCH(1, kActSilu);
        else if (a.act == kActSwiglu) MOE_TILED_BF16_LAUNCH(1, kActSwiglu);
        else MOE_TILED_BF16_LAUNCH(1, kActGelu);
#undef MOE_TILED_BF16_LAUNCH
    }
#undef MOE_TILED_LAUNCH
    return hipGetLastError();
}

}  // namespace moe
