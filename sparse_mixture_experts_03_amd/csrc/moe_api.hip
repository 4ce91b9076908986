// C ABI of the MoE-layer forward: argument checks, workspace carve-up and the
// stream-ordered launch sequence
//   [router encoder: GEMM (one expert) -> GeLU]
//   router (partial logits, finalize) -> permute -> GEMM1 (+GeLU) -> GEMM2 -> combine,
// with capacity-limited dispatch
//   router (+ z and p rows) -> permute -> capacity -> permute -> GEMM1 -> GEMM2 -> combine.
// No host synchronisation and no host<->device copy happens inside a call;
// counts and the dispatch order stay on the device and every kernel finds its
// work from them.
#include <algorithm>
#include <math.h>
#include <mutex>
#include <string.h>

#include "../../include/moe.h"
#include "common.hpp"
#include "launch.hpp"

// Device scratch of moe_forward_no_alloc: one copy per GPU, held from the
// library's load on that GPU until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int64_t kMaxDim = int64_t(1) << 17;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int64_t kStreamingMaxT = 16;  // automatic path: streaming kernel up to 16 tokens
constexpr int64_t kMaxArrayBytes = int64_t(1) << 32;

moe_status hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t elem_bits(int32_t dtype) { return dtype == MOE_DTYPE_F32 ? 32 : dtype == MOE_DTYPE_BF16 ? 16 : 4; }

// The tiled kernel takes INT4 weights when both GEMMs' K (d and d_ff) hold
// whole blocks of 8 scale groups.
bool int4_tiled_ok(const moe_config& c) { return c.d % 1024 == 0 && c.d_ff % 1024 == 0; }

// Rows of each expert's W1: d_ff, or 2 d_ff (gate and up) for SwiGLU.
int64_t w1_rows(const moe_config& c) { return c.expert_act == MOE_ACT_SWIGLU ? 2 * c.d_ff : c.d_ff; }

moe_status check_config(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID_ARGUMENT;
    if (c->T < 0 || c->T > kMaxT) return MOE_ERR_INVALID_ARGUMENT;
    if (c->E < 1 || c->E > kMaxE) return MOE_ERR_INVALID_ARGUMENT;
    if (c->k < 1 || c->k > kMaxK || c->k > c->E) return MOE_ERR_INVALID_ARGUMENT;
    if (c->d < 64 || c->d > kMaxDim || c->d % 64 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (c->d_ff < 64 || c->d_ff > kMaxDim || c->d_ff % 64 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (!(c->tau > 0.0f) || !isfinite(c->tau)) return MOE_ERR_INVALID_ARGUMENT;
    if (c->use_gumbel != 0 && c->use_gumbel != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (c->gemm_path < MOE_GEMM_AUTO || c->gemm_path > MOE_GEMM_TILED) return MOE_ERR_INVALID_ARGUMENT;
    if (c->reserved != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (!(c->capacity_factor == 0.0f || (c->capacity_factor > 0.0f && isfinite(c->capacity_factor))))
        return MOE_ERR_INVALID_ARGUMENT;
    if (c->capacity_policy != MOE_CAPACITY_DROP && c->capacity_policy != MOE_CAPACITY_REROUTE)
        return MOE_ERR_INVALID_ARGUMENT;
    if (c->gate_norm != 0 && c->gate_norm != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (!(c->noise_std >= 0.0f) || !isfinite(c->noise_std)) return MOE_ERR_INVALID_ARGUMENT;
    // a rerouted or dropped slot has no renormalised gate defined
    if (c->gate_norm == 1 && c->capacity_factor > 0.0f) return MOE_ERR_UNSUPPORTED;
    if (c->expert_act < MOE_ACT_GELU || c->expert_act > MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARGUMENT;
    if (c->router_hidden < 0 || c->router_hidden > kMaxDim || c->router_hidden % 64 != 0)
        return MOE_ERR_INVALID_ARGUMENT;
    if (c->act_dtype != MOE_DTYPE_F32 && c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (c->w_dtype < MOE_DTYPE_F32 || c->w_dtype > MOE_DTYPE_INT4_G128) return MOE_ERR_INVALID_ARGUMENT;
    if (c->w_dtype == MOE_DTYPE_INT4_G128 && (c->d % 128 != 0 || c->d_ff % 128 != 0))
        return MOE_ERR_INVALID_ARGUMENT;
    // supported pairings: F32/F32, BF16/BF16, BF16/INT4
    if ((c->act_dtype == MOE_DTYPE_F32) != (c->w_dtype == MOE_DTYPE_F32)) return MOE_ERR_UNSUPPORTED;
    // the tiled INT4 kernel fetches 8 group scales (16 bytes) at a time
    if (c->w_dtype == MOE_DTYPE_INT4_G128 && c->gemm_path == MOE_GEMM_TILED && !int4_tiled_ok(*c))
        return MOE_ERR_UNSUPPORTED;
    // kernels address each activation array and each expert's matrix with 32-bit byte offsets
    const int64_t ab = c->act_dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int64_t Tk = c->T * c->k;
    if (c->T * c->d * ab >= kMaxArrayBytes || Tk * c->d_ff * 4 >= kMaxArrayBytes || Tk * c->d * 4 >= kMaxArrayBytes ||
        (int64_t)c->router_hidden * c->d * ab >= kMaxArrayBytes || c->T * c->router_hidden * 4 >= kMaxArrayBytes ||
        w1_rows(*c) * c->d * elem_bits(c->w_dtype) / 8 >= kMaxArrayBytes)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Expert capacity ceil(T k / E * capacity_factor), evaluated in binary64 and
// clamped to T (no expert can receive more than T assignments, since a
// token's k experts are distinct); 0 means dropless dispatch.
int64_t capacity_of(const moe_config& c) {
    if (c.capacity_factor == 0.0f || c.T == 0) return 0;
    const double v = ceil((double)c.T * (double)c.k / (double)c.E * (double)c.capacity_factor);
    return v >= (double)c.T ? c.T : (int64_t)v;
}

// Capacity can change the routing only when it is below T.
bool capacity_active(const moe_config& c) { return capacity_of(c) > 0 && capacity_of(c) < c.T; }

// Router workspace: the partial logits of the (last) router layer, and with a
// router encoder its one-expert offsets, fp32 pre-activations and hidden layer.
struct RouterLayout {
    size_t partial, enc_offsets, enc_pre, enc_h, total;
};

RouterLayout router_layout_of(const moe_config& c) {
    RouterLayout R;
    const int64_t d_in = c.router_hidden > 0 ? c.router_hidden : c.d;
    size_t off = 0;
    R.partial = off;
    off = round_up(off + moe::router_plan(c.T, d_in, c.E).partial_bytes, 256);
    R.enc_offsets = R.enc_pre = R.enc_h = 0;
    if (c.router_hidden > 0) {
        const size_t ab = c.act_dtype == MOE_DTYPE_F32 ? 4 : 2;
        R.enc_offsets = off;
        off += 256;
        R.enc_pre = off;
        off = round_up(off + sizeof(float) * (size_t)c.T * (size_t)c.router_hidden, 256);
        R.enc_h = off;
        off = round_up(off + ab * (size_t)c.T * (size_t)c.router_hidden, 256);
    }
    R.total = c.T == 0 ? 0 : off;
    return R;
}

struct Layout {
    size_t partial, offsets, sorted_token, pos, H, Y, z_rows, prob_rows, P1, total;
};

int gemm_path_of(const moe_config& c);

// K halves of the layer's GEMM1 (streaming bf16 kernel at decode sizes), as
// fp32 partials that act_halves_kernel adds in a fixed order before the
// activation: GEMM1 0.320 -> 0.312 ms on the 8-token, 128-expert decode.
int w1_ksplit_of(const moe_config& c) {
    return c.w_dtype == MOE_DTYPE_BF16 && gemm_path_of(c) == MOE_GEMM_STREAMING && c.T <= 16 ? 2 : 1;
}

// K halves of the layer's GEMM2, written as two fp32 partials that the
// combine adds in a fixed order: 2 for the streaming kernel at decode sizes
// (twice the workgroups streaming the same weights: bf16 decode layer step
// 0.687 -> 0.672 ms, INT4 decode unchanged), and for the bf16 tiled kernel
// when its grid holds fewer than four rounds of 256-row tiles for 256 CUs,
// so that the last, partly filled round of long tiles (K = d_ff) is split in
// two.  1 otherwise.
int w2_ksplit_of(const moe_config& c) {
    if (c.w_dtype != MOE_DTYPE_F32 && gemm_path_of(c) == MOE_GEMM_STREAMING && c.T <= 16) return 2;
    if (c.w_dtype != MOE_DTYPE_BF16 || gemm_path_of(c) != MOE_GEMM_TILED || c.d_ff % 128 != 0) return 1;
    const int64_t Tk = c.T * (int64_t)c.k;
    const int64_t mtiles = Tk / 256 + std::min<int64_t>(Tk, c.E);
    const int64_t ntiles = (c.d + 255) / 256;
    return mtiles * ntiles < 4 * 256 ? 2 : 1;
}

Layout layout_of(const moe_config& c) {
    Layout L;
    const size_t Tk = (size_t)c.T * (size_t)c.k;
    const size_t hbytes = c.w_dtype == MOE_DTYPE_F32 ? 4 : 2;
    size_t off = 0;
    L.partial = off;  // the router workspace
    off = round_up(off + router_layout_of(c).total, 256);
    L.offsets = off;
    off = round_up(off + sizeof(int32_t) * (size_t)(c.E + 1), 256);
    L.sorted_token = off;
    off = round_up(off + sizeof(int32_t) * Tk, 256);
    L.pos = off;
    off = round_up(off + sizeof(int32_t) * Tk, 256);
    L.H = off;
    off = round_up(off + hbytes * Tk * (size_t)c.d_ff, 256);
    L.Y = off;
    off = round_up(off + sizeof(float) * Tk * (size_t)c.d * (size_t)w2_ksplit_of(c), 256);
    L.P1 = 0;
    if (w1_ksplit_of(c) == 2) {
        L.P1 = off;
        off = round_up(off + 2 * sizeof(float) * Tk * (size_t)w1_rows(c), 256);
    }
    L.z_rows = L.prob_rows = 0;
    if (capacity_active(c)) {
        L.z_rows = off;
        off = round_up(off + sizeof(double) * (size_t)c.T * (size_t)c.E, 256);
        L.prob_rows = off;
        off = round_up(off + sizeof(double) * (size_t)c.T * (size_t)c.E, 256);
    }
    L.total = c.T == 0 ? 0 : off;
    return L;
}

// GEMM kernel for a config: 0 (F32 weights), MOE_GEMM_STREAMING or MOE_GEMM_TILED.
// (Streaming experts of at most 64 rows while tiling the rest measured slower
// than tiling all of them above 16 tokens.)
int gemm_path_of(const moe_config& c) {
    if (c.w_dtype == MOE_DTYPE_F32) return 0;
    if (c.gemm_path != MOE_GEMM_AUTO) return c.gemm_path;
    if (c.T <= kStreamingMaxT) return MOE_GEMM_STREAMING;
    if (c.w_dtype == MOE_DTYPE_INT4_G128 && !int4_tiled_ok(c)) return MOE_GEMM_STREAMING;
    return MOE_GEMM_TILED;
}

// Expert weight pointer/stride checks for an N x K matrix per expert.
moe_status check_weights(const moe_config& c, const void* W, const void* S, int64_t stride, int64_t N, int64_t K) {
    if (!W || !aligned(W, 16)) return MOE_ERR_INVALID_ARGUMENT;
    const int64_t bytes = N * K * elem_bits(c.w_dtype) / 8;
    if (stride < bytes || stride % 16 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (c.w_dtype == MOE_DTYPE_INT4_G128) {
        if (!S || !aligned(S, gemm_path_of(c) == MOE_GEMM_TILED ? 16 : 2)) return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

hipError_t run_gemm(const moe_config& c, int which, const void* A, const int32_t* a_rows, const int32_t* offsets,
                    const void* W, const void* S, int64_t stride, void* out, hipStream_t stream, int ksplit = 1) {
    moe::GemmArgs g;
    g.which = which;
    g.A = A;
    g.a_rows = a_rows;
    g.offsets = offsets;
    g.W = W;
    g.W_scales = S;
    g.W_stride = stride;
    g.out = out;
    g.T = c.T;
    g.N = which == 1 ? w1_rows(c) : c.d;
    g.K = which == 1 ? c.d : c.d_ff;
    g.E = c.E;
    g.k = c.k;
    g.w_dtype = c.w_dtype;
    g.act_dtype = c.act_dtype;
    g.path = gemm_path_of(c);
    g.act = which == 1 ? c.expert_act : 0;
    g.rows_lo = 0;
    g.rows_hi = 0x7fffffff;
    // a token adds at most one row to an expert, so no expert holds more than T rows
    g.stream_mt = c.T <= 16 ? 1 : c.T <= 32 ? 2 : 4;
    g.ksplit = ksplit;
    if (c.w_dtype == MOE_DTYPE_F32) return moe::launch_gemm_f32(g, stream);
    if (g.path == MOE_GEMM_STREAMING) return moe::launch_gemm_stream(g, stream);
    return moe::launch_gemm_tiled(g, stream);
}

// The router encoder's product W_in x as a grouped GEMM with one expert of T
// rows (which == 2: no gather, fp32 out, N = d_r, K = d).
moe_config encoder_gemm_config(const moe_config& c) {
    moe_config g;
    memset(&g, 0, sizeof g);
    g.T = c.T;
    g.d = c.router_hidden;  // GEMM2's N
    g.d_ff = c.d;           // GEMM2's K
    g.E = 1;
    g.k = 1;
    g.act_dtype = c.act_dtype;
    g.w_dtype = c.act_dtype;
    g.tau = 1.0f;
    g.gemm_path = MOE_GEMM_AUTO;
    return g;
}

// Two-layer router, first layer: h = GeLU(W_in x + b_in) into h_out (by
// default the router workspace's hidden layer).
hipError_t run_router_encoder(const moe_config& c, const void* x, const void* W_in, const float* b_in, char* rws,
                              hipStream_t stream, void* h_out = nullptr) {
    const RouterLayout R = router_layout_of(c);
    int32_t* offsets = reinterpret_cast<int32_t*>(rws + R.enc_offsets);
    float* pre = reinterpret_cast<float*>(rws + R.enc_pre);
    hipError_t e = moe::launch_encoder_offsets(offsets, c.T, stream);
    if (e != hipSuccess) return e;
    const moe_config g = encoder_gemm_config(c);
    const int64_t stride = (int64_t)c.router_hidden * c.d * (c.act_dtype == MOE_DTYPE_F32 ? 4 : 2);
    e = run_gemm(g, 2, x, nullptr, offsets, W_in, nullptr, stride, pre, stream);
    if (e != hipSuccess) return e;
    return moe::launch_encoder_act(pre, b_in, h_out ? h_out : rws + R.enc_h, c.T, c.router_hidden, c.act_dtype,
                                   stream);
}

bool encoder_args_ok(const moe_config& c, const void* W_in, const float* b_in) {
    if (c.router_hidden == 0) return W_in == nullptr && b_in == nullptr;
    return W_in && aligned(W_in, 16) && (!b_in || aligned(b_in, 4));
}

// Router arguments on the workspace `rws` (router_layout_of): with an encoder
// the router reads the hidden layer it wrote, with d = router_hidden.
moe::RouterArgs router_args(const moe_config& c, const void* x, const void* Wg, const float* bias, int32_t* ids,
                            float* gates, void* rws) {
    moe::RouterArgs r;
    const RouterLayout R = router_layout_of(c);
    r.x = c.router_hidden > 0 ? static_cast<const void*>(static_cast<char*>(rws) + R.enc_h) : x;
    r.Wg = Wg;
    r.bias = bias;
    r.T = c.T;
    r.d = c.router_hidden > 0 ? c.router_hidden : c.d;
    r.E = c.E;
    r.k = c.k;
    r.act_dtype = c.act_dtype;
    r.tau = c.tau;
    r.use_gumbel = c.use_gumbel;
    r.noise_std = c.noise_std;
    r.gate_norm = c.gate_norm;
    r.seed = c.seed;
    r.token_offset = c.token_offset;
    r.partial = reinterpret_cast<double*>(static_cast<char*>(rws) + R.partial);
    r.ids = ids;
    r.gates = gates;
    return r;
}

// The whole router: the encoder when configured, then partial logits and finalize.
hipError_t run_router(const moe_config& c, const void* x, const void* W_in, const float* b_in,
                      const moe::RouterArgs& r, char* rws, hipStream_t stream) {
    if (c.router_hidden > 0) {
        hipError_t e = run_router_encoder(c, x, W_in, b_in, rws, stream);
        if (e != hipSuccess) return e;
    }
    return moe::launch_router(r, stream);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device with that
// device current (the first no-alloc call on it).
hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    *bytes = layout_of(*cfg).total;
    return MOE_OK;
}

moe_status moe_router_workspace_size(const moe_config* cfg, size_t* bytes) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    *bytes = router_layout_of(*cfg).total;
    return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const void* x, const void* Wg, const float* router_bias,
                       const void* router_W_in, const float* router_b_in, const void* W1, const void* W1_scales, int64_t W1_expert_stride, const void* W2,
                       const void* W2_scales, int64_t W2_expert_stride, void* y, int32_t* expert_ids,
                       float* gate_weights, int32_t* counts, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (!counts || !aligned(counts, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (c.T == 0) {
        hipError_t e = moe::launch_zero_counts(counts, c.E, nullptr, stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e);
    }
    if (!x || !aligned(x, 16) || !Wg || !aligned(Wg, 16) || !y || !aligned(y, 16)) return MOE_ERR_INVALID_ARGUMENT;
    if (!expert_ids || !aligned(expert_ids, 4) || !gate_weights || !aligned(gate_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (router_bias && !aligned(router_bias, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (!encoder_args_ok(c, router_W_in, router_b_in)) return MOE_ERR_INVALID_ARGUMENT;
    if ((s = check_weights(c, W1, W1_scales, W1_expert_stride, w1_rows(c), c.d)) != MOE_OK) return s;
    if ((s = check_weights(c, W2, W2_scales, W2_expert_stride, c.d, c.d_ff)) != MOE_OK) return s;
    const Layout L = layout_of(c);
    if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

    char* ws = static_cast<char*>(workspace);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* sorted_token = reinterpret_cast<int32_t*>(ws + L.sorted_token);
    int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
    void* H = ws + L.H;
    float* Y = reinterpret_cast<float*>(ws + L.Y);

    moe::RouterArgs r = router_args(c, x, Wg, router_bias, expert_ids, gate_weights, ws + L.partial);
    const bool limited = capacity_active(c);
    if (limited) {
        r.z_rows = reinterpret_cast<double*>(ws + L.z_rows);
        r.prob_rows = reinterpret_cast<double*>(ws + L.prob_rows);
    }
    hipError_t e = run_router(c, x, router_W_in, router_b_in, r, ws + L.partial, stream);
    if (e != hipSuccess) return hip_fail(e);
    e = moe::launch_permute(expert_ids, c.T, c.E, c.k, counts, offsets, sorted_token, pos, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (limited) {
        // queue ranks come from the top-k dispatch order; the GEMMs use the dispatch of the final ids
        e = moe::launch_capacity(expert_ids, gate_weights, pos, offsets, counts, r.z_rows, r.prob_rows, c.T, c.E,
                                 c.k, (int)capacity_of(c), c.capacity_policy, stream);
        if (e != hipSuccess) return hip_fail(e);
        e = moe::launch_permute(expert_ids, c.T, c.E, c.k, counts, offsets, sorted_token, pos, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (w1_ksplit_of(c) == 2) {
        float* P = reinterpret_cast<float*>(ws + L.P1);
        const int64_t Tk = (int64_t)c.T * c.k;
        e = run_gemm(c, 1, x, sorted_token, offsets, W1, W1_scales, W1_expert_stride, P, stream, 2);
        if (e != hipSuccess) return hip_fail(e);
        e = moe::launch_act_halves(P, Tk * w1_rows(c), H, Tk, (int)w1_rows(c), (int)c.d_ff, c.expert_act, stream);
    } else {
        e = run_gemm(c, 1, x, sorted_token, offsets, W1, W1_scales, W1_expert_stride, H, stream);
    }
    if (e != hipSuccess) return hip_fail(e);
    const int ksplit = w2_ksplit_of(c);
    e = run_gemm(c, 2, H, nullptr, offsets, W2, W2_scales, W2_expert_stride, Y, stream, ksplit);
    if (e != hipSuccess) return hip_fail(e);
    const float* Y2 = ksplit == 2 ? Y + (int64_t)c.T * c.k * c.d : nullptr;
    e = moe::launch_combine(Y, pos, gate_weights, y, c.T, c.d, c.k, c.act_dtype, stream, Y2);
    if (e != hipSuccess) return hip_fail(e);
    return MOE_OK;
}

moe_status moe_forward_no_alloc(const moe_config* cfg, const void* x, const void* Wg, const float* router_bias,
                                const void* router_W_in, const float* router_b_in, const void* W1,
                                const void* W1_scales, int64_t W1_expert_stride, const void* W2,
                                const void* W2_scales, int64_t W2_expert_stride, void* y, int32_t* expert_ids,
                                float* gate_weights, int32_t* counts, hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if (layout_of(*cfg).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e);
    return moe_forward(cfg, x, Wg, router_bias, router_W_in, router_b_in, W1, W1_scales, W1_expert_stride, W2,
                       W2_scales, W2_expert_stride, y, expert_ids, gate_weights, counts, ws,
                       (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

moe_status moe_router(const moe_config* cfg, const void* x, const void* Wg, const float* router_bias,
                      const void* router_W_in, const float* router_b_in, int32_t* expert_ids, float* gate_weights,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (c.T == 0) return MOE_OK;
    if (!x || !aligned(x, 16) || !Wg || !aligned(Wg, 16)) return MOE_ERR_INVALID_ARGUMENT;
    if (!expert_ids || !aligned(expert_ids, 4) || !gate_weights || !aligned(gate_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (router_bias && !aligned(router_bias, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (!encoder_args_ok(c, router_W_in, router_b_in)) return MOE_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < router_layout_of(c).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    char* rws = static_cast<char*>(workspace);
    hipError_t e = run_router(c, x, router_W_in, router_b_in,
                              router_args(c, x, Wg, router_bias, expert_ids, gate_weights, rws), rws, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

moe_status moe_router_encoder(const moe_config* cfg, const void* x, const void* router_W_in,
                              const float* router_b_in, void* hidden, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (c.router_hidden == 0) return MOE_ERR_INVALID_ARGUMENT;
    if (c.T == 0) return MOE_OK;
    if (!x || !aligned(x, 16) || !hidden || !aligned(hidden, 16)) return MOE_ERR_INVALID_ARGUMENT;
    if (!encoder_args_ok(c, router_W_in, router_b_in)) return MOE_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    const RouterLayout R = router_layout_of(c);
    if (workspace_bytes < R.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    char* rws = static_cast<char*>(workspace);
    hipError_t e = run_router_encoder(c, x, router_W_in, router_b_in, rws, stream, hidden);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

// Router-statistics workspace: router partials, then [T][E] softmax rows,
// [T] entropies and the reduction scratch.
struct StatsLayout {
    size_t partial, prob_rows, entropy_rows, scratch, total;
};
StatsLayout stats_layout_of(const moe_config& c) {
    StatsLayout L;
    size_t off = 0;
    L.partial = off;  // the router workspace
    off = round_up(off + router_layout_of(c).total, 256);
    L.prob_rows = off;
    off = round_up(off + sizeof(double) * (size_t)c.T * (size_t)c.E, 256);
    L.entropy_rows = off;
    off = round_up(off + sizeof(double) * (size_t)c.T, 256);
    L.scratch = off;
    off = round_up(off + moe::stats_scratch_bytes(c.E), 256);
    L.total = c.T == 0 ? 0 : off;
    return L;
}

moe_status moe_router_stats_workspace_size(const moe_config* cfg, size_t* bytes) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    *bytes = stats_layout_of(*cfg).total;
    return MOE_OK;
}

moe_status moe_router_stats(const moe_config* cfg, const void* x, const void* Wg, const float* router_bias,
                            const void* router_W_in, const float* router_b_in, int32_t* expert_ids, float* gate_weights, double* expert_fraction, double* mean_prob,
                            double* scalars, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (!expert_fraction || !aligned(expert_fraction, 8) || !mean_prob || !aligned(mean_prob, 8) || !scalars ||
        !aligned(scalars, 8))
        return MOE_ERR_INVALID_ARGUMENT;
    if (c.T == 0) {
        hipError_t e = moe::launch_zero_stats(c.E, expert_fraction, mean_prob, scalars, stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e);
    }
    if (!x || !aligned(x, 16) || !Wg || !aligned(Wg, 16)) return MOE_ERR_INVALID_ARGUMENT;
    if (!expert_ids || !aligned(expert_ids, 4) || !gate_weights || !aligned(gate_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (router_bias && !aligned(router_bias, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (!encoder_args_ok(c, router_W_in, router_b_in)) return MOE_ERR_INVALID_ARGUMENT;
    const StatsLayout L = stats_layout_of(c);
    if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    char* ws = static_cast<char*>(workspace);
    moe::RouterArgs r = router_args(c, x, Wg, router_bias, expert_ids, gate_weights, ws + L.partial);
    r.prob_rows = reinterpret_cast<double*>(ws + L.prob_rows);
    r.entropy_rows = reinterpret_cast<double*>(ws + L.entropy_rows);
    hipError_t e = run_router(c, x, router_W_in, router_b_in, r, ws + L.partial, stream);
    if (e != hipSuccess) return hip_fail(e);
    e = moe::launch_router_stats(r.prob_rows, r.entropy_rows, expert_ids, c.T, c.E, c.k, ws + L.scratch,
                                 expert_fraction, mean_prob, scalars, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

moe_status moe_permute(const moe_config* cfg, const int32_t* expert_ids, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_token, int32_t* pos, hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (!counts || !aligned(counts, 4) || !offsets || !aligned(offsets, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (c.T > 0) {
        if (!expert_ids || !aligned(expert_ids, 4) || !sorted_token || !aligned(sorted_token, 4) || !pos ||
            !aligned(pos, 4))
            return MOE_ERR_INVALID_ARGUMENT;
    }
    hipError_t e = moe::launch_permute(expert_ids, c.T, c.E, c.k, counts, offsets, sorted_token, pos, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

moe_status moe_grouped_gemm(const moe_config* cfg, int32_t which, const void* A, const int32_t* a_rows,
                            const int32_t* offsets, const void* W, const void* W_scales, int64_t W_expert_stride,
                            void* out, hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (which != 1 && which != 2) return MOE_ERR_INVALID_ARGUMENT;
    if (c.T == 0) return MOE_OK;
    if (!A || !aligned(A, 16) || !offsets || !aligned(offsets, 4) || !out || !aligned(out, 16))
        return MOE_ERR_INVALID_ARGUMENT;
    if (which == 1 && (!a_rows || !aligned(a_rows, 4))) return MOE_ERR_INVALID_ARGUMENT;
    const int64_t N = which == 1 ? w1_rows(c) : c.d;
    const int64_t K = which == 1 ? c.d : c.d_ff;
    if ((s = check_weights(c, W, W_scales, W_expert_stride, N, K)) != MOE_OK) return s;
    hipError_t e = run_gemm(c, which, A, a_rows, offsets, W, W_scales, W_expert_stride, out, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

moe_status moe_combine(const moe_config* cfg, const float* Y, const int32_t* pos, const float* gate_weights, void* y,
                       hipStream_t stream) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    const moe_config& c = *cfg;
    if (c.T == 0) return MOE_OK;
    if (!Y || !aligned(Y, 16) || !pos || !aligned(pos, 4) || !gate_weights || !aligned(gate_weights, 4) || !y ||
        !aligned(y, 16))
        return MOE_ERR_INVALID_ARGUMENT;
    hipError_t e = moe::launch_combine(Y, pos, gate_weights, y, c.T, c.d, c.k, c.act_dtype, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
