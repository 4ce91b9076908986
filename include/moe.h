/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer (sources: five web pages on sparse MoE layers; P1..P5 below):
 *   P1 devpress.csdn.net/awstech/6a46250010ee7a33f285d330  ("动态稀疏激活"的工程革命)
 *   P2 devpress.csdn.net/awstech/6a919c0d2b83d06f0ec6f601  (参数规模与稀疏激活的真相拆解)
 *   P3 devpress.csdn.net/awstech/6a46202710ee7a33f285c5a4  (参数规模与稀疏激活的真相拆解, 2nd article)
 *   P4 hotelren.com/news/2927663                            (gating kernel and vLLM patch)
 *   P5 aicoding.csdn.net/6a320eef10ee7a33f27e52b3           (这句话到底在说什么？)
 *
 *   logits  l = x . Wg (+ b)                    P2 §2.2 (single linear router), P5 §3.2
 *   z       = (l + g) / tau, g Gumbel or 0      P1 §3.1 (Gumbel noise, temperature)
 *   ids     = top-k of z, gates = softmax(z)[ids]  (not renormalised)   P2 §2.2, P5 §3.1
 *   y[t]    = sum_j gates[t,j] * W2_e GeLU(W1_e x[t]),  e = ids[t,j]   P3 §3.2 (d->4d->d GELU MLP)
 *   INT4 experts: w = q * s, q in [-8,7], one bf16 scale per 128 inputs   P1 §5.4, P2 §2.3
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device, owned by the caller, 16-byte aligned, and must not alias an
 *    output.  The library allocates nothing and keeps no state besides a
 *    thread-local copy of the last HIP error code, and, for
 *    moe_forward_no_alloc only, one static device scratch array per GPU and
 *    its address per device.
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call returns
 *    without waiting; outputs are valid once the stream has been synchronised.
 *    Nothing is copied between host and device inside a call.
 *  - Arguments are checked before anything is enqueued: a rejected call
 *    returns an error code and enqueues nothing.  A failed launch returns
 *    MOE_ERR_HIP (moe_last_hip_error() holds hipError_t).  Nothing is printed
 *    and no C++ exception crosses the ABI.  NaN or Inf in the data is not an
 *    error: a NaN logit ranks below every number (the token still gets k
 *    distinct experts) and NaN propagates into y.
 *  - Calls that share a workspace must be ordered on one stream.
 *  - Layouts are row-major.  Weights are [E][N][K] (output rows, input
 *    columns contiguous): W1 is [E][d_ff][d], W2 is [E][d][d_ff].  INT4
 *    codes pack two signed two's-complement nibbles per byte, even column in
 *    the low nibble ([E][N][K/2] bytes); their scales are bf16 [E][N][K/128].
 *  - Sizes: 0 <= T <= 2^24, 1 <= E <= 256, 1 <= k <= min(E, 8), d and d_ff
 *    multiples of 64 (of 128 for INT4 experts), d, d_ff <= 2^17.  Every
 *    activation array (x, y, and the workspace's [T*k][d_ff] and
 *    [T*k][d] float intermediates) and each expert's matrix must stay below
 *    4 GiB (larger batches are split by the caller); otherwise
 *    MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,  /* null/misaligned pointer, size out of range, bad tau ... */
    MOE_ERR_UNSUPPORTED = 2,       /* valid but not implemented (e.g. an odd dtype pairing) */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                /* a HIP launch failed; see moe_last_hip_error() */
} moe_status;

/* Storage types.  Activations (x, Wg, y) are F32 or BF16; expert weights are
 * F32 (with F32 activations), BF16 or INT4_G128 (with BF16 activations). */
typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,
    MOE_DTYPE_BF16 = 1,
    MOE_DTYPE_INT4_G128 = 2
} moe_dtype;

/* Expert-GEMM implementation choice. */
typedef enum moe_gemm_path {
    MOE_GEMM_AUTO = 0,       /* streaming when T <= 16 (or INT4 weights that the tiled kernel
                                cannot take), tiled otherwise */
    MOE_GEMM_STREAMING = 1,  /* weight-streaming kernel: every weight read once per 16 rows of an
                                expert (T <= 16), 32 rows (T <= 32) or 64 rows */
    MOE_GEMM_TILED = 2       /* LDS-tiled MFMA kernel for many tokens per expert; INT4 weights need d and
                                d_ff multiples of 1024 (else MOE_ERR_UNSUPPORTED) and 16-byte aligned scales */
} moe_gemm_path;

typedef struct moe_config {
    int64_t T;             /* tokens */
    int64_t d;             /* model width */
    int64_t d_ff;          /* expert hidden width */
    int32_t E;             /* experts */
    int32_t k;             /* experts per token */
    int32_t act_dtype;     /* moe_dtype of x, Wg and y */
    int32_t w_dtype;       /* moe_dtype of W1 and W2 */
    float tau;             /* temperature: z = (l + g) / tau; finite and > 0 */
    int32_t use_gumbel;    /* 0: g = 0;  1: g = -ln(-ln u) per (seed, token_offset + t, e) */
    uint64_t seed;
    uint64_t token_offset; /* absolute index of token 0, so successive calls draw fresh noise */
    int32_t gemm_path;     /* moe_gemm_path */
    int32_t reserved;      /* must be 0 */
    float capacity_factor; /* 0: dropless (every token gets k experts); > 0 (finite): expert capacity
                              cap = ceil(T k / E * capacity_factor) in binary64 (P5 §3.2; P2 §3.2),
                              which only moe_forward applies; a cap >= T changes nothing */
    int32_t capacity_policy; /* moe_capacity_policy (must be valid even when capacity_factor == 0) */
    int32_t gate_norm;     /* 0: gate = softmax over all E experts at the chosen ids (not renormalised);
                              1: softmax over the k chosen z only (P4 §4.3); not combinable with a capacity */
    float noise_std;       /* sigma >= 0 (finite) of Gaussian router noise (P5 §3.3): z = (l + g + sigma n) / tau,
                              n standard normal by Box-Muller from words 2 and 3 of the (seed, token, expert)
                              Philox block; 0: none */
    int32_t expert_act;    /* moe_expert_act */
    int32_t router_hidden; /* 0: single linear router (l = Wg^T x + b).  d_r > 0 (multiple of 64): two-layer
                              router (P3 §3.1, §4.2; d/4 there): h = GeLU(W_in x + b_in), W_in [d_r][d] and h in
                              act_dtype (h rounded to nearest even), then l = Wg^T h + b with Wg [d_r][E] */
} moe_config;

/* The experts' hidden activation (P3 §3.2 GELU; P1 §3.3 and §4.2 SiLU-gated units). */
typedef enum moe_expert_act {
    MOE_ACT_GELU = 0,   /* o = W2 GeLU(W1 x), GeLU(h) = h Phi(h); W1 has d_ff rows */
    MOE_ACT_SILU = 1,   /* o = W2 SiLU(W1 x), SiLU(a) = a / (1 + e^-a); W1 has d_ff rows */
    MOE_ACT_SWIGLU = 2  /* o = W2 (SiLU(G x) * U x): W1 has 2 d_ff rows interleaved in blocks of 16, rows
                           32 b .. 32 b + 15 the gate rows of hidden units 16 b .. 16 b + 15 and the next 16 rows
                           their up rows (INT4 scales follow the same rows) */
} moe_expert_act;

/* What happens to an assignment whose expert is full (P5 §3.2; P2 §3.2).  The
 * T k assignments queue in row-major (token, slot) order; each keeps its
 * expert while that expert holds fewer than cap.  DROP: an overflowing
 * assignment is dropped.  REROUTE: then, in the same order, each overflowing
 * assignment moves to the best-ranked expert (larger z first, NaN last, ties
 * to the lower index) that its token does not already use and that holds
 * fewer than cap; with none left it is dropped.  A dropped assignment has
 * expert id -1 and gate 0 and adds nothing to y; gates are never renormalised. */
typedef enum moe_capacity_policy {
    MOE_CAPACITY_DROP = 0,
    MOE_CAPACITY_REROUTE = 1
} moe_capacity_policy;

/* Bytes of device workspace moe_forward needs for `cfg` (0 when T == 0); capacity-limited
 * dispatch adds the [T][E] logit and probability rows, and a bf16 tiled GEMM2 run in two
 * K halves (small tile grids) a second [T*k][d] float intermediate. */
moe_status moe_workspace_size(const moe_config *cfg, size_t *bytes);

/* Bytes of device workspace moe_router needs for `cfg`. */
moe_status moe_router_workspace_size(const moe_config *cfg, size_t *bytes);

/*
 * The whole layer (P2 §2.2 steps 1-4; P1 §3.1; P3 §3.2).
 *   x            [T][d]   act_dtype                      (device, in)
 *   Wg           [d][E]   act_dtype ([router_hidden][E] with a router encoder)    (device, in)
 *   router_bias  [E]      float, or NULL for none        (device, in)
 *   router_W_in  [router_hidden][d] act_dtype, router_b_in [router_hidden] float or NULL: the encoder
 *                layer when router_hidden > 0; both NULL otherwise            (device, in)
 *   W1, W2       expert 0's matrix ([d_ff][d], or [2 d_ff][d] for SwiGLU; [d][d_ff]); expert e starts
 *                e * W*_expert_stride bytes later
 *                (stride >= the matrix's bytes, multiple of 16)   (device, in)
 *   W1_scales, W2_scales  bf16 [E][N][K/128] for INT4 weights, NULL otherwise (device, in)
 *   y            [T][d]   act_dtype                      (device, out)
 *   expert_ids   [T][k]   int32, best first              (device, out)
 *   gate_weights [T][k]   float, softmax(z)[ids]         (device, out)
 *   counts       [E]      int32, tokens routed per expert (sum = T*k)  (device, out)
 *   workspace    >= moe_workspace_size() bytes, 256-byte aligned       (device, scratch)
 * With a capacity (capacity_factor > 0) expert_ids and gate_weights hold the
 * dispatched routing: a rerouted slot names its new expert (no longer in z
 * order), a dropped slot has id -1 and gate 0, and counts sum to the
 * assignments kept.
 * T == 0 is a valid no-op that writes counts = 0.
 */
moe_status moe_forward(const moe_config *cfg, const void *x, const void *Wg, const float *router_bias,
                       const void *router_W_in, const float *router_b_in, const void *W1, const void *W1_scales, int64_t W1_expert_stride,
                       const void *W2, const void *W2_scales, int64_t W2_expert_stride,
                       void *y, int32_t *expert_ids, float *gate_weights, int32_t *counts,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer, arguments and outputs, but no workspace argument.  The workspace
 * is the library's own static device array of MOE_STATIC_SCRATCH_BYTES, one
 * per GPU, held from the library's load on that GPU until the process ends;
 * its address is looked up once per device on the first call there (with that
 * device current).  Nothing is allocated or freed.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (no kernel relies on
 * them being zero): calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race on it and must be serialised
 * by the caller.  A configuration whose moe_workspace_size() exceeds
 * MOE_STATIC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE_TOO_SMALL with nothing
 * enqueued; other errors as moe_forward.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)
moe_status moe_forward_no_alloc(const moe_config *cfg, const void *x, const void *Wg, const float *router_bias,
                                const void *router_W_in, const float *router_b_in, const void *W1,
                                const void *W1_scales, int64_t W1_expert_stride, const void *W2,
                                const void *W2_scales, int64_t W2_expert_stride, void *y, int32_t *expert_ids,
                                float *gate_weights, int32_t *counts, hipStream_t stream);

/*
 * Router stage (P2 §2.2 steps 1-3; P1 §3.1; P5 §3.2): logits accumulated in
 * binary64 from exact products, optional counter-based Gumbel noise
 * (Philox4x64-10, key (seed, 0), counter (token_offset + t, e, 0, 0),
 * u = (top 53 bits of word 0 + 1/2) * 2^-53), temperature, top-k by z
 * (ties to the lower expert index), softmax in binary64.
 * With router_hidden > 0 the logits come from the encoder's hidden layer
 * (moe_router_encoder) instead of x.
 *   expert_ids [T][k] int32, gate_weights [T][k] float   (device, out)
 *   workspace  >= moe_router_workspace_size() bytes        (device, scratch)
 */
moe_status moe_router(const moe_config *cfg, const void *x, const void *Wg, const float *router_bias,
                      const void *router_W_in, const float *router_b_in, int32_t *expert_ids, float *gate_weights,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Router encoder stage (P3 §3.1 input encoder, §4.2 GeLU between the router's
 * two linear layers), for cfg->router_hidden = d_r > 0:
 *   hidden[t][j] = GeLU( sum_i W_in[j][i] x[t][i] + b_in[j] ),  j < d_r,
 * accumulated in fp32 (MFMA for bf16), GeLU h * erfc(-h / sqrt 2) / 2 in fp32,
 * stored in act_dtype (bf16: round to nearest even).
 *   x [T][d], router_W_in [d_r][d] act_dtype; router_b_in [d_r] float or NULL (device, in)
 *   hidden [T][d_r] act_dtype, 16-byte aligned                                (device, out)
 *   workspace >= moe_router_workspace_size() bytes, 256-byte aligned          (device, scratch)
 * MOE_ERR_INVALID_ARGUMENT when router_hidden == 0.
 */
moe_status moe_router_encoder(const moe_config *cfg, const void *x, const void *router_W_in,
                              const float *router_b_in, void *hidden, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Router statistics (P1 §3.2 router entropy; P3 §4.2 expert_load, the mean
 * selection probability; P5 §3.2 balance loss over assignment fractions; P3
 * §3.2 the same sum over probabilities; P5 §4 spread of expert utilisation).
 * Routes exactly as moe_router (same expert_ids and gate_weights), then, in
 * binary64 and in a fixed summation order:
 *   expert_fraction[e] = #{(t, j): expert_ids[t][j] = e} / (T k)      [E]
 *   mean_prob[e]       = (1/T) sum_t softmax(z_t)[e]                    [E]
 *   scalars[0] = (1/T) sum_t -sum_e p ln p  (router entropy, nats; 0 ln 0 = 0)
 *   scalars[1] = sum_e (expert_fraction[e] - 1/E)^2
 *   scalars[2] = sum_e (mean_prob[e] - 1/E)^2
 *   scalars[3] = sqrt(scalars[1] / E)   (standard deviation of expert_fraction)
 *   scalars[4] = E sum_e expert_fraction[e] * mean_prob[e]   (product form of the
 *                balance term; 1 when both are uniform)
 * All outputs are device pointers (double arrays 8-byte aligned).  T == 0
 * writes zeros.  workspace >= moe_router_stats_workspace_size() bytes,
 * 256-byte aligned (it holds the T x E softmax rows).
 */
moe_status moe_router_stats_workspace_size(const moe_config *cfg, size_t *bytes);
moe_status moe_router_stats(const moe_config *cfg, const void *x, const void *Wg, const float *router_bias,
                            const void *router_W_in, const float *router_b_in, int32_t *expert_ids, float *gate_weights, double *expert_fraction, double *mean_prob,
                            double *scalars, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dispatch stage (P3 §4.2: per-expert load vector; tokens scattered to
 * experts): counts[e], exclusive offsets[E+1] (offsets[E] = T*k), and the
 * stable expert-major order of the T*k assignments taken in row-major
 * (token, slot) order: sorted_token[offsets[e] + r] is the token of the r-th
 * assignment to e, pos[t][j] is the position of assignment (t, j).
 * Bit-exact and deterministic.  An id outside [0, E) (a dropped slot, -1)
 * is left out: its pos is -1 and offsets[E] counts only the others.
 *   expert_ids [T][k] (device, in); counts [E], offsets [E+1],
 *   sorted_token [T*k], pos [T][k]: int32 (device, out)
 */
moe_status moe_permute(const moe_config *cfg, const int32_t *expert_ids, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_token, int32_t *pos, hipStream_t stream);

/*
 * One grouped expert GEMM over the dispatch order (P3 §3.2; P2 §2.3; P2 §3.3
 * fused activation).  For each expert e and each position s in
 * [offsets[e], offsets[e+1]):
 *   which == 1:  out[s][n] = act( sum_c W1_e[n][c] * A[row(s)][c] ),  n < d_ff, act per
 *                expert_act (SwiGLU: SiLU of the unit's gate row times its up row, W1_e of 2 d_ff rows),
 *                row(s) = a_rows[s] (A = x, [T][d]); out = H, [T*k][d_ff],
 *                bf16 for BF16/INT4 weights, float for F32 weights.
 *   which == 2:  out[s][c] = sum_n W2_e[c][n] * A[s][n],  c < d;
 *                A = H as written by which == 1 (a_rows ignored); out = Y,
 *                float [T*k][d].
 * GeLU(h) = h * Phi(h) (erf form).  Accumulation is fp32 (MFMA for BF16/INT4
 * weights).  INT4 weights are applied as exact q * s by the streaming kernel;
 * the tiled kernel multiplies by q * s rounded to bf16 (nearest even; relative
 * error at most 2^-8 per weight).
 *   offsets [E+1] int32 (device, in), as written by moe_permute.
 */
moe_status moe_grouped_gemm(const moe_config *cfg, int32_t which, const void *A, const int32_t *a_rows,
                            const int32_t *offsets, const void *W, const void *W_scales,
                            int64_t W_expert_stride, void *out, hipStream_t stream);

/*
 * Combine stage (P2 §2.2 step 4; P5 §3.2): y[t][c] = sum_{j<k} gate_weights[t][j] * Y[pos[t][j]][c],
 * summed in ascending j in fp32 over the slots with pos >= 0, stored in
 * act_dtype (round to nearest even).
 *   Y [T*k][d] float, pos [T][k] int32, gate_weights [T][k] float (device, in);
 *   y [T][d] act_dtype (device, out)
 */
moe_status moe_combine(const moe_config *cfg, const float *Y, const int32_t *pos, const float *gate_weights,
                       void *y, hipStream_t stream);

/* Static description of a status code. */
const char *moe_status_string(moe_status status);

/* hipError_t of the last failed HIP call made by this library on this thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
