/*
 * moe_oracle.c -- plain, slow, single-threaded fp64 CPU oracle for the forward
 * pass of one sparse Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The GPU product
 * path never links, loads or falls back to it, and this file shares no code,
 * header, table or constant generator with the HIP kernels.
 *
 * Sources (the five web pages that define the method; cited by page and section):
 *   P1  "这不是参数堆砌，而是动态稀疏激活的工程革命"
 *       devpress.csdn.net/awstech/6a46250010ee7a33f285d330
 *   P2  "项目概述：参数规模与稀疏激活的真相拆解"
 *       devpress.csdn.net/awstech/6a919c0d2b83d06f0ec6f601
 *   P3  "项目概述：参数规模与稀疏激活的真相拆解" (second article, same heading)
 *       devpress.csdn.net/awstech/6a46202710ee7a33f285c5a4
 *   P4  hotelren.com/news/2927663 (MoE gating article under an unrelated headline)
 *   P5  "这句话到底在说什么？" aicoding.csdn.net/6a320eef10ee7a33f27e52b3
 *
 * What is computed, per token t (all arithmetic in IEEE binary64):
 *   1. logits  l[e] = sum_i x[t,i] * Wg[i,e]  (+ b[e])        P2 §2.2 steps 1-2; P5 §3.2 "处理"
 *      Wg is d x E row-major (P5 §3.2 gives W_router as a d x 128 matrix).
 *      The sum runs over ascending i.  bf16 and fp32 inputs widen exactly and
 *      their pairwise products are exact in binary64.
 *   2. noise   g[e] = -ln(-ln u),  u in (0,1) from Philox4x64-10   P1 §3.1 steps 2-3
 *      (counter-based generator of Salmon et al., SC'11, keyed on
 *      (seed, token, expert); g = 0 when noise is off)
 *   3. z[e] = (l[e] + g[e]) / tau                                   P1 §3.1 step 3
 *   4. ids  = the k experts with the largest z, ordered by z descending;
 *      exact ties go to the lower expert index; NaN ranks below every number.
 *      Selecting on z equals selecting on softmax(z) (softmax is monotone). P1 §3.1 step 4; P2 §2.2 step 3
 *   5. p = softmax(z) over all E, max-subtracted; gate[j] = p[ids[j]] (not
 *      renormalised over the k chosen).                              P2 §2.2 step 4; P5 §3.1 worked example
 *   Variants (oracle_route_ex, oracle_router_encoder):
 *   1'. two-layer router: a hidden layer h = GeLU(W_in x + b_in) of width
 *      d_r (d/4 in the pages), stored in the activation dtype (rounded to
 *      nearest even), then the linear router of step 1 on h.           P3 §3.1 (input encoder), §4.2
 *   2'. Gaussian noise sigma * n[e] added to the logits, n standard normal by
 *      Box-Muller from the same Philox block: z = (l + g + sigma n) / tau   P5 §3.3 (router noise injection)
 *   5'. renormalised gates: gate[j] = softmax over the k chosen z values
 *      (= p[ids[j]] / sum_j' p[ids[j']])                                   P4 §4.3 (softmax over the top-k)
 *   6. expert FFN  o = W2_e * GeLU(W1_e * x),  GeLU(h) = h * Phi(h)
 *                  = 0.5 h erfc(-h / sqrt 2), no bias.           P3 §3.2 (d -> 4d -> d MLP, GELU)
 *      W1_e is d_ff x d, W2_e is d x d_ff (out x in, input dim contiguous).
 *      INT4 experts: w[n,c] = q[n,c] * s[n, c/128] exactly, q in [-8,7]
 *      (symmetric group-128 codes with bf16 scales).                 P1 §5.4; P2 §2.3 (dequantize step)
 *   6'. expert activations (expert_act): 1 = SiLU, o = W2_e * SiLU(W1_e * x)
 *      with SiLU(a) = a / (1 + e^-a); 2 = SwiGLU, o = W2_e * (SiLU(G x) * (U x))
 *      where W1_e holds 2 d_ff rows: the gate row of hidden unit n is
 *      32 (n / 16) + n % 16 and its up row is 16 rows further.        P1 §3.3, §4.2 (SwiGLU experts)
 *   7. y[t] = sum_j p[ids[j]] * o_{ids[j]}                           P2 §2.2 step 4; P5 §3.2 "合并"
 * Dispatch bookkeeping (per-expert counts, exclusive offsets, a stable
 * counting sort of the (token, slot) assignments) follows P3 §4.2's per-expert
 * load vector and its note that tokens are scattered to experts.
 *
 * Nothing is blocked, fused or reordered beyond the definitions above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_INT4_G128 2

/* ---------------------------------------------------------------- decoding */

/* binary64 -> bf16 bits, rounded to nearest even in one step.  The value is
 * first rounded to binary32 (nearest even); when that lands exactly on a bf16
 * midpoint, the binary64 value decides the direction (above or below the
 * midpoint in magnitude; an exact midpoint goes to the even neighbour). */
static uint16_t double_to_bf16_bits(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
    uint32_t hi = u >> 16, low = u & 0xffffu;
    int up;
    if (low != 0x8000u)
        up = low > 0x8000u;
    else if (fabs(v) != fabs((double)f))
        up = fabs(v) > fabs((double)f);
    else
        up = (int)(hi & 1u);
    return (uint16_t)(hi + (uint32_t)up);
}

static double bf16_to_double(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Element idx of an activation-typed array (x, Wg). */
static double load_act(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    return bf16_to_double(((const uint16_t *)base)[idx]);
}

/* One signed 4-bit code: two's complement nibble, even column in the low nibble. */
static int int4_code(const uint8_t *codes, int64_t K, int64_t n, int64_t c)
{
    uint8_t byte = codes[n * (K / 2) + c / 2];
    int nib = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

/* Weight element [n][c] of one expert's N x K matrix. */
static double load_w(const void *w, const void *scales, int32_t dtype, int64_t K, int64_t n, int64_t c)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)w)[n * K + c];
    if (dtype == ORACLE_BF16)
        return bf16_to_double(((const uint16_t *)w)[n * K + c]);
    {
        int q = int4_code((const uint8_t *)w, K, n, c);
        double s = bf16_to_double(((const uint16_t *)scales)[n * (K / 128) + c / 128]);
        return (double)q * s;
    }
}

/* ------------------------------------------------------ Philox4x64-10 (SC'11) */

/* One Philox4x64 block with 10 rounds.  Round function: two 64x64->128
 * multiplies of words 0 and 2, outputs (hi1^x1^k0, lo1, hi0^x3^k1, lo0); the
 * key is bumped by the two Weyl constants between rounds. */
void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        unsigned __int128 p0 = (unsigned __int128)M0 * x0;
        unsigned __int128 p1 = (unsigned __int128)M1 * x2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        k0 += W0;
        k1 += W1;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Uniform u strictly inside (0,1) for (seed, token, expert): the top 53 bits of
 * the block's first word, offset by half an ulp. */
double oracle_uniform(uint64_t seed, uint64_t token, uint64_t expert)
{
    uint64_t ctr[4] = {token, expert, 0, 0}, key[2] = {seed, 0}, r[4];
    oracle_philox4x64_10(ctr, key, r);
    return ((double)(r[0] >> 11) + 0.5) * (1.0 / 9007199254740992.0); /* 2^-53 */
}

/* Standard Gumbel draw g = -ln(-ln u)   (P1 §3.1 step 2). */
double oracle_gumbel(uint64_t seed, uint64_t token, uint64_t expert)
{
    double u = oracle_uniform(seed, token, expert);
    return -log(-log(u));
}

/* Standard normal draw for (seed, token, expert): the Box-Muller transform
 * (Box & Muller, 1958) sqrt(-2 ln u1) cos(2 pi u2) of two uniforms built like
 * oracle_uniform from words 2 and 3 of the same Philox block (word 0 feeds
 * the Gumbel draw).   P5 §3.3 (Gaussian noise on the router logits). */
double oracle_normal(uint64_t seed, uint64_t token, uint64_t expert)
{
    uint64_t ctr[4] = {token, expert, 0, 0}, key[2] = {seed, 0}, r[4];
    oracle_philox4x64_10(ctr, key, r);
    const double two_pi = 6.283185307179586; /* 2 pi rounded to binary64 */
    double u1 = ((double)(r[2] >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    double u2 = ((double)(r[3] >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* SiLU (swish with beta = 1): a * sigmoid(a) = a / (1 + e^-a). */
double oracle_silu(double a)
{
    return a / (1.0 + exp(-a));
}

/* GeLU in its exact form h * Phi(h), with Phi(h) = erfc(-h / sqrt 2) / 2
 * (no cancellation in the negative tail, where 1 + erf(h / sqrt 2) rounds to 0). */
double oracle_gelu(double h)
{
    return 0.5 * h * erfc(-h / sqrt(2.0));
}

/* ------------------------------------------------------------------ routing */

/* Is expert a ranked before expert b?  Larger z first, NaN last, ties to the
 * lower index. */
static int ranks_before(const double *z, int32_t a, int32_t b)
{
    int na = isnan(z[a]), nb = isnan(z[b]);
    if (na != nb)
        return nb; /* the non-NaN one wins */
    if (!na && z[a] != z[b])
        return z[a] > z[b];
    return a < b;
}

/*
 * Router for all T tokens.  Writes ids[T][k] (best first), gates[T][k] =
 * (float) gate, and optionally gate_p[T][k] (the same gates in binary64),
 * z_out[T][E] and p_out[T][E] (the full softmax rows).  bias may be NULL.
 * noise_std: sigma of the Gaussian logit noise (0: none).  gate_norm: 0 gives
 * gate = p[id]; 1 gives the softmax over the k chosen z, max-subtracted at the
 * best one and summed in slot order.  Returns 0, or -1 on a bad argument.
 */
int oracle_route_ex(int64_t T, int64_t d, int32_t E, int32_t k, int32_t act_dtype,
                    const void *x, const void *Wg, const float *bias,
                    double tau, int32_t use_gumbel, double noise_std, int32_t gate_norm,
                    uint64_t seed, uint64_t token_offset,
                    int32_t *ids, float *gates, double *gate_p, double *z_out, double *p_out)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || !(tau > 0.0))
        return -1;
    if (!(noise_std >= 0.0) || (gate_norm != 0 && gate_norm != 1))
        return -1;
    if (act_dtype != ORACLE_F32 && act_dtype != ORACLE_BF16)
        return -1;
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    double *z = (double *)malloc(sizeof(double) * (size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *taken = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!l || !z || !p || !taken) {
        free(l); free(z); free(p); free(taken);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        /* 1. logits: each l[e] accumulates over ascending i. */
        for (int32_t e = 0; e < E; ++e)
            l[e] = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double xi = load_act(x, act_dtype, t * d + i);
            for (int32_t e = 0; e < E; ++e)
                l[e] += xi * load_act(Wg, act_dtype, i * (int64_t)E + e);
        }
        if (bias)
            for (int32_t e = 0; e < E; ++e)
                l[e] += (double)bias[e];
        /* 2-3. noise and temperature. */
        for (int32_t e = 0; e < E; ++e) {
            double g = use_gumbel ? oracle_gumbel(seed, token_offset + (uint64_t)t, (uint64_t)e) : 0.0;
            double v = l[e] + g;
            if (noise_std > 0.0)
                v += noise_std * oracle_normal(seed, token_offset + (uint64_t)t, (uint64_t)e);
            z[e] = v / tau;
        }
        /* 5. softmax over all experts. */
        double m = z[0];
        for (int32_t e = 1; e < E; ++e)
            if (z[e] > m)
                m = z[e];
        double s = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            p[e] = exp(z[e] - m);
            s += p[e];
        }
        for (int32_t e = 0; e < E; ++e)
            p[e] /= s;
        /* 4. top-k by repeated selection of the best expert not yet taken. */
        for (int32_t e = 0; e < E; ++e)
            taken[e] = 0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(z, e, best)))
                    best = e;
            taken[best] = 1;
            ids[t * k + j] = best;
            gates[t * k + j] = (float)p[best];
            if (gate_p)
                gate_p[t * k + j] = p[best];
        }
        if (gate_norm) {
            /* 5'. softmax over the chosen z (z[ids[0]] is their maximum) */
            double top = z[ids[t * k]], den = 0.0;
            for (int32_t j = 0; j < k; ++j)
                den += exp(z[ids[t * k + j]] - top);
            for (int32_t j = 0; j < k; ++j) {
                double gj = exp(z[ids[t * k + j]] - top) / den;
                gates[t * k + j] = (float)gj;
                if (gate_p)
                    gate_p[t * k + j] = gj;
            }
        }
        if (z_out)
            memcpy(z_out + t * E, z, sizeof(double) * (size_t)E);
        if (p_out)
            memcpy(p_out + t * E, p, sizeof(double) * (size_t)E);
    }
    free(l); free(z); free(p); free(taken);
    return 0;
}

/*
 * Hidden layer of the two-layer router (step 1'): for every token t and hidden
 * unit j < d_r, r = sum_i x[t,i] W_in[j,i] (ascending i) + b_in[j], and
 * h[t][j] = GeLU(r) stored in act_dtype (float, or bf16 bits rounded to
 * nearest even from the binary64 value).  W_in is d_r x d (out x in), in
 * act_dtype; b_in (float) may be NULL.  Returns 0, or -1 on a bad argument.
 */
int oracle_router_encoder(int64_t T, int64_t d, int64_t d_r, int32_t act_dtype, const void *x,
                          const void *W_in, const float *b_in, void *h_out)
{
    if (T < 0 || d < 1 || d_r < 1 || (act_dtype != ORACLE_F32 && act_dtype != ORACLE_BF16))
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < d_r; ++j) {
            double r = 0.0;
            for (int64_t i = 0; i < d; ++i)
                r += load_act(x, act_dtype, t * d + i) * load_act(W_in, act_dtype, j * d + i);
            if (b_in)
                r += (double)b_in[j];
            double a = oracle_gelu(r);
            if (act_dtype == ORACLE_F32)
                ((float *)h_out)[t * d_r + j] = (float)a;
            else
                ((uint16_t *)h_out)[t * d_r + j] = double_to_bf16_bits(a);
        }
    return 0;
}

/* The router of steps 1-5 (no Gaussian noise, gates not renormalised). */
int oracle_route(int64_t T, int64_t d, int32_t E, int32_t k, int32_t act_dtype,
                 const void *x, const void *Wg, const float *bias,
                 double tau, int32_t use_gumbel, uint64_t seed, uint64_t token_offset,
                 int32_t *ids, float *gates, double *gate_p, double *z_out, double *p_out)
{
    return oracle_route_ex(T, d, E, k, act_dtype, x, Wg, bias, tau, use_gumbel, 0.0, 0, seed, token_offset,
                           ids, gates, gate_p, z_out, p_out);
}

/* ----------------------------------------------------------------- dispatch */

/*
 * Per-expert counts, exclusive offsets[E+1], and the stable counting sort of
 * the T*k assignments taken in row-major (token, slot) order:
 *   sorted_token[offsets[e] + r] = token of the r-th assignment to e,
 *   pos[t*k + j] = the position of assignment (t, j) in that order.
 * An id of -1 marks an assignment dropped by capacity-limited dispatch: it
 * is not counted and gets pos = -1.  Returns 0, or -1 if an id is otherwise
 * out of range.
 */
int oracle_permute(int64_t T, int32_t E, int32_t k, const int32_t *ids,
                   int32_t *counts, int32_t *offsets, int32_t *sorted_token, int32_t *pos)
{
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < T * k; ++a) {
        if (ids[a] == -1)
            continue;
        if (ids[a] < 0 || ids[a] >= E)
            return -1;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            if (e == -1) {
                pos[t * k + j] = -1;
                continue;
            }
            int32_t slot = offsets[e] + fill[e];
            fill[e] += 1;
            sorted_token[slot] = (int32_t)t;
            pos[t * k + j] = slot;
        }
    free(fill);
    return 0;
}

/* ------------------------------------------------ capacity-limited dispatch */

/*
 * Expert capacity: ceil(T k / E * capacity_factor), evaluated in binary64 in
 * that order (P5 §3.2 prints the formula and the value 64 for T = 2048,
 * k = 2, E = 128, factor 2).
 */
int64_t oracle_capacity(int64_t T, int32_t E, int32_t k, double capacity_factor)
{
    return (int64_t)ceil((double)T * (double)k / (double)E * capacity_factor);
}

/*
 * Capacity-limited dispatch of a routing (P5 §3.2: an expert whose queue is
 * full sends further tokens to their next-best expert; P2 §3.2: the capacity
 * factor trades drops against idle capacity, and dropped requests are
 * retried at the next-best expert).  Read as two passes over the T k
 * assignments in row-major (token, slot) order, the order in which they
 * queue:
 *   1. an assignment keeps its expert while that expert holds fewer than
 *      cap assignments; otherwise it overflows;
 *   2. (policy 1, reroute) each overflowed assignment, in the same order,
 *      moves to the best-ranked expert (larger z first, NaN last, ties to the
 *      lower index) that its token does not already use and that holds fewer
 *      than cap assignments; with no such expert, or under policy 0 (drop),
 *      it is dropped: id -1.
 * ids [T][k] is read (the top-k routing) and rewritten; z and p are the
 * routing's [T][E] logits-over-tau and softmax rows.  gates/gate_p receive
 * p[t][id] (0 for a dropped assignment), not renormalised.  counts[E]
 * receives the per-expert totals.  Returns 0, or -1 on a bad argument.
 */
int oracle_capacity_dispatch(int64_t T, int32_t E, int32_t k, int64_t cap, int32_t policy,
                             const double *z, const double *p, int32_t *ids, float *gates,
                             double *gate_p, int32_t *counts)
{
    if (T < 0 || E < 1 || k < 1 || cap < 0 || (policy != 0 && policy != 1))
        return -1;
    uint8_t *overflow = (uint8_t *)calloc((size_t)(T * k > 0 ? T * k : 1), 1);
    if (!overflow)
        return -1;
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    /* pass 1 */
    for (int64_t a = 0; a < T * k; ++a) {
        int32_t e = ids[a];
        if (e < 0 || e >= E) {
            free(overflow);
            return -1;
        }
        if (counts[e] < cap) {
            counts[e] += 1;
        } else {
            overflow[a] = 1;
            ids[a] = -1;
        }
    }
    /* pass 2 */
    if (policy == 1) {
        for (int64_t t = 0; t < T; ++t)
            for (int32_t j = 0; j < k; ++j) {
                if (!overflow[t * k + j])
                    continue;
                int32_t best = -1;
                for (int32_t e = 0; e < E; ++e) {
                    if (counts[e] >= cap)
                        continue;
                    int used = 0;
                    for (int32_t jj = 0; jj < k; ++jj)
                        if (ids[t * k + jj] == e)
                            used = 1;
                    if (used)
                        continue;
                    if (best < 0 || ranks_before(z + t * E, e, best))
                        best = e;
                }
                if (best >= 0) {
                    ids[t * k + j] = best;
                    counts[best] += 1;
                }
            }
    }
    for (int64_t a = 0; a < T * k; ++a) {
        double g = ids[a] >= 0 ? p[(a / k) * E + ids[a]] : 0.0;
        gates[a] = (float)g;
        if (gate_p)
            gate_p[a] = g;
    }
    free(overflow);
    return 0;
}

/* ------------------------------------------------------- router statistics */

/*
 * Batch statistics of the routing (ids [T][k], full softmax rows p [T][E]):
 *   fraction[e]  = #{(t, j): ids[t][j] = e} / (T k)       share of the assignments,
 *                  whose target is 1/E                     P5 §3.2 balance loss
 *   mean_prob[e] = (1/T) sum_t p[t][e]                     P3 §4.2 expert_load buffer
 *   scalars[0]   = (1/T) sum_t ( -sum_e p[t][e] ln p[t][e] ), with 0 ln 0 = 0
 *                                                          P1 §3.2 router entropy
 *   scalars[1]   = sum_e (fraction[e] - 1/E)^2             P5 §3.2 (without lambda)
 *   scalars[2]   = sum_e (mean_prob[e] - 1/E)^2            P3 §3.2 (without lambda)
 *   scalars[3]   = sqrt( (1/E) sum_e (fraction[e] - 1/E)^2 ) spread of expert
 *                  utilisation (population standard deviation) P5 §4 monitoring
 *   scalars[4]   = E sum_e fraction[e] * mean_prob[e]       the product form of the
 *                  balance term, pairing P5 §3.2's assignment fractions with
 *                  P3 §4.2's mean probabilities (1 when both are uniform)
 * Sums run in ascending index order.  Returns 0, or -1 if T < 1 or an id is
 * out of range.
 */
int oracle_router_stats(int64_t T, int32_t E, int32_t k, const int32_t *ids, const double *p,
                        double *fraction, double *mean_prob, double *scalars)
{
    if (T < 1)
        return -1;
    for (int32_t e = 0; e < E; ++e) {
        fraction[e] = 0.0;
        mean_prob[e] = 0.0;
    }
    for (int64_t a = 0; a < T * k; ++a) {
        if (ids[a] < 0 || ids[a] >= E)
            return -1;
        fraction[ids[a]] += 1.0;
    }
    double entropy = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        double h = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            const double q = p[t * E + e];
            mean_prob[e] += q;
            if (q != 0.0)
                h -= q * log(q);
        }
        entropy += h;
    }
    double sf = 0.0, sp = 0.0, fp = 0.0;
    for (int32_t e = 0; e < E; ++e) {
        fraction[e] /= (double)T * (double)k;
        mean_prob[e] /= (double)T;
        sf += (fraction[e] - 1.0 / E) * (fraction[e] - 1.0 / E);
        sp += (mean_prob[e] - 1.0 / E) * (mean_prob[e] - 1.0 / E);
        fp += fraction[e] * mean_prob[e];
    }
    scalars[0] = entropy / (double)T;
    scalars[1] = sf;
    scalars[2] = sp;
    scalars[3] = sqrt(sf / E);
    scalars[4] = (double)E * fp;
    return 0;
}

/* --------------------------------------------------------------- expert FFN */

/*
 * o[0..d) = W2_e * act(W1_e * xr) for one token row xr (binary64, length d).
 * act 0 = GeLU, 1 = SiLU: W1e is d_ff x d.  act 2 = SwiGLU: W1e is 2 d_ff x d
 * with the gate/up rows of step 6' and a[n] = SiLU(gate . x) * (up . x).
 * W2e is d x d_ff; all in w_dtype; S1e/S2e are the bf16 group scales for INT4
 * (ignored otherwise).  Returns 0, or -1 on a bad argument.
 */
int oracle_expert_ffn(int64_t d, int64_t d_ff, int32_t w_dtype, int32_t act,
                      const double *xr, const void *W1e, const void *S1e,
                      const void *W2e, const void *S2e, double *o)
{
    if (w_dtype == ORACLE_INT4_G128 && (d % 128 != 0 || d_ff % 128 != 0 || !S1e || !S2e))
        return -1;
    if (act < 0 || act > 2 || (act == 2 && d_ff % 16 != 0))
        return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)d_ff);
    if (!a)
        return -1;
    for (int64_t n = 0; n < d_ff; ++n) {
        if (act == 2) {
            /* SwiGLU: the unit's gate and up rows of the 2 d_ff-row W1 */
            int64_t rg = 32 * (n / 16) + n % 16, ru = rg + 16;
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < d; ++i)
                g += load_w(W1e, S1e, w_dtype, d, rg, i) * xr[i];
            for (int64_t i = 0; i < d; ++i)
                u += load_w(W1e, S1e, w_dtype, d, ru, i) * xr[i];
            a[n] = oracle_silu(g) * u;
            continue;
        }
        double h = 0.0;
        for (int64_t i = 0; i < d; ++i)
            h += load_w(W1e, S1e, w_dtype, d, n, i) * xr[i];
        if (act == 1)
            a[n] = oracle_silu(h);
        else
            a[n] = oracle_gelu(h);
    }
    for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t n = 0; n < d_ff; ++n)
            acc += load_w(W2e, S2e, w_dtype, d_ff, c, n) * a[n];
        o[c] = acc;
    }
    free(a);
    return 0;
}

/*
 * One expert linear map, out[n] = sum_i W_e[n][i] * xr[i] for n < N (ascending
 * i), with W_e an N x K matrix in w_dtype (INT4: q * s exactly, from the bf16
 * group scales S_e [N][K/128]).  This is each of the two products of step 6
 * taken alone (P3 §3.2; P1 §5.4 and P2 §2.3 for the INT4 weights).  Returns 0,
 * or -1 on a bad argument.
 */
int oracle_expert_linear(int64_t N, int64_t K, int32_t w_dtype, const double *xr, const void *We,
                         const void *Se, double *out)
{
    if (N < 1 || K < 1 || (w_dtype == ORACLE_INT4_G128 && (K % 128 != 0 || !Se)))
        return -1;
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i)
            acc += load_w(We, Se, w_dtype, K, n, i) * xr[i];
        out[n] = acc;
    }
    return 0;
}

/*
 * Layer output for the listed tokens: y[r][c] = sum_j gate_p[t][j] * o_j[c],
 * t = tokens[r], o_j the FFN of expert ids[t][j].  W1/S1/W2/S2 are arrays of E
 * per-expert pointers (an expert no listed token routes to may be NULL).
 * Returns 0, or -1 on a bad argument or a missing expert.
 */
int oracle_forward_tokens(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k,
                          int32_t act_dtype, int32_t w_dtype, int32_t act, const void *x,
                          const int32_t *ids, const double *gate_p,
                          const void *const *W1, const void *const *S1,
                          const void *const *W2, const void *const *S2,
                          int64_t ntok, const int64_t *tokens, double *y)
{
    double *xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!xr || !o) {
        free(xr); free(o);
        return -1;
    }
    int rc = 0;
    for (int64_t r = 0; r < ntok && rc == 0; ++r) {
        int64_t t = tokens[r];
        if (t < 0 || t >= T) {
            rc = -1;
            break;
        }
        for (int64_t i = 0; i < d; ++i)
            xr[i] = load_act(x, act_dtype, t * d + i);
        for (int64_t c = 0; c < d; ++c)
            y[r * d + c] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            if (e == -1)
                continue; /* dropped by capacity-limited dispatch */
            if (e < 0 || e >= E || !W1[e] || !W2[e]) {
                rc = -1;
                break;
            }
            rc = oracle_expert_ffn(d, d_ff, w_dtype, act, xr, W1[e], S1 ? S1[e] : NULL,
                                   W2[e], S2 ? S2[e] : NULL, o);
            if (rc != 0)
                break;
            double w = gate_p[t * k + j];
            for (int64_t c = 0; c < d; ++c)
                y[r * d + c] += w * o[c];
        }
    }
    free(xr);
    free(o);
    return rc;
}
