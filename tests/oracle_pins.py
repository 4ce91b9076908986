"""Pins of the CPU oracle to things other than itself.

Each pin takes an `Oracle` instance and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix: library routines
(numpy's Philox bit generator, numpy matmul, scipy's normal CDF and softmax,
numpy's stable sort), closed forms, brute force over all expert subsets, the
Gumbel-max theorem, and the router example printed on page P5 §3.1.  The
mutation test runs the same pins against deliberately broken copies of the
oracle and requires every copy to fail at least one of them.
"""
import json
import math
import os

import numpy as np
from scipy import stats

from oracle.oracle import BF16, F32, INT4_G128
from tests import npref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16(a):
    return npref.f64_to_bf16_bits(a)


def _tiny(seed, T=12, d=16, d_ff=32, E=6, dtype=F32):
    """A tiny random layer in float32 or bf16 bits, plus float64 views."""
    r = _rng(seed)
    x = r.standard_normal((T, d))
    Wg = r.standard_normal((d, E)) / math.sqrt(d)
    W1 = r.standard_normal((E, d_ff, d)) / math.sqrt(d)
    W2 = r.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)
    if dtype == F32:
        raw = [a.astype(np.float32) for a in (x, Wg, W1, W2)]
        f64 = [a.astype(np.float64) for a in raw]
    else:
        raw = [_bf16(a) for a in (x, Wg, W1, W2)]
        f64 = [npref.bf16_bits_to_f64(a) for a in raw]
    return raw, f64


# ------------------------------------------------------------------ generator

def pin_philox_matches_numpy(orc):
    """Philox4x64-10 blocks equal numpy's Philox bit generator.  numpy advances
    its 256-bit counter by one before producing a block, so counter c-1 yields
    the block of counter c."""
    mask = (1 << 64) - 1
    cases = [((0, 0, 0, 0), (0, 0)), ((1, 2, 3, 4), (5, 6)), ((0, 1, 0, 0), (mask, 7)),
             ((mask, 0, 0, 0), (123456789, 987654321)), ((17, 4, 0, 0), (0, 0)),
             ((2**40 + 3, 255, 0, 0), (2**63 + 11, 0))]
    for ctr, key in cases:
        c = list(ctr)
        # subtract one with borrow
        i = 0
        while True:
            if c[i] == 0:
                c[i] = mask
                i += 1
                if i == 4:
                    break
            else:
                c[i] -= 1
                break
        bg = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        want = bg.random_raw(4)
        got = orc.philox(ctr, key)
        assert np.array_equal(got, want), (ctr, key, got, want)


def pin_philox_known_answer(orc):
    """The published Philox4x64-10 known-answer vectors (tests/golden/philox4x64_10_kat.txt)."""
    with open(os.path.join(GOLDEN, "philox4x64_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v = [int(w, 16) for w in line.split()]
            got = orc.philox(v[0:4], v[4:6])
            assert [int(a) for a in got] == v[6:10], (line, [hex(int(a)) for a in got])


def pin_uniform_and_gumbel_distribution(orc):
    """u lies strictly inside (0,1) and is uniform; g = -ln(-ln u) follows the
    standard Gumbel law (Kolmogorov-Smirnov against scipy's CDFs)."""
    us = np.array([orc.uniform(3, t, e) for t in range(400) for e in range(10)])
    assert np.all(us > 0.0) and np.all(us < 1.0)
    assert stats.kstest(us, "uniform").pvalue > 1e-4
    gs = np.array([orc.gumbel(3, t, e) for t in range(400) for e in range(10)])
    assert np.all(np.isfinite(gs))
    assert stats.kstest(gs, stats.gumbel_r.cdf).pvalue > 1e-4
    # distinct (token, expert) keys give distinct draws; the seed matters
    assert len(np.unique(gs)) == len(gs)
    assert orc.gumbel(4, 0, 0) != orc.gumbel(3, 0, 0)
    assert orc.gumbel(3, 1, 0) != orc.gumbel(3, 0, 1)


def pin_uniform_stream_layout(orc):
    """The noise stream's layout (a reading: the pages only ask for a draw per
    (seed, token, expert)): u for (seed, t, e) takes the top 53 bits of word 0
    of the Philox4x64-10 block with key (seed, 0) and counter (t, e, 0, 0),
    read here from numpy's Philox bit generator, plus half an ulp."""
    for seed, t, e in ((0, 0, 0), (7, 3, 1), (2**40 + 1, 12345, 127), (5, 2**33, 255)):
        ctr = [t, e, 0, 0]
        c = list(ctr)
        i = 0
        while i < 4 and c[i] == 0:  # counter minus one (numpy pre-increments)
            c[i] = (1 << 64) - 1
            i += 1
        if i < 4:
            c[i] -= 1
        r0 = int(np.random.Philox(counter=np.array(c, dtype=np.uint64),
                                  key=np.array([seed, 0], dtype=np.uint64)).random_raw(1)[0])
        assert orc.uniform(seed, t, e) == ((r0 >> 11) + 0.5) / 2.0**53
        assert orc.gumbel(seed, t, e) == -math.log(-math.log(((r0 >> 11) + 0.5) / 2.0**53))


def _philox_block_numpy(seed, t, e):
    """The four words of the Philox4x64-10 block with key (seed, 0) and counter
    (t, e, 0, 0), from numpy's Philox bit generator (which pre-increments its
    counter, so it is started at counter - 1)."""
    c = [t, e, 0, 0]
    i = 0
    while i < 4 and c[i] == 0:
        c[i] = (1 << 64) - 1
        i += 1
    if i < 4:
        c[i] -= 1
    bg = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array([seed, 0], dtype=np.uint64))
    return [int(w) for w in bg.random_raw(4)]


def pin_normal_stream_layout(orc):
    """The Gaussian noise draw for (seed, t, e), exactly: the Box-Muller
    transform (Box & Muller 1958), sqrt(-2 ln u1) cos(2 pi u2), of u1 and u2
    built like the Gumbel uniform from words 2 and 3 of the Philox4x64-10
    block with key (seed, 0) and counter (t, e, 0, 0), the words read here from
    numpy's Philox bit generator and the transform evaluated with Python's math
    module (the same C library functions, so the result is bit-identical).  A
    sine for the cosine, words 2 and 3 swapped, or the Gumbel's word 0 reused
    all change the value."""
    keys = [(0, 0, 0), (7, 3, 1), (17, 1999, 9), (2**40 + 1, 12345, 127), (5, 2**33, 255), (2**64 - 1, 1, 2)]
    for seed, t, e in keys:
        r = _philox_block_numpy(seed, t, e)
        u1 = ((r[2] >> 11) + 0.5) / 2.0**53
        u2 = ((r[3] >> 11) + 0.5) / 2.0**53
        want = math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2)
        got = orc.normal(seed, t, e)
        assert got == want, (seed, t, e, got, want)


# ----------------------------------------------------------------------- GeLU

def pin_gelu(orc):
    """GeLU(h) = h * Phi(h): table value Phi(1) = 0.8413447460685429, zero at
    zero, odd-part identity GeLU(h) - GeLU(-h) = h, scipy's normal CDF, and
    relative accuracy in the negative tail (Phi(-10) = 7.62e-24 from scipy's
    log CDF), where 1 + erf cancels to zero."""
    assert orc.gelu(0.0) == 0.0
    assert abs(orc.gelu(1.0) - 0.8413447460685429) < 1e-15
    for h in np.linspace(-6, 6, 97):
        want = npref.gelu_cdf(h)
        assert abs(orc.gelu(h) - want) <= 1e-14 * max(1.0, abs(want)), h
        assert abs(orc.gelu(h) - orc.gelu(-h) - h) <= 1e-14 * max(1.0, abs(h)), h
    assert orc.gelu(40.0) == 40.0
    assert abs(orc.gelu(-40.0)) < 1e-300
    for h in (-8.0, -10.0, -20.0, -30.0):
        want = h * np.exp(stats.norm.logcdf(h))
        assert abs(orc.gelu(h) - want) <= 1e-12 * abs(want), h  # erfc at x = |h|/sqrt 2: ~2 x^2 ulp


# -------------------------------------------------------------------- routing

def pin_logits_closed_forms(orc):
    """One-hot tokens select rows of Wg exactly; small-integer tokens and gates
    give exact integer logits (numpy int64 matmul)."""
    r = _rng(1)
    d, E = 24, 7
    Wg = r.standard_normal((d, E)).astype(np.float32)
    x = np.zeros((d, d), dtype=np.float32)
    np.fill_diagonal(x, 1.0)
    out = orc.route(x, Wg, 2, F32, want_zp=True)
    assert np.array_equal(out["z"], Wg.astype(np.float64))
    xi = r.integers(-9, 10, size=(10, d))
    Wi = r.integers(-9, 10, size=(d, E))
    out = orc.route(xi.astype(np.float32), Wi.astype(np.float32), 2, F32, want_zp=True)
    assert np.array_equal(out["z"], (xi @ Wi).astype(np.float64))
    # the same through bf16 storage (small integers are exact in bf16)
    out = orc.route(_bf16(xi), _bf16(Wi), 2, BF16, want_zp=True)
    assert np.array_equal(out["z"], (xi @ Wi).astype(np.float64))


def pin_logits_library(orc):
    """bf16 and fp32 logits agree with numpy float64 matmul to rounding."""
    for dtype in (F32, BF16):
        (x, Wg, _, _), (xf, Wgf, _, _) = _tiny(2, T=20, d=64, E=9, dtype=dtype)
        bias = _rng(3).standard_normal(9).astype(np.float32)
        out = orc.route(x, Wg, 2, dtype, bias=bias, want_zp=True)
        want = xf @ Wgf + bias.astype(np.float64)
        assert np.max(np.abs(out["z"] - want)) <= 1e-13 * np.max(np.abs(want))


def pin_temperature_scaling(orc):
    """z = (l + g)/tau: tau=0.5 doubles z exactly, with or without noise."""
    (x, Wg, _, _), _ = _tiny(4, dtype=BF16)
    for gum in (False, True):
        a = orc.route(x, Wg, 2, BF16, tau=1.0, use_gumbel=gum, seed=9, want_zp=True)
        b = orc.route(x, Wg, 2, BF16, tau=0.5, use_gumbel=gum, seed=9, want_zp=True)
        assert np.array_equal(b["z"], 2.0 * a["z"])
        assert np.array_equal(a["ids"], b["ids"])


def pin_noise_is_additive_gumbel(orc):
    """With noise on, z - z_noiseless equals the generator's Gumbel draw for
    (seed, token_offset + t, e), up to the rounding of one addition."""
    (x, Wg, _, _), _ = _tiny(5, T=6, E=5, dtype=F32)
    a = orc.route(x, Wg, 2, F32, want_zp=True)
    b = orc.route(x, Wg, 2, F32, use_gumbel=True, seed=11, token_offset=100, want_zp=True)
    for t in range(6):
        for e in range(5):
            g = orc.gumbel(11, 100 + t, e)
            assert abs((b["z"][t, e] - a["z"][t, e]) - g) <= 1e-15 * (abs(a["z"][t, e]) + abs(g) + 1)


def pin_token_offset(orc):
    """Noise is keyed on the absolute token index: routing tokens [5, 5+T) of a
    batch with offset 0 equals routing the same rows alone with offset 5."""
    (x, Wg, _, _), _ = _tiny(6, T=16, E=8, dtype=BF16)
    full = orc.route(x, Wg, 2, BF16, tau=0.5, use_gumbel=True, seed=2, want_zp=True)
    part = orc.route(x[5:], Wg, 2, BF16, tau=0.5, use_gumbel=True, seed=2, token_offset=5,
                     want_zp=True)
    assert np.array_equal(part["z"], full["z"][5:])
    assert np.array_equal(part["ids"], full["ids"][5:])


def pin_topk_bruteforce(orc):
    """The chosen set is the unique k-subset with the largest sum of z (all
    C(E,k) subsets enumerated), listed in descending z."""
    for seed, E, k in ((7, 6, 1), (8, 6, 2), (9, 7, 3), (10, 8, 2), (11, 5, 5)):
        (x, Wg, _, _), _ = _tiny(seed, T=25, E=E, dtype=F32)
        out = orc.route(x, Wg, k, F32, use_gumbel=(seed % 2 == 0), seed=seed, want_zp=True)
        for t in range(25):
            z = out["z"][t]
            ids = out["ids"][t]
            assert set(ids.tolist()) == npref.topk_bruteforce(z, k)
            assert len(set(ids.tolist())) == k
            assert all(z[ids[j]] >= z[ids[j + 1]] for j in range(k - 1))


def pin_topk_ties_and_nan(orc):
    """Exact ties go to the lower expert index; NaN ranks below every number."""
    d, E = 4, 6
    Wg = np.zeros((d, E), dtype=np.float32)
    Wg[0, :] = [1.0, 3.0, 3.0, 2.0, 3.0, 0.5]
    x = np.array([[1, 0, 0, 0]], dtype=np.float32)
    out = orc.route(x, Wg, 3, F32)
    assert out["ids"].tolist() == [[1, 2, 4]]
    out = orc.route(np.zeros((1, d), np.float32), Wg, 4, F32)  # all logits 0
    assert out["ids"].tolist() == [[0, 1, 2, 3]]
    Wn = Wg.copy()
    Wn[0, 1] = np.nan                       # expert 1's logit becomes NaN
    out = orc.route(x, Wn, 6, F32)
    assert out["ids"].tolist() == [[2, 4, 3, 0, 5, 1]]
    xn = np.array([[np.nan, 0, 0, 0]], dtype=np.float32)  # every logit NaN
    out = orc.route(xn, Wg, 2, F32)
    assert out["ids"].tolist() == [[0, 1]]


def pin_softmax_properties(orc):
    """Probabilities sum to one, are invariant to a constant logit shift, are
    1/E for equal logits, equal scipy's softmax, and the gates are exactly the
    chosen probabilities rounded to fp32 (no renormalisation)."""
    (x, Wg, _, _), (xf, Wgf, _, _) = _tiny(12, T=30, E=9, dtype=BF16)
    out = orc.route(x, Wg, 2, BF16, want_zp=True)
    assert np.allclose(out["p"].sum(axis=1), 1.0, rtol=0, atol=1e-15)
    from scipy import special
    assert np.max(np.abs(out["p"] - special.softmax(out["z"], axis=1))) <= 1e-15
    assert np.array_equal(out["gate_p"], np.take_along_axis(out["p"], out["ids"].astype(np.int64), 1))
    assert np.array_equal(out["gates"], out["gate_p"].astype(np.float32))
    shifted = orc.route(x, Wg, 2, BF16, bias=np.full(9, 3.0, np.float32), want_zp=True)
    assert np.max(np.abs(shifted["p"] - out["p"])) <= 1e-15
    assert np.array_equal(shifted["ids"], out["ids"])
    eq = orc.route(np.zeros((3, 16), np.float32), np.ones((16, 9), np.float32), 2, F32, want_zp=True)
    assert np.allclose(eq["p"], 1.0 / 9, rtol=0, atol=1e-16)
    one = orc.route(np.ones((3, 16), np.float32), np.ones((16, 1), np.float32), 1, F32)
    assert np.all(one["gates"] == 1.0) and np.all(one["ids"] == 0)


def pin_router_worked_example(orc):
    """P5 §3.1 prints a router distribution over 128 experts: 0.42 for expert
    03, 0.38 for 17, 0.12 for 55, 0.05 for 89 and the rest below 0.01, and says
    top-2 takes experts 03 and 17 with combined probability 0.80.  Feeding
    logits ln p (the remaining 0.03 spread evenly over the other 124 experts)
    through the router must reproduce that choice and those gates."""
    with open(os.path.join(GOLDEN, "p5_router_example.json")) as f:
        ex = json.load(f)
    E = ex["num_experts"]
    p = np.full(E, ex["rest_mass"] / (E - len(ex["listed"])))
    for e, pe in ex["listed"].items():
        p[int(e)] = pe
    logits = np.log(p).astype(np.float32)
    out = orc.route(np.zeros((1, 8), np.float32), np.zeros((8, E), np.float32), 2, F32,
                    bias=logits, want_zp=True)
    assert out["ids"].tolist() == [ex["top2_ids"]]
    assert np.allclose(out["gates"][0], ex["top2_gates"], rtol=0, atol=1e-6)
    assert abs(out["gates"][0].sum() - ex["top2_sum"]) < 1e-6
    # every listed expert below the top-2 has < 0.13; the rest < 0.01
    assert np.all(np.sort(out["p"][0])[:-4] < 0.01)


def pin_renormalised_gates(orc):
    """P4 §4.3 takes the softmax over the k chosen values.  On P5 §3.1's worked
    example this turns 0.42 and 0.38 into 0.42/0.80 = 0.525 and 0.475.  In
    general: the same experts as without renormalisation; the gates sum to 1;
    their ratio is exp(z_a - z_b); they equal p[ids] / sum p[ids] of the plain
    router; with k = 1 the gate is exactly 1."""
    with open(os.path.join(GOLDEN, "p5_router_example.json")) as f:
        ex = json.load(f)
    E = ex["num_experts"]
    p = np.full(E, ex["rest_mass"] / (E - len(ex["listed"])))
    for e, pe in ex["listed"].items():
        p[int(e)] = pe
    logits = np.log(p).astype(np.float32)
    out = orc.route(np.zeros((1, 8), np.float32), np.zeros((8, E), np.float32), 2, F32, bias=logits,
                    gate_norm=1)
    assert out["ids"].tolist() == [ex["top2_ids"]]
    assert np.allclose(out["gates"][0], [0.42 / 0.80, 0.38 / 0.80], rtol=0, atol=1e-6)

    (x, Wg, _, _), _ = _tiny(21, T=30, E=9, dtype=BF16)
    for k in (1, 2, 3):
        plain = orc.route(x, Wg, k, BF16, use_gumbel=True, seed=4, tau=0.5, want_zp=True)
        ren = orc.route(x, Wg, k, BF16, use_gumbel=True, seed=4, tau=0.5, want_zp=True, gate_norm=1)
        assert np.array_equal(ren["ids"], plain["ids"]) and np.array_equal(ren["z"], plain["z"])
        g = ren["gate_p"]
        assert np.all(np.abs(g.sum(axis=1) - 1.0) <= 1e-15)
        want = plain["gate_p"] / plain["gate_p"].sum(axis=1, keepdims=True)
        assert np.max(np.abs(g - want) / want) <= 1e-14
        if k == 1:
            assert np.all(ren["gates"] == 1.0)
        else:
            zs = np.take_along_axis(ren["z"], ren["ids"].astype(np.int64), 1)
            assert np.max(np.abs(g[:, 0] / g[:, 1] / np.exp(zs[:, 0] - zs[:, 1]) - 1.0)) <= 1e-14


def pin_gaussian_noise(orc):
    """P5 §3.3 adds Gaussian noise to the router logits.  The draws are standard
    normal (KS test against scipy over 20,000 (token, expert) keys; sample mean
    and variance), independent of the Gumbel draw of the same key (neither n
    nor n^2 correlates with it); the noise
    enters as z = (l + sigma n)/tau, keyed on the absolute token (routing a
    slice with its token offset reproduces the rows of the whole batch)."""
    n = np.array([orc.normal(17, t, e) for t in range(2000) for e in range(10)])
    g = np.array([orc.gumbel(17, t, e) for t in range(2000) for e in range(10)])
    assert stats.kstest(n, "norm").pvalue > 1e-3
    assert abs(n.mean()) < 4.0 / math.sqrt(len(n)) and abs(n.var() - 1.0) < 0.05
    assert abs(np.corrcoef(n, g)[0, 1]) < 4.0 / math.sqrt(len(n))
    assert abs(np.corrcoef(n * n, g)[0, 1]) < 4.0 / math.sqrt(len(n))  # magnitudes independent too
    (x, Wg, _, _), _ = _tiny(22, T=8, E=6, dtype=F32)
    a = orc.route(x, Wg, 2, F32, tau=0.5, want_zp=True)
    b = orc.route(x, Wg, 2, F32, tau=0.5, seed=3, token_offset=40, noise_std=0.1, want_zp=True)
    for t in range(8):
        for e in range(6):
            dn = 0.1 * orc.normal(3, 40 + t, e) / 0.5
            assert abs((b["z"][t, e] - a["z"][t, e]) - dn) <= 1e-14 * (abs(a["z"][t, e]) + abs(dn) + 1)
    part = orc.route(x[3:], Wg, 2, F32, tau=0.5, seed=3, token_offset=43, noise_std=0.1, want_zp=True)
    assert np.array_equal(part["z"], b["z"][3:]) and np.array_equal(part["ids"], b["ids"][3:])


def pin_router_encoder(orc):
    """P3 §3.1/§4.2: a two-layer router, h = GeLU(W_in x + b_in) of width d/4,
    then the linear router on h.  The hidden layer is stored in the
    activation dtype.  Pins: (1) bf16 rounding of h in one step from binary64:
    with one-hot W_in rows, r = 16 + c + 1/16 where c = +-2^-30 or 0 comes from
    a second bf16 input, and GeLU(r) = r exactly at this size; 16 + 1/16 is
    the midpoint between the bf16 neighbours 16 and 16.125, where the binary32
    value sits for all three c: +2^-30 must round up, -2^-30 down, 0 to the
    even neighbour 16.  (2) With small-integer inputs every sum is exact, and
    h equals numpy's GeLU (scipy normal CDF) rounded to the nearest bf16 by
    comparing neighbour distances.  (3) The routing on h equals the dense
    numpy softmax/top-k of h @ W_out."""
    W_in = np.zeros((3, 2), np.float64)
    W_in[:, 0] = 1.0
    W_in[:, 1] = 1.0
    x = np.array([[16.0, 2.0 ** -30], [16.0, -(2.0 ** -30)], [16.0, 0.0]])
    h = orc.router_encoder(_bf16(x), _bf16(W_in), np.full(3, 0.0625, np.float32), BF16)
    assert h[:, 0].tolist() == [0x4181, 0x4180, 0x4180]   # 16.125, 16, 16

    r = _rng(27)
    T, d, d_r, E = 20, 32, 16, 6
    xi = r.integers(-2, 3, (T, d)).astype(np.float64)
    Wi = r.integers(-1, 2, (d_r, d)).astype(np.float64)
    bi = (r.integers(-8, 9, d_r) / 8.0).astype(np.float32)
    h = orc.router_encoder(_bf16(xi), _bf16(Wi), bi, BF16)
    pre = xi @ Wi.T + bi.astype(np.float64)
    assert np.array_equal(h, npref.f64_to_bf16_nearest(npref.gelu_cdf(pre)))
    hf = orc.router_encoder(xi.astype(np.float32), Wi.astype(np.float32), bi, F32)
    ulp = np.spacing(np.abs(npref.gelu_cdf(pre).astype(np.float32)))
    assert np.all(np.abs(hf.astype(np.float64) - npref.gelu_cdf(pre)) <= ulp)
    Wo = r.standard_normal((d_r, E)).astype(np.float32)
    out = orc.route(_bf16(xi), npref.f64_to_bf16_bits(Wo), 2, BF16, encoder=(_bf16(Wi), bi), want_zp=True)
    assert np.array_equal(out["h"], h)
    z = npref.bf16_bits_to_f64(h) @ npref.bf16_bits_to_f64(npref.f64_to_bf16_bits(Wo))
    assert np.max(np.abs(out["z"] - z)) <= 1e-13 * np.max(np.abs(z))
    assert np.array_equal(out["ids"], npref.topk_lexsort(z, 2))


def pin_gumbel_max_theorem(orc):
    """Gumbel-max: with noise and tau=1, the first choice is distributed as
    softmax(l), and the ordered pair (a, b) of the top-2 as p_a p_b / (1 - p_a)
    (sampling without replacement).  Chi-square over 6000 independent tokens."""
    E, T = 4, 6000
    l = np.array([1.0, 0.0, -0.5, 0.7], dtype=np.float32)
    out = orc.route(np.zeros((T, 2), np.float32), np.zeros((2, E), np.float32), 2, F32,
                    bias=l, use_gumbel=True, seed=12345)
    p = np.exp(l.astype(np.float64))
    p /= p.sum()
    first = np.bincount(out["ids"][:, 0], minlength=E)
    assert stats.chisquare(first, p * T).pvalue > 1e-4
    pairs = np.zeros((E, E))
    for a, b in out["ids"]:
        pairs[a, b] += 1
    want = np.array([[p[a] * p[b] / (1 - p[a]) if a != b else 0.0 for b in range(E)] for a in range(E)])
    off = ~np.eye(E, dtype=bool)
    assert stats.chisquare(pairs[off], want[off] * T).pvalue > 1e-4
    # without noise every token picks the same pair
    det = orc.route(np.zeros((5, 2), np.float32), np.zeros((2, E), np.float32), 2, F32, bias=l)
    assert np.all(det["ids"] == [0, 3])


# ------------------------------------------------------------------- dispatch

def pin_permute_library(orc):
    """Counts are numpy's bincount, offsets its cumulative sum, and the
    dispatch order numpy's stable argsort of the row-major expert ids."""
    r = _rng(13)
    for T, k, E in ((50, 2, 8), (37, 3, 5), (1, 1, 1), (64, 2, 128), (0, 2, 4)):
        ids = np.array([r.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        out = orc.permute(ids, E)
        flat = ids.ravel()
        assert np.array_equal(out["counts"], np.bincount(flat, minlength=E))
        assert np.array_equal(out["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(out["sorted_token"], order // k)
        inv = np.empty_like(order)
        inv[order] = np.arange(len(order))
        assert np.array_equal(out["pos"].ravel(), inv)


# ---------------------------------------------------------------- expert FFN

def pin_ffn_permutation_closed_form(orc):
    """W1 and W2 as (non-symmetric) 0/1 selection matrices give
    o = W2 GeLU(W1 x) by index arithmetic alone: o[c] = GeLU(x[src(c)])."""
    d, d_ff = 8, 12
    r = _rng(14)
    rows = r.permutation(d_ff)[:d]          # W1[rows[i], i] = 1 -> h[rows[i]] = x[i]
    W1 = np.zeros((d_ff, d), np.float32)
    W1[rows, np.arange(d)] = 1.0
    perm = r.permutation(d)                 # W2[c, rows[perm[c]]] = 1 -> o[c] = gelu(x[perm[c]])
    W2 = np.zeros((d, d_ff), np.float32)
    W2[np.arange(d), rows[perm]] = 1.0
    x = r.standard_normal(d)
    o = orc.expert_ffn(x, W1, W2, F32)
    assert np.max(np.abs(o - npref.gelu_cdf(x[perm]))) <= 1e-15


def pin_single_expert_equals_dense(orc):
    """E=1, k=1: the layer equals the dense FFN W2 GeLU(W1 x), computed with
    numpy matmul and scipy's normal CDF, in fp32 and in bf16 storage."""
    for dtype in (F32, BF16):
        (x, Wg, W1, W2), (xf, _, W1f, W2f) = _tiny(15, T=9, d=32, d_ff=64, E=1, dtype=dtype)
        out = orc.forward(x, Wg, W1, W2, 1, dtype, dtype)
        want = npref.gelu_cdf(xf @ W1f[0].T) @ W2f[0].T
        assert np.all(out["ids"] == 0) and np.all(out["gates"] == 1.0)
        assert np.max(np.abs(out["y"] - want)) <= 1e-13 * np.max(np.abs(want))


def _swiglu_split(W1):
    """Gate and up matrices of a SwiGLU W1 whose 2 d_ff rows alternate in
    blocks of 16 (16 gate rows, then the same 16 units' up rows)."""
    rows, d = W1.shape
    blocks = W1.reshape(rows // 32, 2, 16, d)
    return blocks[:, 0].reshape(rows // 2, d), blocks[:, 1].reshape(rows // 2, d)


def pin_silu_and_swiglu_experts(orc):
    """P1 §3.3/§4.2 give the experts SiLU-gated (SwiGLU) FFNs.  SiLU: 0 at 0,
    silu(x) - silu(-x) = x, and x * scipy's expit(x).  SwiGLU with 0/1
    selection matrices: unit n's gate row picks x[a(n)], its up row x[b(n)],
    so o[c] = silu(x[a]) * x[b] by index arithmetic (two 16-unit blocks, so
    the block interleave is exercised).  Single-expert layers equal numpy/scipy
    dense FFNs: W2 silu(W1 x) and W2 (silu(G x) * U x) with G and U unpacked by
    a reshape, in fp32, bf16 and INT4 storage."""
    from scipy import special
    xs = np.array([0.0, 1e-3, 0.5, -0.5, 2.0, -3.0, 20.0, -40.0, 700.0, -700.0])
    assert orc.silu(0.0) == 0.0
    for v in xs:
        assert abs(orc.silu(v) - orc.silu(-v) - v) <= 1e-15 * max(1.0, abs(v))
        assert abs(orc.silu(v) - v * special.expit(v)) <= 1e-15 * max(1.0, abs(v))

    d, d_ff = 8, 32
    r = _rng(23)
    a_src, b_src = r.integers(0, d, d_ff), r.integers(0, d, d_ff)
    W1 = np.zeros((2 * d_ff, d), np.float32)
    for n in range(d_ff):
        rg = 32 * (n // 16) + n % 16
        W1[rg, a_src[n]] = 1.0
        W1[rg + 16, b_src[n]] = 1.0
    pick = r.permutation(d_ff)[:d]
    W2 = np.zeros((d, d_ff), np.float32)
    W2[np.arange(d), pick] = 1.0
    x = r.standard_normal(d)
    o = orc.expert_ffn(x, W1, W2, F32, act=2)
    want = x[a_src[pick]] * special.expit(x[a_src[pick]]) * x[b_src[pick]]
    assert np.max(np.abs(o - want)) <= 1e-15

    for dtype in (F32, BF16):
        (x, Wg, W1, W2), (xf, _, W1f, W2f) = _tiny(24, T=9, d=32, d_ff=64, E=1, dtype=dtype)
        out = orc.forward(x, Wg, W1, W2, 1, dtype, dtype, act=1)
        h = xf @ W1f[0].T
        want = (h * special.expit(h)) @ W2f[0].T
        assert np.max(np.abs(out["y"] - want)) <= 1e-13 * np.max(np.abs(want))
        (x, Wg, W1, W2), (xf, _, W1f, W2f) = _tiny(25, T=9, d=32, d_ff=128, E=1, dtype=dtype)
        W2h, W2hf = W2[:, :, :64], W2f[:, :, :64]     # d x d_ff with d_ff = 64 hidden units
        out = orc.forward(x, Wg, W1, np.ascontiguousarray(W2h), 1, dtype, dtype, act=2)
        G, U = _swiglu_split(W1f[0])
        g, u = xf @ G.T, xf @ U.T
        want = (g * special.expit(g) * u) @ W2hf[0].T
        assert np.max(np.abs(out["y"] - want)) <= 1e-13 * np.max(np.abs(want))

    # INT4 SwiGLU expert against the dense formula on the decoded q * s weights
    r = _rng(26)
    d, d_ff = 128, 128
    q1 = r.integers(-8, 8, (2 * d_ff, d))
    q2 = r.integers(-8, 8, (d, d_ff))
    s1 = _bf16(r.uniform(0.01, 0.05, (2 * d_ff, d // 128)))
    s2 = _bf16(r.uniform(0.01, 0.05, (d, d_ff // 128)))
    c1, c2 = npref.pack_int4(q1), npref.pack_int4(q2)
    x = r.standard_normal(d)
    o = orc.expert_ffn(x, c1, c2, INT4_G128, S1e=s1, S2e=s2, act=2)
    G, U = _swiglu_split(npref.dequant_int4(c1, s1))
    g, u = G @ x, U @ x
    want = npref.dequant_int4(c2, s2) @ (g * special.expit(g) * u)
    assert np.max(np.abs(o - want)) <= 1e-13 * np.max(np.abs(want))


def pin_expert_linear(orc):
    """One expert linear map alone (each of the FFN's two products): with unit
    scales and integer inputs an INT4 map is an exact integer matrix product
    (numpy int64 matmul); with random codes and scales it equals numpy's
    float64 matmul on the dequantised weights q * s, and with bf16 and fp32
    weights numpy's matmul on the widened values; one-hot inputs pick one
    column exactly (every group's own scale)."""
    r = _rng(41)
    N, K = 96, 384
    q = r.integers(-8, 8, size=(N, K))
    codes = npref.pack_int4(q)
    ones = _bf16(np.ones((N, K // 128)))
    xi = r.integers(-5, 6, size=K)
    got = orc.expert_linear(xi.astype(np.float64), codes, INT4_G128, Se=ones)
    assert np.array_equal(got, (q @ xi).astype(np.float64))
    sc = _bf16(r.uniform(0.001, 0.05, size=(N, K // 128)))
    Wf = npref.dequant_int4(codes, sc)
    x = r.standard_normal(K)
    got = orc.expert_linear(x, codes, INT4_G128, Se=sc)
    want = Wf @ x
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))
    for c in (0, 127, 128, 200, 383):
        e = np.zeros(K)
        e[c] = 1.0
        assert np.array_equal(orc.expert_linear(e, codes, INT4_G128, Se=sc), Wf[:, c])
    wb = _bf16(r.standard_normal((N, K)) / math.sqrt(K))
    got = orc.expert_linear(x, wb, BF16)
    want = npref.bf16_bits_to_f64(wb) @ x
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))
    wf = (r.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    got = orc.expert_linear(x, wf, F32)
    want = wf.astype(np.float64) @ x
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))


def pin_int4_decode(orc):
    """All sixteen signed codes decode (two's complement nibbles, even column in
    the low nibble), each 128-column group takes its own scale, and an INT4
    expert equals the dense FFN on q*s weights."""
    d, d_ff = 256, 384
    # every code at every parity, identity-like probing with one-hot rows
    q = np.tile(np.arange(-8, 8), (d_ff, d // 16))
    q = np.roll(q, 3, axis=1)
    scales = np.ones((d_ff, d // 128))
    scales[:, 1] = 2.0 ** -3
    codes = npref.pack_int4(q)
    sb = _bf16(scales)
    # W2: identity on the first d hidden units, scale 1
    q2 = np.zeros((d, d_ff), dtype=np.int64)
    q2[np.arange(d), np.arange(d)] = 1
    codes2, sb2 = npref.pack_int4(q2), _bf16(np.ones((d, d_ff // 128)))
    for i in (0, 1, 2, 127, 128, 129, 255):
        x = np.zeros(d)
        x[i] = 1.0
        o = orc.expert_ffn(x, codes, codes2, INT4_G128, S1e=sb, S2e=sb2)
        h = q[:d, i] * scales[:d, i // 128]
        want = npref.gelu_cdf(h)
        assert np.max(np.abs(o - want)) <= 1e-15 * max(1.0, np.max(np.abs(want))), i
    # random codes and scales against the dense formulation
    r = _rng(16)
    qa = r.integers(-8, 8, size=(d_ff, d))
    qb = r.integers(-8, 8, size=(d, d_ff))
    sa = _bf16(r.uniform(0.001, 0.02, size=(d_ff, d // 128)))
    sb_ = _bf16(r.uniform(0.001, 0.02, size=(d, d_ff // 128)))
    ca, cb = npref.pack_int4(qa), npref.pack_int4(qb)
    x = r.standard_normal(d)
    o = orc.expert_ffn(x, ca, cb, INT4_G128, S1e=sa, S2e=sb_)
    W1f = npref.dequant_int4(ca, sa)
    W2f = npref.dequant_int4(cb, sb_)
    want = W2f @ npref.gelu_cdf(W1f @ x)
    assert np.max(np.abs(o - want)) <= 1e-13 * np.max(np.abs(want))
    # integer GEMM exactness: scales 1, integer x -> integer h before GeLU
    ones_a = _bf16(np.ones((d_ff, d // 128)))
    xi = r.integers(-3, 4, size=d).astype(np.float64)
    h_exact = qa @ xi.astype(np.int64)
    W2sel = np.zeros((d, d_ff), dtype=np.int64)
    W2sel[np.arange(d), np.arange(d)] = 1
    o = orc.expert_ffn(xi, ca, npref.pack_int4(W2sel), INT4_G128, S1e=ones_a,
                       S2e=_bf16(np.ones((d, d_ff // 128))))
    want = npref.gelu_cdf(h_exact[:d].astype(np.float64))
    assert np.max(np.abs(o - want)) <= 1e-14 * np.max(np.abs(want))


# ----------------------------------------------------------------- the layer

def pin_layer_equals_dense_formulation(orc):
    """The sparse oracle equals the dense evaluate-every-expert-then-mask
    formulation (numpy) in y, ids and gates, with and without bias and noise."""
    for seed, dtype, E, k, use_bias, gum, tau in ((17, F32, 6, 2, False, False, 1.0),
                                                  (18, BF16, 5, 2, True, False, 1.0),
                                                  (19, BF16, 7, 3, False, True, 0.5),
                                                  (20, F32, 4, 1, True, True, 0.8)):
        (x, Wg, W1, W2), (xf, Wgf, W1f, W2f) = _tiny(seed, T=10, d=16, d_ff=24, E=E, dtype=dtype)
        bias = _rng(seed).standard_normal(E).astype(np.float32) if use_bias else None
        out = orc.forward(x, Wg, W1, W2, k, dtype, dtype, bias=bias, tau=tau, use_gumbel=gum,
                          seed=seed)
        g = None
        if gum:
            g = np.array([[orc.gumbel(seed, t, e) for e in range(E)] for t in range(10)])
        ref = npref.dense_moe(xf, Wgf, W1f, W2f, k, bias=None if bias is None else bias.astype(np.float64),
                              tau=tau, g=g)
        assert np.array_equal(out["ids"], ref["ids"])
        assert np.max(np.abs(out["gate_p"] - ref["gate_p"])) <= 1e-14
        assert np.max(np.abs(out["y"] - ref["y"])) <= 1e-12 * np.max(np.abs(ref["y"]))


def pin_token_permutation_equivariance(orc):
    """Permuting the tokens permutes y, ids and gates and leaves counts alone."""
    (x, Wg, W1, W2), _ = _tiny(21, T=14, E=6, dtype=BF16)
    a = orc.forward(x, Wg, W1, W2, 2, BF16, BF16)
    perm = _rng(22).permutation(14)
    b = orc.forward(x[perm], Wg, W1, W2, 2, BF16, BF16)
    assert np.array_equal(b["ids"], a["ids"][perm])
    assert np.array_equal(b["gates"], a["gates"][perm])
    assert np.array_equal(b["y"], a["y"][perm])
    assert np.array_equal(b["counts"], a["counts"])


def pin_invariants_at_tiny_workload(orc):
    """On the T=64, d=128, d_ff=512, E=8 fp32 workload: k distinct experts per
    token, counts summing to T*k, and an average active fraction of exactly k/E
    per token (P2 §2.2 gives 2/128 = 1.56% for 128 experts)."""
    r = _rng(23)
    T, d, d_ff, E, k = 64, 128, 512, 8, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    Wg = (r.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
    W1 = (r.standard_normal((E, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    W2 = (r.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)).astype(np.float32)
    out = orc.forward(x, Wg, W1, W2, k, F32, F32)
    assert all(len(set(row)) == k for row in out["ids"].tolist())
    assert out["counts"].sum() == T * k
    active = np.zeros((T, E), bool)
    active[np.arange(T)[:, None], out["ids"]] = True
    assert active.sum(axis=1).mean() / E == k / E
    assert np.all(np.isfinite(out["y"]))


# --------------------------------------------------- capacity-limited dispatch

def pin_capacity_formula(orc):
    """P5 §3.2 prints ceil(2048 * 2 / 128 * 2) = 64; two more values by hand."""
    assert orc.capacity(2048, 128, 2, 2.0) == 64
    assert orc.capacity(4096, 16, 2, 1.25) == 640
    assert orc.capacity(10, 3, 2, 1.0) == 7          # ceil(6.67)
    assert orc.capacity(8, 128, 2, 1.0) == 1         # ceil(0.125)


def _ranked_routing(orc, T, E, k, order_bias):
    """Every token ranks the experts alike: bias alone sets the logits."""
    return orc.route(np.zeros((T, 4), np.float32), np.zeros((4, E), np.float32), k, F32,
                     bias=np.asarray(order_bias, np.float32), want_zp=True)


def pin_capacity_by_hand(orc):
    """All 10 tokens rank experts 0 > 1 > 2 > 3 (k = 1) and the capacity is 3
    (factor 1.2: ceil(10/4*1.2) = 3).  Drop: tokens 0-2 keep expert 0, the
    rest are dropped (id -1, gate 0).  Reroute: tokens 3-5 move to expert 1,
    6-8 to expert 2, token 9 to expert 3, each gated by its own probability.
    With k = 2 (every token's top-2 = {0, 1}) and capacity 2 (factor 0.4:
    ceil(10*2/4*0.4) = 2): tokens 0 and 1 keep both; token 2's two slots move
    to experts 2 and then 3 (not 2 again: the token already uses it); token 3
    fills the second places of experts 2 and 3; every later slot is dropped."""
    r = _ranked_routing(orc, 10, 4, 1, [3.0, 2.0, 1.0, 0.0])
    drop = orc.capacity_dispatch(r, 1.2, 0)
    assert drop["cap"] == 3
    assert drop["ids"].ravel().tolist() == [0, 0, 0] + [-1] * 7
    assert drop["counts"].tolist() == [3, 0, 0, 0]
    assert np.all(drop["gates"].ravel()[3:] == 0) and np.all(drop["gates"].ravel()[:3] == r["gates"].ravel()[:3])
    rr = orc.capacity_dispatch(r, 1.2, 1)
    assert rr["ids"].ravel().tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2, 3]
    assert rr["counts"].tolist() == [3, 3, 3, 1]
    want = np.array([r["p"][t, e] for t, e in enumerate(rr["ids"].ravel())])
    assert np.array_equal(rr["gate_p"].ravel(), want)

    r2 = _ranked_routing(orc, 10, 4, 2, [3.0, 2.0, 1.0, 0.0])
    assert np.all(r2["ids"] == [0, 1])
    rr2 = orc.capacity_dispatch(r2, 0.4, 1)
    assert rr2["cap"] == 2
    assert rr2["ids"].tolist() == [[0, 1], [0, 1], [2, 3], [2, 3]] + [[-1, -1]] * 6
    assert rr2["counts"].tolist() == [2, 2, 2, 2]
    dr2 = orc.capacity_dispatch(r2, 0.4, 0)
    assert dr2["ids"].tolist() == [[0, 1], [0, 1]] + [[-1, -1]] * 8


def pin_capacity_invariants(orc):
    """Random skewed routing: no expert exceeds the capacity; a token never
    uses an expert twice; under drop the kept assignments are exactly the
    first `cap` of each expert in row-major order (numpy's stable argsort
    rank); kept gates equal the uncapped ones; a capacity of at least T k
    changes nothing; reroute with factor 2 drops nothing here; counts equal
    numpy's bincount of the surviving ids."""
    (x, Wg, _, _), _ = _tiny(41, T=60, E=6, dtype=BF16)
    bias = np.array([2.0, 1.0, 0.5, 0.0, -0.5, -1.0], np.float32)
    r = orc.route(x, Wg, 2, BF16, bias=bias, want_zp=True)
    T, k, E = 60, 2, 6
    flat = r["ids"].ravel()
    order = np.argsort(flat, kind="stable")
    rank = np.empty_like(order)
    for e in range(E):
        sel = order[flat[order] == e]
        rank[sel] = np.arange(len(sel))
    for cf in (0.5, 0.9, 1.3):
        dr = orc.capacity_dispatch(r, cf, 0)
        cap = dr["cap"]
        keep = rank < cap
        assert np.array_equal(dr["ids"].ravel(), np.where(keep, flat, -1))
        assert np.array_equal(dr["gates"].ravel(), np.where(keep, r["gates"].ravel(), 0.0))
        assert np.array_equal(dr["counts"], np.bincount(flat[keep], minlength=E))
        for pol in (0, 1):
            out = orc.capacity_dispatch(r, cf, pol)
            assert out["counts"].max() <= out["cap"]
            for row in out["ids"]:
                live = row[row >= 0]
                assert len(set(live.tolist())) == len(live)
            live = out["ids"].ravel()
            assert np.array_equal(out["counts"], np.bincount(live[live >= 0], minlength=E))
    big = orc.capacity_dispatch(r, 100.0, 1)
    assert np.array_equal(big["ids"], r["ids"]) and np.array_equal(big["gates"], r["gates"])
    rr = orc.capacity_dispatch(r, 2.0, 1)
    assert np.all(rr["ids"] >= 0) and rr["counts"].sum() == T * k


# ---------------------------------------------------------- router statistics

def pin_router_stats_closed_forms(orc):
    """Uniform logits: every p is 1/E (mean-probability balance term 0,
    entropy ln E) and ties send every token to experts 0..k-1, so the
    assignment fractions are 1/k there and 0 elsewhere.  A dominating bias
    makes p one-hot: entropy exactly 0 and that expert's mean probability 1.
    Two experts, two tokens with logit gaps +ln 3 and -ln 3: p = (3/4, 1/4)
    and (1/4, 3/4), mean probabilities 1/2, entropy = the binary entropy of
    1/4 (scipy), and top-1 fractions 1/2 each.  The product term
    E sum_e f_e P_e is 1 whenever the mean probabilities are uniform, and
    E * (1/2) * 1 = E/2 for the one-hot case (half the assignments on the
    expert that holds all the probability)."""
    T, d, E, k = 10, 8, 6, 2
    uni = orc.route(np.zeros((T, d), np.float32), np.zeros((d, E), np.float32), k, F32, want_zp=True)
    st = orc.router_stats(uni["ids"], uni["p"])
    want_f = np.array([1.0 / k] * k + [0.0] * (E - k))
    assert np.array_equal(uni["ids"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.allclose(st["fraction"], want_f, rtol=0, atol=1e-15)
    assert np.allclose(st["mean_prob"], 1.0 / E, rtol=0, atol=1e-15)
    assert abs(st["lb_prob"]) <= 1e-30
    assert abs(st["entropy"] - math.log(E)) <= 1e-14
    lb_f = k * (1.0 / k - 1.0 / E) ** 2 + (E - k) * (1.0 / E) ** 2
    assert abs(st["lb_fraction"] - lb_f) <= 1e-15
    assert abs(st["fraction_std"] - math.sqrt(lb_f / E)) <= 1e-15
    assert abs(st["lb_product"] - 1.0) <= 1e-15

    bias = np.zeros(E, np.float32)
    bias[3] = 1000.0
    hot = orc.route(np.zeros((T, d), np.float32), np.zeros((d, E), np.float32), k, F32, bias=bias, want_zp=True)
    st = orc.router_stats(hot["ids"], hot["p"])
    assert st["entropy"] == 0.0 and st["mean_prob"][3] == 1.0
    assert np.all(hot["ids"][:, 0] == 3)
    assert st["lb_product"] == E / 2

    # two tokens x = +1 and -1 against Wg = (q, -q), q = fp32(ln 3 / 2): logit gaps +-2q
    q = float(np.float32(math.log(3.0) / 2))
    two = orc.route(np.array([[1.0], [-1.0]], np.float32), np.array([[q, -q]], np.float32), 1, F32, want_zp=True)
    st = orc.router_stats(two["ids"], two["p"])
    pa = math.exp(2 * q) / (math.exp(2 * q) + 1.0)  # ~3/4
    assert abs(pa - 0.75) < 1e-7
    assert np.array_equal(two["ids"].ravel(), [0, 1])
    assert np.allclose(st["mean_prob"], [0.5, 0.5], rtol=0, atol=1e-15)
    assert np.array_equal(st["fraction"], [0.5, 0.5])
    assert abs(st["entropy"] - stats.entropy([pa, 1.0 - pa])) <= 1e-15
    assert st["lb_fraction"] == 0.0 and st["fraction_std"] == 0.0
    assert abs(st["lb_product"] - 1.0) <= 1e-15


def pin_router_stats_invariants(orc):
    """On random routings: the fractions and mean probabilities each sum to
    one, 0 <= entropy <= ln E, the balance terms are >= 0 with std^2 * E equal
    to the fraction term; relabelling the experts (permuting Wg's columns)
    permutes the per-expert results and leaves the scalars unchanged; the
    fractions equal numpy's bincount of the ids over T k."""
    (x, Wg, _, _), _ = _tiny(31, T=40, E=7, dtype=BF16)
    out = orc.route(x, Wg, 2, BF16, want_zp=True)
    st = orc.router_stats(out["ids"], out["p"])
    assert abs(st["fraction"].sum() - 1.0) <= 1e-15 and abs(st["mean_prob"].sum() - 1.0) <= 1e-14
    assert 0.0 <= st["entropy"] <= math.log(7) + 1e-15
    assert st["lb_fraction"] >= 0 and st["lb_prob"] >= 0
    assert abs(st["fraction_std"] ** 2 * 7 - st["lb_fraction"]) <= 1e-15
    assert np.array_equal(st["fraction"], np.bincount(out["ids"].ravel(), minlength=7) / (40 * 2))
    perm = np.array([3, 6, 0, 5, 1, 2, 4])
    outp = orc.route(x, np.ascontiguousarray(Wg[:, perm]), 2, BF16, want_zp=True)
    sp = orc.router_stats(outp["ids"], outp["p"])
    assert np.allclose(sp["fraction"], st["fraction"][perm], rtol=0, atol=0)
    assert np.allclose(sp["mean_prob"], st["mean_prob"][perm], rtol=0, atol=1e-15)
    assert st["lb_product"] > 0
    for key in ("entropy", "lb_fraction", "lb_prob", "fraction_std", "lb_product"):
        assert abs(sp[key] - st[key]) <= 1e-14 * max(1.0, abs(st[key]))


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
