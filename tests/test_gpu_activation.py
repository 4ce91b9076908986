"""GPU check of the GEMM1 epilogues (GeLU, SiLU, SwiGLU) in isolation.

W1 rows are one-hot, so every sum the grouped GEMM forms has a single
non-zero bf16 * bf16 product and is exact in fp32: H must equal the
activation of known inputs, rounded once to bf16.  Bound, per element:
|H - act_ref| <= 2^-7 |act_ref| + 1e-6 |h| (one bf16 rounding step, plus
the activations' own approximation error, which matters only where the
result is tiny: GeLU's negative tail), with act_ref the oracle's binary64
activation.  Every kernel variant is covered: the streaming kernel with 16-,
32- and 64-row dispatch tiles and the tiled kernel with experts of 200, 100
and 40 rows (its 256-, 128- and 64-row tile heights)."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_03_amd as moe
from tests import npref

pytestmark = pytest.mark.gpu

D, DFF = 256, 256
ACTS = {"gelu": moe.ACT_GELU, "silu": moe.ACT_SILU, "swiglu": moe.ACT_SWIGLU}
SHAPES = [(moe.GEMM_STREAMING, 12), (moe.GEMM_STREAMING, 24), (moe.GEMM_STREAMING, 40), (moe.GEMM_TILED, 340)]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


def _counts(T):
    return [200, 100, 40] if T == 340 else [T - T // 3 - T // 4, T // 3, T // 4]


@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("path,T", SHAPES, ids=[f"path{p}-T{t}" for p, t in SHAPES])
def test_epilogue_activation(dev, oracle, act, path, T):
    code = ACTS[act]
    E = 3
    counts = _counts(T)
    rng = np.random.default_rng(T * 10 + code)
    # token values spread over [-8, 8] (GeLU's and SiLU's tails included), stored as bf16
    xv = rng.uniform(-8.0, 8.0, (T, D))
    xb = npref.f64_to_bf16_bits(xv)
    xf = npref.bf16_bits_to_f64(xb)
    N = 2 * DFF if code == moe.ACT_SWIGLU else DFF
    src = rng.integers(0, D, (E, N))
    W1 = np.zeros((E, N, D), np.float64)
    for e in range(E):
        W1[e, np.arange(N), src[e]] = 1.0
    W1b = npref.f64_to_bf16_bits(W1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a_rows = np.arange(T, dtype=np.int32)  # expert e's slots are tokens offsets[e] .. offsets[e+1]-1
    c = moe.config(T, D, DFF, E, 1, moe.BF16, moe.BF16, gemm_path=path, expert_act=code)
    x_t = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    W_t = torch.from_numpy(W1b.view(np.int16)).view(torch.bfloat16).to(dev)
    H = torch.full((T, DFF), float("nan"), dtype=torch.bfloat16, device=dev)
    moe.moe_grouped_gemm(c, 1, x_t, torch.from_numpy(a_rows).to(dev), torch.from_numpy(offsets).to(dev), W_t, None, H)
    torch.cuda.synchronize()
    got = npref.bf16_bits_to_f64(H.cpu().view(torch.int16).numpy().view(np.uint16))
    want = np.empty((T, DFF))
    hmag = np.empty((T, DFF))
    for e in range(E):
        for t in range(offsets[e], offsets[e + 1]):
            for u in range(DFF):
                if code == moe.ACT_SWIGLU:
                    rg = 32 * (u // 16) + u % 16
                    g, v = xf[t, src[e, rg]], xf[t, src[e, rg + 16]]
                    want[t, u] = oracle.silu(g) * v
                    hmag[t, u] = abs(g * v)
                else:
                    h = xf[t, src[e, u]]
                    want[t, u] = oracle.gelu(h) if code == moe.ACT_GELU else oracle.silu(h)
                    hmag[t, u] = abs(h)
    bound = 2.0 ** -7 * np.abs(want) + 1e-6 * hmag
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{act}: token {worst[0]} unit {worst[1]}: got {got[worst]}, want {want[worst]}"
