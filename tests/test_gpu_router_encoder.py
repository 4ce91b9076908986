"""GPU parity of the two-layer router (router_hidden = d_r > 0).

Stage: moe_router_encoder's hidden layer h = GeLU(W_in x + b_in) against the
oracle's, element by element.  The GPU accumulates in fp32 (MFMA for bf16)
where the oracle sums in binary64, so an element may round to the other
neighbour: the bound is one storage rounding (bf16: 2^-8 relative) plus the
fp32 accumulation error d 2^-24 sum_i |W_in x| (times GeLU's slope, below 1.13).

Routing: the second layer reads h, so a rounding flip in h moves z by
dz[e] = sum_j (h_gpu - h_ref)[j] W_out[j][e] / tau, computed here from the
two hidden layers.  A token is ambiguous when two of its top-(k+1) z are
closer than twice its largest |dz| (or the usual 1e-12 relative margin);
everywhere else the ids must be bit-exact and the gates within 4 fp32 ulp
plus the effect of dz.  y is checked on the unambiguous tokens."""
import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import gpu_harness as H
from tests import npref

pytestmark = pytest.mark.gpu

F32, BF16, INT4 = moe.F32, moe.BF16, moe.INT4_G128


def case(T, d, d_ff, E, d_r, k=2, act=BF16, w=BF16, bias=False, tau=1.0, gumbel=False):
    return dict(T=T, d=d, d_ff=d_ff, E=E, k=k, act=act, w=w, bias=bias, tau=tau, gumbel=gumbel, router_hidden=d_r,
                name="case")


CASES = {
    # d_r = d/4 as in the pages; streaming (T <= 16) and tiled first layers; fp32 with the fp32 GEMM
    "bf16-T200-d512-dr128-E16": case(200, 512, 1024, 16, 128),
    "bf16-T12-d1024-dr256-E8-bias": case(12, 1024, 512, 8, 256, bias=True),
    "bf16-T77-d768-dr192-E16-gumbel-tau0.5": case(77, 768, 512, 16, 192, tau=0.5, gumbel=True),
    "int4-T40-d1024-dr256-E8": case(40, 1024, 1024, 8, 256, w=INT4),
    "f32-T64-d256-dr64-E8-k3": case(64, 256, 256, 8, 64, k=3, act=F32, w=F32),
}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


def _inputs(cfg, dev, seed):
    return {k: (v.to(dev) if v is not None else None) for k, v in moe_synth.generate(cfg, "cpu", seed).items()}


def _f64(t):
    return npref.bf16_bits_to_f64(moe_synth.to_bits(t)) if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def _hidden(cfg, inp, dev):
    c = H.abi_config(cfg)
    ws = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    h = torch.empty((cfg["T"], cfg["router_hidden"]), dtype=inp["x"].dtype, device=dev)
    moe.moe_router_encoder(c, inp["x"], inp["W_in"], inp["b_in"], h, ws)
    torch.cuda.synchronize()
    return h


def _hidden_bound(cfg, inp, h_ref):
    """Per-element bound on |h_gpu - h_ref| (see the module docstring)."""
    x, W = _f64(inp["x"]), _f64(inp["W_in"])
    S = np.abs(x) @ np.abs(W).T
    rel = 2.0 ** -8 if cfg["act"] == BF16 else 2.0 ** -23
    return rel * np.abs(h_ref) + 1.13 * cfg["d"] * 2.0 ** -24 * S + 1e-30


@pytest.mark.parametrize("name", list(CASES))
def test_encoder_stage(dev, oracle, name):
    cfg = CASES[name]
    inp = _inputs(cfg, dev, seed=8)
    h = _hidden(cfg, inp, dev)
    ref = oracle.router_encoder(moe_synth.to_bits(inp["x"]), moe_synth.to_bits(inp["W_in"]),
                                inp["b_in"].cpu().numpy(), cfg["act"])
    h_ref = npref.bf16_bits_to_f64(ref) if cfg["act"] == BF16 else ref.astype(np.float64)
    got = _f64(h)
    err = np.abs(got - h_ref)
    bound = _hidden_bound(cfg, inp, h_ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3e}"
    print(f"\n{name}: hidden elements differing from the oracle: {np.count_nonzero(err)} of {err.size}")


@pytest.mark.parametrize("name", list(CASES))
def test_encoder_routing_and_layer(dev, oracle, name):
    cfg = CASES[name]
    inp = _inputs(cfg, dev, seed=9)
    out = H.run_forward(cfg, inp, noise_seed=4)
    ref = H.oracle_route(oracle, cfg, inp, noise_seed=4)
    # z shift caused by the hidden layer's rounding differences
    h = _hidden(cfg, inp, dev)
    h_ref = npref.bf16_bits_to_f64(ref["h"]) if cfg["act"] == BF16 else ref["h"].astype(np.float64)
    dz = (_f64(h) - h_ref) @ _f64(inp["Wg"]) / H.tau32(cfg["tau"])
    dzmax = np.max(np.abs(dz), axis=1)
    k, E = cfg["k"], cfg["E"]
    z = ref["z"]
    zs = -np.sort(-z, axis=1)[:, :min(k + 1, E)]
    gaps = zs[:, :-1] - zs[:, 1:]
    margin = 2.0 * dzmax[:, None] + H.AMBIGUOUS_REL * np.max(np.abs(z), axis=1, keepdims=True)
    amb = set(np.where(np.any(gaps <= margin, axis=1))[0].tolist())
    assert len(amb) <= max(1, cfg["T"] // 20), f"{len(amb)} ambiguous tokens"
    ids = out["ids"].cpu().numpy()
    gates = out["gates"].cpu().numpy().astype(np.float64)
    ok = np.array([t not in amb for t in range(cfg["T"])])
    assert np.array_equal(ids[ok], ref["ids"][ok])
    ulp = np.spacing(np.abs(ref["gates"]).astype(np.float32)).astype(np.float64)
    allow = 4 * ulp + 2.5 * dzmax[:, None] * np.abs(ref["gates"].astype(np.float64))
    assert np.all(np.abs(gates - ref["gates"])[ok] <= allow[ok])
    # the router stage and the statistics entry point route the same way as the layer
    c = H.abi_config(cfg, seed=4)
    ids2 = torch.empty_like(out["ids"])
    g2 = torch.empty_like(out["gates"])
    ws = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    moe.moe_router(c, inp["x"], inp["Wg"], inp["bias"], ids2, g2, ws, W_in=inp["W_in"], b_in=inp["b_in"])
    wss = torch.empty(max(256, moe.moe_router_stats_workspace_size(c)), dtype=torch.uint8, device=dev)
    f64 = dict(dtype=torch.float64, device=dev)
    ids3, g3 = torch.empty_like(ids2), torch.empty_like(g2)
    moe.moe_router_stats(c, inp["x"], inp["Wg"], inp["bias"], ids3, g3, torch.empty(E, **f64),
                         torch.empty(E, **f64), torch.empty(5, **f64), wss, W_in=inp["W_in"], b_in=inp["b_in"])
    torch.cuda.synchronize()
    assert torch.equal(ids2, out["ids"]) and torch.equal(g2, out["gates"])
    assert torch.equal(ids3, out["ids"]) and torch.equal(g3, out["gates"])
    tokens = np.where(ok)[0]
    y_ref = H.oracle_y(oracle, cfg, inp, ref, tokens)
    H.check_y(out["y"], tokens, y_ref, cfg["act"])
    print(f"\n{name}: ambiguous {len(amb)}, largest |dz| {dzmax.max():.2e}")
