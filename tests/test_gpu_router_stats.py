"""GPU parity of the router statistics (moe_router_stats, through the C ABI)
against the oracle's statistics of the oracle's own routing: assignment
fractions bit-exact (integer counts over T k), mean probabilities, entropy and
balance terms within 1e-12 (binary64 on both sides; only the exp/log
roundings and the summation order differ).  The ids and gates must equal
moe_router's."""
import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

F32, BF16, INT4 = moe.F32, moe.BF16, moe.INT4_G128


def case(T, d, E, k=2, act=BF16, bias=False, tau=1.0, gumbel=False):
    w = F32 if act == F32 else BF16
    return dict(T=T, d=d, d_ff=64, E=E, k=k, act=act, w=w, bias=bias, tau=tau, gumbel=gumbel, name="stats")


CASES = {
    "f32-T64-d128-E8": case(64, 128, 8, act=F32),
    "bf16-T200-d512-E128": case(200, 512, 128),
    "bf16-T333-d1024-E16-bias": case(333, 1024, 16, bias=True),
    "bf16-T77-d768-E16-gumbel-tau0.5": case(77, 768, 16, tau=0.5, gumbel=True),
    "bf16-T50-d256-E256-k8": case(50, 256, 256, k=8),
    "bf16-T4096-d1024-E16-bias": case(4096, 1024, 16, bias=True),
    "bf16-T1-d2048-E64": case(1, 2048, 64),
}


def _router_inputs(cfg, dev, seed):
    return {k: (v.to(dev) if v is not None else None) for k, v in moe_synth.generate_router(cfg, "cpu", seed).items()}


def _run_stats(cfg, inp, dev, noise_seed=9):
    c = H.abi_config(cfg, seed=noise_seed, token_offset=500)
    T, E, k = cfg["T"], cfg["E"], cfg["k"]
    ids = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    gates = torch.zeros((T, k), dtype=torch.float32, device=dev)
    frac = torch.full((E,), -1.0, dtype=torch.float64, device=dev)
    mprob = torch.full((E,), -1.0, dtype=torch.float64, device=dev)
    scal = torch.full((5,), -1.0, dtype=torch.float64, device=dev)
    ws = torch.empty(max(256, moe.moe_router_stats_workspace_size(c)), dtype=torch.uint8, device=dev)
    moe.moe_router_stats(c, inp["x"], inp["Wg"], inp["bias"], ids, gates, frac, mprob, scal, ws)
    # the plain router for comparison
    ids2 = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    gates2 = torch.zeros((T, k), dtype=torch.float32, device=dev)
    ws2 = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    moe.moe_router(c, inp["x"], inp["Wg"], inp["bias"], ids2, gates2, ws2)
    torch.cuda.synchronize()
    return dict(ids=ids, gates=gates, frac=frac, mprob=mprob, scal=scal, ids2=ids2, gates2=gates2)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(CASES))
def test_router_stats_parity(dev, oracle, name):
    cfg = CASES[name]
    inp = _router_inputs(cfg, dev, seed=2)
    out = _run_stats(cfg, inp, dev)
    assert torch.equal(out["ids"], out["ids2"]) and torch.equal(out["gates"], out["gates2"])
    ref = H.oracle_route(oracle, cfg, inp, noise_seed=9, token_offset=500)
    ids = out["ids"].cpu().numpy()
    amb = H.check_routing(ids, out["gates"].cpu().numpy(), ref, cfg["k"])
    assert not amb, f"ambiguous tokens {amb}: statistics would depend on a rounding-level tie"
    st = oracle.router_stats(ref["ids"], ref["p"])
    frac = out["frac"].cpu().numpy()
    assert np.array_equal(frac, st["fraction"]), np.max(np.abs(frac - st["fraction"]))
    assert np.max(np.abs(out["mprob"].cpu().numpy() - st["mean_prob"])) <= 1e-12
    scal = out["scal"].cpu().numpy()
    for i, key in enumerate(("entropy", "lb_fraction", "lb_prob", "fraction_std", "lb_product")):
        assert abs(scal[i] - st[key]) <= 1e-12 * max(1.0, abs(st[key])), (key, scal[i], st[key])


def test_router_stats_empty_batch(dev):
    cfg = case(0, 256, 8)
    c = H.abi_config(cfg)
    frac = torch.full((8,), 7.0, dtype=torch.float64, device=dev)
    mprob = torch.full((8,), 7.0, dtype=torch.float64, device=dev)
    scal = torch.full((5,), 7.0, dtype=torch.float64, device=dev)
    moe.moe_router_stats(c, None, None, None, None, None, frac, mprob, scal, None)
    torch.cuda.synchronize()
    assert frac.abs().sum().item() == 0 and mprob.abs().sum().item() == 0 and scal.abs().sum().item() == 0
