"""GPU parity of capacity-limited dispatch (moe_forward with capacity_factor >
0): expert ids, counts and gates bit-exact / within 4 fp32 ulp of the oracle's
capacity_dispatch of the oracle's own routing, and y against the oracle's
forward over the dispatched routing (dropped slots add nothing).

The reroute order depends on the full z order of every overflowing token, so
each case first asserts that no token of its seeded inputs has two z within
the binary64 rounding margin (1e-12 relative): then the routing is unique."""
import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

F32, BF16, INT4 = moe.F32, moe.BF16, moe.INT4_G128
DROP, REROUTE = moe.CAPACITY_DROP, moe.CAPACITY_REROUTE


def case(T, d, d_ff, E, k=2, act=BF16, w=BF16, bias=False, tau=1.0, gumbel=False):
    return dict(T=T, d=d, d_ff=d_ff, E=E, k=k, act=act, w=w, bias=bias, tau=tau, gumbel=gumbel, name="case")


CASES = {
    # skewed routing (bias b_e = 2 ln(1/(e+1))): the first experts overflow
    "bf16-T300-d512-dff1024-E8-skewed-cf1": (case(300, 512, 1024, 8, bias=True), 1.0),
    # heavy overflow: most assignments cannot be placed once the spare capacity runs out
    "bf16-T200-d256-dff512-E16-skewed-cf0.5": (case(200, 256, 512, 16, bias=True), 0.5),
    # k = 8 of 256 experts; capacity 2
    "bf16-T40-d256-dff256-E256-k8-cf1.25": (case(40, 256, 256, 256, k=8), 1.25),
    # k = 3 (chunks of 1365 whole tokens): two chunks and more than 256 overflowing slots in one
    "f32-T1500-d128-dff256-E5-k3-skewed-cf1.1": (case(1500, 128, 256, 5, k=3, act=F32, w=F32, bias=True), 1.1),
    # three chunks of 2048 tokens
    "bf16-T5000-d128-dff256-E16-skewed-cf1": (case(5000, 128, 256, 16, bias=True), 1.0),
    # Gumbel noise, tau = 0.5, INT4 experts
    "int4-T200-d384-dff768-E8-gumbel-cf0.9": (case(200, 384, 768, 8, w=INT4, tau=0.5, gumbel=True), 0.9),
    # decode: capacity ceil(8 * 2 / 128) = 1, streaming GEMMs
    "bf16-T8-d512-dff1024-E128-cf1": (case(8, 512, 1024, 128), 1.0),
    # the routing of the skewed T2048 E128 prefill layer at capacity factor 2 (about 3,700 overflowing slots walked in
    # batches of 32, each batch ranked while the one before it fills experts)
    "bf16-T2048-d128-dff256-E128-skewed-cf2": (case(2048, 128, 256, 128, bias=True), 2.0),
    # k = 8 of 256 skewed experts over two chunks
    "bf16-T1024-d128-dff128-E256-k8-skewed-cf1": (case(1024, 128, 128, 256, k=8, bias=True), 1.0),
    # 160 experts (three 64-expert words per lane of the walk, 30-row batches), k = 4
    "bf16-T700-d128-dff128-E160-k4-skewed-cf1": (case(700, 128, 128, 160, k=4, bias=True), 1.0),
    # exactly one 64-expert word
    "bf16-T1000-d128-dff128-E64-skewed-cf1.5": (case(1000, 128, 128, 64, bias=True), 1.5),
    # k = 1: every overflowing assignment is its token's only one
    "bf16-T1500-d128-dff128-E32-k1-skewed-cf1": (case(1500, 128, 128, 32, k=1, bias=True), 1.0),
}
PARAMS = [(n, pol) for n in CASES for pol in (DROP, REROUTE)]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


def _inputs(cfg, dev, seed):
    return {k: (v.to(dev) if v is not None else None) for k, v in moe_synth.generate(cfg, "cpu", seed).items()}


def _config(cfg, cf, policy, noise_seed, gemm_path=moe.GEMM_AUTO):
    return moe.config(cfg["T"], cfg["d"], cfg["d_ff"], cfg["E"], cfg["k"], cfg["act"], cfg["w"], tau=cfg["tau"],
                      use_gumbel=cfg["gumbel"], seed=noise_seed, gemm_path=gemm_path, capacity_factor=cf,
                      capacity_policy=policy)


def _run(c, inp):
    layer = moe.MoELayerForward(c, device="cuda")
    y, ids, gates, counts = layer(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W2"], inp["S1"], inp["S2"])
    torch.cuda.synchronize()
    return y, ids.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy()


@pytest.mark.parametrize("name,policy", PARAMS, ids=[f"{n}-{'reroute' if p else 'drop'}" for n, p in PARAMS])
def test_capacity_parity(dev, oracle, name, policy):
    cfg, cf = CASES[name]
    print(f"capacity case {name} policy {policy}", flush=True)
    inp = _inputs(cfg, dev, seed=11)
    y, ids, gates, counts = _run(_config(cfg, cf, policy, noise_seed=5), inp)
    route = H.oracle_route(oracle, cfg, inp, noise_seed=5)
    assert len(H.ambiguous_tokens(route["z"], cfg["E"])) == 0, "seeded inputs hold a z tie; pick another seed"
    ref = oracle.capacity_dispatch(route, float(np.float32(cf)), policy)
    assert 1 <= ref["cap"] < cfg["T"]
    assert np.any(ref["ids"] != route["ids"]), "the case should exercise overflow"
    assert np.array_equal(ids, ref["ids"]), f"ids differ at tokens {np.where(np.any(ids != ref['ids'], 1))[0][:10]}"
    assert np.array_equal(counts, ref["counts"])
    assert int(counts.sum()) == int((ids >= 0).sum())
    assert counts.max() <= ref["cap"]
    ulp = np.spacing(np.abs(ref["gates"]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(gates.astype(np.float64) - ref["gates"]) <= 4 * ulp)
    assert np.all(gates[ids < 0] == 0.0)
    if policy == DROP:  # dropping keeps every surviving slot where the router put it
        kept = ids >= 0
        assert np.array_equal(ids[kept], route["ids"][kept])
    tokens = np.arange(cfg["T"]) if cfg["T"] <= 400 else H.sample_tokens(np.where(ids < 0, 0, ids), cfg["E"], 200)
    # dropped tokens (all k slots -1) must come out as exact zeros
    y_ref = H.oracle_y(oracle, cfg, inp, ref, tokens)
    H.check_y(y, tokens, y_ref, cfg["act"])
    gone = np.where(np.all(ids < 0, axis=1))[0]
    if len(gone):
        assert torch.count_nonzero(y[torch.as_tensor(gone, device=y.device)]).item() == 0


def test_capacity_at_least_T_is_dropless(dev):
    """ceil(T k / E * cf) >= T cannot overflow: the call equals the dropless one bit for bit."""
    cfg = case(300, 512, 1024, 8, bias=True)
    inp = _inputs(cfg, dev, seed=12)
    a = _run(_config(cfg, 0.0, DROP, 3), inp)
    for cf, pol in [(4.0, DROP), (1000.0, REROUTE)]:
        b = _run(_config(cfg, cf, pol, 3), inp)
        assert torch.equal(a[0], b[0])
        for u, v in zip(a[1:], b[1:]):
            assert np.array_equal(u, v)


def test_capacity_deterministic_and_paths_agree(dev):
    cfg = case(300, 512, 1024, 8, bias=True)
    inp = _inputs(cfg, dev, seed=13)
    s = _run(_config(cfg, 1.0, REROUTE, 2, moe.GEMM_STREAMING), inp)
    t = _run(_config(cfg, 1.0, REROUTE, 2, moe.GEMM_TILED), inp)
    t2 = _run(_config(cfg, 1.0, REROUTE, 2, moe.GEMM_TILED), inp)
    assert torch.equal(t[0], t2[0]) and np.array_equal(t[1], t2[1])
    assert np.array_equal(s[1], t[1]) and np.array_equal(s[3], t[3])
    err = (s[0].double() - t[0].double()).abs().max() / t[0].double().abs().max()
    assert err < 1e-2
