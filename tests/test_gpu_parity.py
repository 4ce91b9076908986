"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles and ragged tails, plus edge cases."""
import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

F32, BF16, INT4 = moe.F32, moe.BF16, moe.INT4_G128


def case(T, d, d_ff, E, k=2, act=BF16, w=BF16, bias=False, tau=1.0, gumbel=False, gate_norm=0, noise=0.0, ffn=0):
    return dict(T=T, d=d, d_ff=d_ff, E=E, k=k, act=act, w=w, bias=bias, tau=tau, gumbel=gumbel, gate_norm=gate_norm,
                noise=noise, ffn=ffn, name="case")


SILU, SWIGLU = moe.ACT_SILU, moe.ACT_SWIGLU


ROUTER_CASES = {
    "tiny-f32-T64-E8": case(64, 128, 512, 8, act=F32, w=F32),
    "bf16-T200-d512-E128": case(200, 512, 64, 128),
    "bf16-T333-d1024-E16-bias": case(333, 1024, 64, 16, bias=True),
    "bf16-T77-d768-E16-gumbel-tau0.5": case(77, 768, 128, 16, w=INT4, tau=0.5, gumbel=True),
    "bf16-T50-d256-E256-k8": case(50, 256, 64, 256, k=8),
    "bf16-T31-d192-E5-k3": case(31, 192, 64, 5, k=3),
    "f32-T40-d64-E1-k1": case(40, 64, 64, 1, k=1, act=F32, w=F32),
    "bf16-T1-d8192-E128": case(1, 8192, 64, 128),
    # fp64-MFMA router (bf16, T >= 64): partial 32-expert blocks, E just past the 16-expert layout, d split unevenly
    "bf16-T130-d640-E40-k3": case(130, 640, 64, 40, k=3),
    "bf16-T70-d448-E17-bias": case(70, 448, 64, 17, bias=True),
    # variants: Gaussian logit noise, renormalised gates, both with Gumbel noise and a temperature
    "bf16-T200-d512-E64-gaussian0.1": case(200, 512, 64, 64, noise=0.1),
    "bf16-T77-d768-E16-gumbel-gaussian0.3-tau0.5-renorm": case(77, 768, 128, 16, tau=0.5, gumbel=True, noise=0.3,
                                                                gate_norm=1),
    "bf16-T50-d256-E256-k8-renorm": case(50, 256, 64, 256, k=8, gate_norm=1),
    "f32-T40-d64-E1-k1-renorm": case(40, 64, 64, 1, k=1, act=F32, w=F32, gate_norm=1),
}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


def _inputs(cfg, dev, seed=0):
    return {k: (v.to(dev) if v is not None else None) for k, v in moe_synth.generate(cfg, "cpu", seed).items()}


@pytest.mark.parametrize("name", list(ROUTER_CASES))
def test_router_parity(dev, oracle, name):
    cfg = ROUTER_CASES[name]
    inp = _inputs(cfg, dev, seed=1)
    c = H.abi_config(cfg, seed=7, token_offset=1000)
    ids = torch.full((cfg["T"], cfg["k"]), -1, dtype=torch.int32, device=dev)
    gates = torch.zeros((cfg["T"], cfg["k"]), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    moe.moe_router(c, inp["x"], inp["Wg"], inp["bias"], ids, gates, ws)
    torch.cuda.synchronize()
    ref = H.oracle_route(oracle, cfg, inp, noise_seed=7, token_offset=1000)
    amb = H.check_routing(ids.cpu().numpy(), gates.cpu().numpy(), ref, cfg["k"])
    assert len(amb) == 0 or len(amb) < cfg["T"] // 100 + 1


def _random_ids(rng, T, E, k, skew=None):
    if skew == "one":
        base = np.arange(k)[None, :].repeat(T, 0)
        return base.astype(np.int32)
    out = np.empty((T, k), dtype=np.int32)
    p = None
    if skew == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False, p=p)
    return out


PERMUTE_CASES = [(64, 8, 2, None), (333, 16, 2, "zipf"), (50, 256, 8, None), (1, 1, 1, None), (8192, 16, 2, "zipf"),
                 (1000, 128, 2, None), (97, 7, 3, "one"), (4097, 256, 4, "zipf")]


@pytest.mark.parametrize("T,E,k,skew", PERMUTE_CASES, ids=[f"T{c[0]}-E{c[1]}-k{c[2]}-{c[3]}" for c in PERMUTE_CASES])
def test_permute_parity(dev, oracle, T, E, k, skew):
    rng = np.random.default_rng(T * 1000 + E)
    ids_h = _random_ids(rng, T, E, k, skew)
    c = moe.config(T, 64, 64, E, k, BF16, BF16)
    ids = torch.from_numpy(ids_h).to(dev)
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    sorted_token = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    pos = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    moe.moe_permute(c, ids, counts, offsets, sorted_token, pos)
    torch.cuda.synchronize()
    H.check_dispatch(oracle, ids_h, E, counts.cpu().numpy(), offsets.cpu().numpy(), sorted_token.cpu().numpy(),
                     pos.cpu().numpy())


def test_permute_empty(dev):
    c = moe.config(0, 64, 64, 9, 2, BF16, BF16)
    counts = torch.full((9,), 5, dtype=torch.int32, device=dev)
    offsets = torch.full((10,), 5, dtype=torch.int32, device=dev)
    moe.moe_permute(c, None, counts, offsets, None, None)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 9 and offsets.cpu().tolist() == [0] * 10


FORWARD_CASES = {
    # name: (config, paths)
    "tiny-f32-T64-d128-E8": (moe_synth.workload("tiny-f32-T64-d128-E8"), [moe.GEMM_AUTO]),
    "bf16-T16-d512-dff1024-E8": (case(16, 512, 1024, 8), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    # the automatic choice on both sides of its threshold (streaming up to 16 tokens, tiled above), and one token
    "bf16-T17-d512-dff1024-E8": (case(17, 512, 1024, 8), [moe.GEMM_AUTO]),
    "bf16-T1-d512-dff1024-E8": (case(1, 512, 1024, 8), [moe.GEMM_AUTO]),
    # GEMM2's K range shorter than one streaming stage, so one of the layer's two K halves is empty
    "bf16-T8-d256-dff64-E4": (case(8, 256, 64, 4), [moe.GEMM_STREAMING]),
    "int4-T6-d256-dff128-E4": (case(6, 256, 128, 4, w=INT4), [moe.GEMM_STREAMING]),
    "bf16-T300-d512-dff1024-E8-skewed": (case(300, 512, 1024, 8, bias=True), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "bf16-T150-d320-dff576-E6-ntail": (case(150, 320, 576, 6), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    # N tails (576 = 2 x 256 + 64 for W1, 320 for W2) on every tiled tile height: 256-, 128- and 64-row tiles
    "bf16-T300-d320-dff576-E8-skewed-ntail": (case(300, 320, 576, 8, bias=True), [moe.GEMM_TILED]),
    "bf16-T40-d256-dff256-E256-k8": (case(40, 256, 256, 256, k=8), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    # short GEMM2 K ranges on 256-row tiles (the two-group schedule's prologue and last waits): K = 64 (one
    # stage), 128 (two K halves of one stage in the layer), 192 (three stages), 384 (halves of three stages,
    # with N = 320 leaving a 64-row weight tile)
    "bf16-T600-d256-dff64-E3": (case(600, 256, 64, 3), [moe.GEMM_TILED]),
    "bf16-T600-d256-dff128-E3-skewed": (case(600, 256, 128, 3, bias=True), [moe.GEMM_TILED]),
    "bf16-T600-d192-dff192-E3": (case(600, 192, 192, 3), [moe.GEMM_TILED]),
    "bf16-T640-d320-dff384-E2-skewed": (case(640, 320, 384, 2, bias=True), [moe.GEMM_TILED]),
    "bf16-T9-d256-dff512-E1-k1": (case(9, 256, 512, 1, k=1), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    # streaming with 32-row (T <= 32) and 64-row dispatch tiles
    "bf16-T24-d512-dff1024-E4": (case(24, 512, 1024, 4), [moe.GEMM_STREAMING]),
    "int4-T30-d512-dff1024-E8": (case(30, 512, 1024, 8, w=INT4), [moe.GEMM_STREAMING]),
    "int4-T12-d512-dff1024-E8-gumbel": (case(12, 512, 1024, 8, w=INT4, tau=0.5, gumbel=True), [moe.GEMM_AUTO]),
    # K tails in the streaming INT4 kernel: 5 and 9 scale groups, so the last 256-byte stage is partial
    "int4-T30-d640-dff1152-E8": (case(30, 640, 1152, 8, w=INT4), [moe.GEMM_STREAMING]),
    # the same K tails with 16-row dispatch tiles (T <= 16): activations loaded ahead, permuted-K dequantisation,
    # an odd number of scale groups per row (scales read one by one)
    "int4-T12-d640-dff1152-E8": (case(12, 640, 1152, 8, w=INT4), [moe.GEMM_STREAMING]),
    "int4-T5-d1152-dff640-E4-k1": (case(5, 1152, 640, 4, k=1, w=INT4), [moe.GEMM_STREAMING]),
    # 16-row dispatch tiles with K a multiple of 256 (the LDS-ring kernel): K = 5120 gives every wavefront
    # five stages (one full turn of the ring, then one), K = 2304 gives 2, 2, 2 and 3; SwiGLU on the same path
    "int4-T16-d5120-dff2304-E8": (case(16, 5120, 2304, 8, w=INT4), [moe.GEMM_STREAMING]),
    "int4-T7-d2304-dff5120-E8-swiglu": (case(7, 2304, 5120, 8, w=INT4, ffn=SWIGLU), [moe.GEMM_STREAMING]),
    "int4-T200-d384-dff768-E8-gumbel": (case(200, 384, 768, 8, w=INT4, tau=0.5, gumbel=True), [moe.GEMM_AUTO]),
    # K = 1024 and 3072: one and three 32-stage scale blocks; skewed rows exercise all three tile heights
    "int4-T200-d1024-dff3072-E8-skewed": (case(200, 1024, 3072, 8, w=INT4, bias=True),
                                          [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "int4-T40-d1024-dff1024-E64-k8": (case(40, 1024, 1024, 64, k=8, w=INT4), [moe.GEMM_TILED]),
    "f32-T130-d192-dff320-E5-k3": (case(130, 192, 320, 5, k=3, act=F32, w=F32, bias=True), [moe.GEMM_AUTO]),
    # router variants through the whole layer
    "bf16-T300-d512-dff1024-E8-renorm-gaussian0.1": (case(300, 512, 1024, 8, bias=True, gate_norm=1, noise=0.1),
                                                     [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "int4-T12-d512-dff1024-E8-renorm-gumbel": (case(12, 512, 1024, 8, w=INT4, tau=0.5, gumbel=True, gate_norm=1),
                                               [moe.GEMM_AUTO]),
    "f32-T64-d128-dff256-E6-k3-renorm": (case(64, 128, 256, 6, k=3, act=F32, w=F32, gate_norm=1), [moe.GEMM_AUTO]),
    # expert activations: SiLU and SwiGLU on every kernel (streaming with 16-, 32- and 64-row tiles, tiled with
    # its three tile heights, INT4 on both, fp32)
    "bf16-T300-d512-dff1024-E8-skewed-silu": (case(300, 512, 1024, 8, bias=True, ffn=SILU),
                                              [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "bf16-T300-d512-dff1024-E8-skewed-swiglu": (case(300, 512, 1024, 8, bias=True, ffn=SWIGLU),
                                                [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "bf16-T12-d512-dff1024-E8-swiglu": (case(12, 512, 1024, 8, ffn=SWIGLU), [moe.GEMM_STREAMING]),
    "bf16-T10-d512-dff1024-E8-silu": (case(10, 512, 1024, 8, ffn=SILU), [moe.GEMM_STREAMING]),
    "bf16-T24-d512-dff1024-E4-swiglu": (case(24, 512, 1024, 4, ffn=SWIGLU), [moe.GEMM_STREAMING]),
    "bf16-T150-d320-dff576-E6-ntail-swiglu": (case(150, 320, 576, 6, ffn=SWIGLU), [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "int4-T200-d1024-dff1024-E8-skewed-swiglu": (case(200, 1024, 1024, 8, w=INT4, bias=True, ffn=SWIGLU),
                                                 [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "int4-T200-d1024-dff1024-E8-skewed-silu": (case(200, 1024, 1024, 8, w=INT4, bias=True, ffn=SILU),
                                               [moe.GEMM_STREAMING, moe.GEMM_TILED]),
    "int4-T12-d512-dff1024-E8-swiglu": (case(12, 512, 1024, 8, w=INT4, ffn=SWIGLU), [moe.GEMM_AUTO]),
    "f32-T130-d192-dff320-E5-k3-swiglu": (case(130, 192, 320, 5, k=3, act=F32, w=F32, ffn=SWIGLU), [moe.GEMM_AUTO]),
    "f32-T64-d128-dff256-E6-silu": (case(64, 128, 256, 6, act=F32, w=F32, ffn=SILU), [moe.GEMM_AUTO]),
}
FORWARD_PARAMS = [(n, p) for n, (_, paths) in FORWARD_CASES.items() for p in paths]


@pytest.mark.parametrize("name,path", FORWARD_PARAMS, ids=[f"{n}-path{p}" for n, p in FORWARD_PARAMS])
def test_forward_parity(dev, oracle, name, path):
    cfg = FORWARD_CASES[name][0]
    inp = _inputs(cfg, dev, seed=3)
    out = H.run_forward(cfg, inp, gemm_path=path, noise_seed=5)
    ref = H.oracle_route(oracle, cfg, inp, noise_seed=5)
    ids = out["ids"].cpu().numpy()
    amb = H.check_routing(ids, out["gates"].cpu().numpy(), ref, cfg["k"])
    H.check_forward_counts(oracle, ref["ids"], ids, amb, cfg["E"], out["counts"].cpu().numpy())
    assert int(out["counts"].sum()) == cfg["T"] * cfg["k"]
    tokens = np.array([t for t in range(cfg["T"]) if t not in amb], dtype=np.int64)
    y_ref = H.oracle_y(oracle, cfg, inp, ref, tokens)
    H.check_y(out["y"], tokens, y_ref, cfg["act"])


def test_empty_batch(dev):
    cfg = case(0, 256, 512, 8)
    c = H.abi_config(cfg)
    counts = torch.full((8,), 3, dtype=torch.int32, device=dev)
    moe.moe_forward(c, None, None, None, None, None, None, None, None, None, None, counts, None, W1_stride=0,
                    W2_stride=0)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8


def test_deterministic_repeats(dev):
    cfg = case(300, 512, 1024, 8, bias=True)
    inp = _inputs(cfg, dev, seed=4)
    c = H.abi_config(cfg, gemm_path=moe.GEMM_TILED)
    layer = moe.MoELayerForward(c, device=dev)
    first = [t.clone() for t in layer(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W2"])]
    for _ in range(5):
        again = layer(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W2"])
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("w", [BF16, INT4], ids=["bf16", "int4"])
def test_paths_agree(dev, w):
    """The streaming and tiled kernels compute the same function (to fp32
    rounding; INT4: the tiled kernel rounds each q * s to bf16)."""
    cfg = case(64, 1024, 2048, 8, w=w)
    inp = _inputs(cfg, dev, seed=6)
    a = H.run_forward(cfg, inp, gemm_path=moe.GEMM_STREAMING)
    b = H.run_forward(cfg, inp, gemm_path=moe.GEMM_TILED)
    assert torch.equal(a["ids"], b["ids"])
    err = (a["y"].double() - b["y"].double()).abs().max() / b["y"].double().abs().max()
    assert err < 1e-2
