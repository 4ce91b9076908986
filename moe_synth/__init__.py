"""Seeded synthetic inputs for the MoE-layer forward pass.

This module holds the workload shapes and the input recipe and nothing of the
layer's arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle
consume the same bits produced here.

Recipe (per workload, seed 0 unless stated):
  x  ~ N(0, 1)          [T, d]
  Wg ~ N(0, 1/d)        [d, E]     (gating matrix, d x E row-major)
  W1 ~ N(0, 1/d)        [E, d_ff, d]   (out x in, input dim contiguous)
  W2 ~ N(0, 1/d_ff)     [E, d, d_ff]
  router bias (skewed workloads only): b_e = 2 ln(1/(e+1)), fp32
Each tensor (and each expert of W1/W2) draws from its own torch.Generator whose
seed is a splitmix64 mix of (seed, tensor tag, expert).  Draws are fp32 and are
rounded to nearest-even into the storage dtype.  INT4 experts are drawn the same
way and then quantised per output row in groups of 128 inputs:
  s = bf16(absmax / 7);  q = clamp(round_half_even(w / s), -8, 7);  q = 0 where s == 0
and packed two codes per byte, even input index in the low nibble.
"""
import math

import numpy as np
import torch

F32, BF16, INT4_G128 = 0, 1, 2

# The workloads: name -> shape, dtypes and routing options.
WORKLOADS = {
    # T=64 tokens, d=128, d_ff=512, E=8, top-2 softmax gating, fp32 throughout.
    "tiny-f32-T64-d128-E8": dict(T=64, d=128, d_ff=512, E=8, k=2, act=F32, w=F32,
                                 bias=False, tau=1.0, gumbel=False),
    # Decode, bandwidth-bound: 8 tokens, 128 experts of 8192 x 8192, bf16.
    "decode-bf16-T8-d8192-E128": dict(T=8, d=8192, d_ff=8192, E=128, k=2, act=BF16, w=BF16,
                                      bias=False, tau=1.0, gumbel=False),
    # Prefill with a Zipf-like skew from the router bias: 4096 tokens, 16 experts.
    "prefill-skewed-bf16-T4096-d4096-E16": dict(T=4096, d=4096, d_ff=16384, E=16, k=2, act=BF16,
                                                w=BF16, bias=True, tau=1.0, gumbel=False),
    # Large prefill, many experts, balanced and skewed routing from the same tensors.
    "prefill-balanced-bf16-T2048-d8192-E128": dict(T=2048, d=8192, d_ff=8192, E=128, k=2, act=BF16,
                                                   w=BF16, bias=False, tau=1.0, gumbel=False),
    "prefill-skewed-bf16-T2048-d8192-E128": dict(T=2048, d=8192, d_ff=8192, E=128, k=2, act=BF16,
                                                 w=BF16, bias=True, tau=1.0, gumbel=False),
    # Wide experts stored as INT4 (group 128, bf16 scales), Gumbel top-2 at tau=0.5.
    "int4-decode-T16-d12288-E16": dict(T=16, d=12288, d_ff=49152, E=16, k=2, act=BF16,
                                       w=INT4_G128, bias=False, tau=0.5, gumbel=True),
    "int4-prefill-T8192-d12288-E16": dict(T=8192, d=12288, d_ff=49152, E=16, k=2, act=BF16,
                                          w=INT4_G128, bias=False, tau=0.5, gumbel=True),
}

TAGS = {"x": 1, "Wg": 2, "W1": 3, "W2": 4, "W_in": 5, "b_in": 6}
_MASK = (1 << 64) - 1


def workload(name, **override):
    """A copy of a named workload, with fields overridden (e.g. a smaller T)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    cfg["name"] = name
    return cfg


def _splitmix64(v):
    v = (v + 0x9E3779B97F4A7C15) & _MASK
    v = ((v ^ (v >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    v = ((v ^ (v >> 27)) * 0x94D049BB133111EB) & _MASK
    return v ^ (v >> 31)


def stream_seed(seed, tag, expert=0):
    """Seed of one tensor's (or one expert's) generator; fits torch's int64."""
    v = _splitmix64(_splitmix64(_splitmix64(seed) ^ tag) ^ expert)
    return v & ((1 << 63) - 1)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, device, seed):
    t = torch.randn(shape, dtype=torch.float32, device=device, generator=_gen(device, seed))
    if std != 1.0:
        t.mul_(std)
    return t


def _store(t, dtype):
    return t if dtype == F32 else t.to(torch.bfloat16)


def router_bias(E):
    """b_e = 2 ln(1/(e+1)) for e = 0..E-1 (fp32)."""
    return torch.tensor([2.0 * math.log(1.0 / (e + 1)) for e in range(E)], dtype=torch.float32)


def quantize_int4_g128(w):
    """Symmetric group-128 INT4 codes (packed uint8 [N, K/2]) and bf16 scales [N, K/128]."""
    N, K = w.shape
    assert K % 128 == 0
    g = w.reshape(N, K // 128, 128)
    s = (g.abs().amax(dim=2) / 7.0).to(torch.bfloat16)
    sf = s.to(torch.float32).unsqueeze(2)
    q = torch.where(sf == 0, torch.zeros_like(g), torch.round(g / torch.where(sf == 0, 1.0, sf)))
    q = q.clamp_(-8, 7).to(torch.int16).reshape(N, K)
    nib = (q & 0xF).to(torch.uint8)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return packed.contiguous(), s.contiguous()


def generate_router(cfg, device="cpu", seed=0):
    """The router's inputs alone (the same tensors `generate` returns):
    dict(x [T, d], Wg [d, E], bias [E] or None, W_in, b_in).  With
    cfg["router_hidden"] = d_r > 0 (two-layer router): W_in [d_r, d] ~ N(0, 1/d)
    in the activation dtype, b_in [d_r] fp32 ~ N(0, 0.1^2), and Wg [d_r, E]
    ~ N(0, 1/d_r); otherwise W_in and b_in are None."""
    T, d, E, act = cfg["T"], cfg["d"], cfg["E"], cfg["act"]
    d_r = cfg.get("router_hidden", 0)
    x = _store(_normal((T, d), 1.0, device, stream_seed(seed, TAGS["x"])), act)
    d_g = d_r if d_r else d
    Wg = _store(_normal((d_g, E), 1.0 / math.sqrt(d_g), device, stream_seed(seed, TAGS["Wg"])), act)
    bias = router_bias(E).to(device) if cfg.get("bias") else None
    W_in = b_in = None
    if d_r:
        W_in = _store(_normal((d_r, d), 1.0 / math.sqrt(d), device, stream_seed(seed, TAGS["W_in"])), act)
        b_in = _normal((d_r,), 0.1, device, stream_seed(seed, TAGS["b_in"])).float()
    return dict(x=x, Wg=Wg, bias=bias, W_in=W_in, b_in=b_in)


def generate(cfg, device="cpu", seed=0):
    """All inputs of a workload as torch tensors on `device`.

    Returns dict(x, Wg, bias (or None), W1, W2, S1, S2 (INT4 scales or None)).
    W1 is [E, d_ff, d] (INT4: uint8 [E, d_ff, d/2]); W2 is [E, d, d_ff].  With
    cfg["ffn"] == 2 (SwiGLU experts) W1 has 2 d_ff rows, drawn like any other
    (the gate/up interleave is a storage order, not a distribution).
    """
    T, d, d_ff, E = cfg["T"], cfg["d"], cfg["d_ff"], cfg["E"]
    wdt = cfg["w"]
    out = generate_router(cfg, device, seed)
    out.update(S1=None, S2=None)
    n1 = 2 * d_ff if cfg.get("ffn", 0) == 2 else d_ff
    for name, N, K in (("W1", n1, d), ("W2", d, d_ff)):
        std = 1.0 / math.sqrt(K)
        if wdt == INT4_G128:
            codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((E, N, K // 128), dtype=torch.bfloat16, device=device)
            for e in range(E):
                w = _normal((N, K), std, device, stream_seed(seed, TAGS[name], e))
                codes[e], scales[e] = quantize_int4_g128(w)
                del w
            out[name] = codes
            out["S1" if name == "W1" else "S2"] = scales
        else:
            W = torch.empty((E, N, K), dtype=torch.float32 if wdt == F32 else torch.bfloat16,
                            device=device)
            for e in range(E):
                W[e] = _store(_normal((N, K), std, device, stream_seed(seed, TAGS[name], e)), wdt)
            out[name] = W
    return out


def to_bits(t):
    """A torch tensor as the numpy array the oracle reads (bf16 -> uint16 bits)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().contiguous().numpy()

