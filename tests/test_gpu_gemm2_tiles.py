"""GPU check of the bf16 tiled grouped GEMM2 (moe_grouped_gemm, which = 2:
fp32 Y = A . W_e^T per dispatch row, no activation) against the oracle's
binary64 products, element by element (P3 §3.2: each expert is its own
linear map; P3 §4.2: the per-expert work is a grouped GEMM over the rows
dispatched to it).

bf16 inputs are exact in binary64, so the only difference from the oracle is
the fp32 accumulation: per element |Y - Y_ref| <= K 2^-23 sum_i |w_i x_i|.

Experts hold 300, 200, 140, 130, 40 and 0 rows: 256-row tiles (full and
partial, the two-group schedule), the 128- and 64-row tiles, and an empty
expert.  K runs over one, two, three and sixteen 64-wide stages (the short
ranges exercise the schedule's prologue and last waits, one K range as the
stage entry point launches it); N = 320 leaves a 64-row weight tile."""
import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import npref

pytestmark = pytest.mark.gpu

N = 320
COUNTS = [300, 200, 140, 130, 40, 0]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.binding.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("K", [64, 128, 192, 1024])
def test_gemm2_tiles(dev, oracle, K):
    E = len(COUNTS)
    rows = sum(COUNTS)
    rng = np.random.default_rng(K)
    W = torch.from_numpy((rng.standard_normal((E, N, K)) / np.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
    A = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    offsets = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    c = moe.config(rows // 2, N, K, E, 2, moe.BF16, moe.BF16, gemm_path=moe.GEMM_TILED)
    Y = torch.full((rows, N), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_grouped_gemm(c, 2, A.to(dev), None, torch.from_numpy(offsets).to(dev), W.to(dev), None, Y)
    torch.cuda.synchronize()
    Y = Y.cpu().double().numpy()
    Ab = moe_synth.to_bits(A)
    Wb = moe_synth.to_bits(W)
    worst = 0.0
    for e in range(E):
        We = Wb[e]
        Wf = np.abs(npref.bf16_bits_to_f64(We))
        for s in range(int(offsets[e]), int(offsets[e + 1])):
            x = npref.bf16_bits_to_f64(Ab[s])
            ref = oracle.expert_linear(x, We, moe.BF16)
            bound = K * 2.0 ** -23 * (Wf @ np.abs(x))
            err = np.abs(Y[s] - ref)
            assert np.all(np.isfinite(Y[s])), f"K {K} row {s} (expert {e}): non-finite output"
            j = int(np.argmax(err - bound))
            assert np.all(err <= bound), f"K {K} row {s} (expert {e}) col {j}: {Y[s, j]} vs {ref[j]}"
            worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
    print(f"\nK {K}: worst error / fp32 bound {worst:.3f}")
