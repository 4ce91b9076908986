"""Independent numpy/scipy formulations used to pin the oracle on tiny inputs.

These are deliberately *different algorithms* from the oracle's loops: library
matmuls over every expert followed by a mask (the dense formulation), library
softmax, library stable sorts and library normal CDFs.  None of this is used by
the GPU path.
"""
import itertools

import numpy as np
from scipy import special, stats


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a):
    """Round-to-nearest-even of float64 values (exactly representable in fp32) to bf16 bits."""
    f = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (f >> 16) & 1
    return ((f + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f64_to_bf16_nearest(a):
    """bf16 bits of the bf16 value nearest to each float64 (ties to the even code),
    chosen by comparing the distances to the neighbouring bf16 values in float64."""
    shape = np.shape(a)
    a = np.asarray(a, dtype=np.float64).ravel()
    guess = f64_to_bf16_bits(a).astype(np.int64)
    out = np.empty(len(a), dtype=np.uint16)
    for i, (v, g) in enumerate(zip(a, guess)):
        cands = [c for c in (g - 1, g, g + 1) if 0 <= c <= 0xFFFF and ((c >> 15) == (g >> 15))]
        vals = bf16_bits_to_f64(np.array(cands, dtype=np.uint16))
        dist = np.abs(vals - v)
        best = np.flatnonzero(dist == dist.min())
        pick = [cands[j] for j in best]
        out[i] = pick[0] if len(pick) == 1 else [c for c in pick if c % 2 == 0][0]
    return out.reshape(shape)


def unpack_int4(codes):
    """Signed INT4 codes [..., K] from packed bytes [..., K/2] (even index in the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    q = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    return np.where(q >= 8, q - 16, q).astype(np.int64)


def pack_int4(q):
    q = np.asarray(q, dtype=np.int64)
    nib = (q & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def dequant_int4(codes, scales_bits):
    q = unpack_int4(codes).astype(np.float64)
    s = bf16_bits_to_f64(scales_bits)
    return q * np.repeat(s, 128, axis=-1)


def gelu_cdf(h):
    """h * Phi(h) with Phi the library standard-normal CDF."""
    return h * stats.norm.cdf(h)


def topk_lexsort(z, k):
    """Top-k by a library lexicographic sort on (-z, index); NaN last."""
    T, E = z.shape
    key = np.where(np.isnan(z), np.inf, -z)
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), key[t]))
        ids[t] = order[:k]
    return ids


def topk_bruteforce(z_row, k):
    """The k-subset maximising sum(z) (ties: the lexicographically smallest index set)."""
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(len(z_row)), k):
        s = sum(z_row[list(sub)])
        if s > best_sum:
            best, best_sum = sub, s
    return set(best)


def dense_moe(x, Wg, W1, W2, k, bias=None, tau=1.0, g=None):
    """Dense formulation: run every expert on every token, then mask with the
    top-k softmax gates.  x [T,d], Wg [d,E], W1 [E,d_ff,d], W2 [E,d,d_ff]; float64."""
    l = x @ Wg
    if bias is not None:
        l = l + bias
    if g is not None:
        l = l + g
    z = l / tau
    p = special.softmax(z, axis=1)
    ids = topk_lexsort(z, k)
    E = Wg.shape[1]
    mask = np.zeros_like(p)
    for j in range(k):
        mask[np.arange(len(x)), ids[:, j]] = 1.0
    H = np.einsum("end,td->ten", W1, x)           # [T, E, d_ff]
    O = np.einsum("edn,ten->ted", W2, gelu_cdf(H))  # [T, E, d]
    y = np.einsum("te,ted->td", mask * p, O)
    return dict(y=y, ids=ids, z=z, p=p, gate_p=np.take_along_axis(p, ids, axis=1))
