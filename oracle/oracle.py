"""ctypes wrapper around the plain C oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU product path never imports this
module.  Arrays cross as numpy arrays: fp32 as float32, bf16 as their raw
uint16 bit patterns, INT4 codes as uint8 (two codes per byte, even column in the
low nibble) with bf16 scales as uint16.
"""
import ctypes
import os
import subprocess

import numpy as np

F32, BF16, INT4_G128 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

# -ffp-contract=off: every product and sum rounds on its own, as written.
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def build(src=_SRC, out=_LIB, extra=()):
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U64 = ctypes.c_uint64


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path=_LIB):
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_philox4x64_10.argtypes = [_P, _P, _P]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_uniform.argtypes = [_U64, _U64, _U64]
        lib.oracle_uniform.restype = ctypes.c_double
        lib.oracle_gumbel.argtypes = [_U64, _U64, _U64]
        lib.oracle_gumbel.restype = ctypes.c_double
        lib.oracle_normal.argtypes = [_U64, _U64, _U64]
        lib.oracle_normal.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_route.argtypes = [_I64, _I64, _I32, _I32, _I32, _P, _P, _P,
                                     ctypes.c_double, _I32, _U64, _U64, _P, _P, _P, _P, _P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_router_encoder.argtypes = [_I64, _I64, _I64, _I32, _P, _P, _P, _P]
        lib.oracle_router_encoder.restype = ctypes.c_int
        lib.oracle_route_ex.argtypes = [_I64, _I64, _I32, _I32, _I32, _P, _P, _P, ctypes.c_double, _I32,
                                        ctypes.c_double, _I32, _U64, _U64, _P, _P, _P, _P, _P]
        lib.oracle_route_ex.restype = ctypes.c_int
        lib.oracle_permute.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P]
        lib.oracle_permute.restype = ctypes.c_int
        lib.oracle_router_stats.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P]
        lib.oracle_router_stats.restype = ctypes.c_int
        lib.oracle_capacity.argtypes = [_I64, _I32, _I32, ctypes.c_double]
        lib.oracle_capacity.restype = ctypes.c_int64
        lib.oracle_capacity_dispatch.argtypes = [_I64, _I32, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P]
        lib.oracle_capacity_dispatch.restype = ctypes.c_int
        lib.oracle_expert_ffn.argtypes = [_I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]
        lib.oracle_expert_ffn.restype = ctypes.c_int
        lib.oracle_expert_linear.argtypes = [_I64, _I64, _I32, _P, _P, _P, _P]
        lib.oracle_expert_linear.restype = ctypes.c_int
        lib.oracle_forward_tokens.argtypes = [_I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _P,
                                              _P, _P, _P, _P, _P, _P, _I64, _P, _P]
        lib.oracle_forward_tokens.restype = ctypes.c_int
        self.lib = lib

    # -- primitives -----------------------------------------------------------
    def philox(self, ctr, key):
        c = np.ascontiguousarray(ctr, dtype=np.uint64)
        k = np.ascontiguousarray(key, dtype=np.uint64)
        out = np.zeros(4, dtype=np.uint64)
        self.lib.oracle_philox4x64_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
        return out

    def uniform(self, seed, token, expert):
        return self.lib.oracle_uniform(seed, token, expert)

    def gumbel(self, seed, token, expert):
        return self.lib.oracle_gumbel(seed, token, expert)

    def normal(self, seed, token, expert):
        return self.lib.oracle_normal(seed, token, expert)

    def silu(self, a):
        return self.lib.oracle_silu(float(a))

    def gelu(self, h):
        return self.lib.oracle_gelu(float(h))

    # -- routing ----------------------------------------------------------------
    def router_encoder(self, x, W_in, b_in, act_dtype):
        """Hidden layer of the two-layer router: GeLU(x W_in^T + b_in) in act_dtype
        (float32, or bf16 bits as uint16), [T, d_r]."""
        x = np.ascontiguousarray(x)
        W_in = np.ascontiguousarray(W_in)
        T, d = x.shape
        d_r = W_in.shape[0]
        assert W_in.shape[1] == d
        b = None if b_in is None else np.ascontiguousarray(b_in, dtype=np.float32)
        h = np.zeros((T, d_r), dtype=np.float32 if act_dtype == F32 else np.uint16)
        rc = self.lib.oracle_router_encoder(T, d, d_r, act_dtype, x.ctypes.data, W_in.ctypes.data,
                                            None if b is None else b.ctypes.data, h.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_router_encoder rejected its arguments")
        return h

    def route(self, x, Wg, k, act_dtype, bias=None, tau=1.0, use_gumbel=False, seed=0,
              token_offset=0, want_zp=False, noise_std=0.0, gate_norm=0, encoder=None):
        """Returns dict(ids[T,k] int32, gates[T,k] float32, gate_p[T,k] float64 [, z, p]).
        noise_std: sigma of the Gaussian logit noise; gate_norm=1: gates renormalised over the k chosen.
        encoder=(W_in, b_in): two-layer router; Wg is then the second layer [d_r, E] and the
        result also holds the hidden layer "h"."""
        hidden = None
        if encoder is not None:
            hidden = self.router_encoder(x, encoder[0], encoder[1], act_dtype)
            x = hidden
        x = np.ascontiguousarray(x)
        Wg = np.ascontiguousarray(Wg)
        T, d = x.shape
        E = Wg.shape[1]
        assert Wg.shape[0] == d
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        ids = np.zeros((T, k), dtype=np.int32)
        gates = np.zeros((T, k), dtype=np.float32)
        gate_p = np.zeros((T, k), dtype=np.float64)
        z = np.zeros((T, E), dtype=np.float64) if want_zp else None
        p = np.zeros((T, E), dtype=np.float64) if want_zp else None
        rc = self.lib.oracle_route_ex(T, d, E, k, act_dtype, x.ctypes.data, Wg.ctypes.data,
                                      None if b is None else b.ctypes.data, float(tau),
                                      int(bool(use_gumbel)), float(noise_std), int(gate_norm), seed, token_offset,
                                      ids.ctypes.data, gates.ctypes.data, gate_p.ctypes.data,
                                      None if z is None else z.ctypes.data,
                                      None if p is None else p.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_route rejected its arguments")
        out = dict(ids=ids, gates=gates, gate_p=gate_p)
        if want_zp:
            out.update(z=z, p=p)
        if hidden is not None:
            out["h"] = hidden
        return out

    def permute(self, ids, E):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, k = ids.shape
        counts = np.zeros(E, dtype=np.int32)
        offsets = np.zeros(E + 1, dtype=np.int32)
        sorted_token = np.zeros(T * k, dtype=np.int32)
        pos = np.zeros((T, k), dtype=np.int32)
        rc = self.lib.oracle_permute(T, E, k, ids.ctypes.data, counts.ctypes.data,
                                     offsets.ctypes.data, sorted_token.ctypes.data, pos.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_permute: expert id out of range")
        return dict(counts=counts, offsets=offsets, sorted_token=sorted_token, pos=pos)

    def capacity(self, T, E, k, capacity_factor):
        """ceil(T k / E * capacity_factor) in binary64."""
        return int(self.lib.oracle_capacity(T, E, k, float(capacity_factor)))

    def capacity_dispatch(self, route, capacity_factor, policy):
        """Capacity-limited dispatch of a routing made with want_zp=True.  policy 0 drops
        overflow, 1 reroutes it.  Returns dict(ids (-1 = dropped), gates, gate_p, counts, cap)."""
        ids = np.ascontiguousarray(route["ids"], dtype=np.int32).copy()
        z = np.ascontiguousarray(route["z"], dtype=np.float64)
        p = np.ascontiguousarray(route["p"], dtype=np.float64)
        T, k = ids.shape
        E = z.shape[1]
        cap = self.capacity(T, E, k, capacity_factor)
        gates = np.zeros((T, k), dtype=np.float32)
        gate_p = np.zeros((T, k), dtype=np.float64)
        counts = np.zeros(E, dtype=np.int32)
        rc = self.lib.oracle_capacity_dispatch(T, E, k, cap, policy, z.ctypes.data, p.ctypes.data, ids.ctypes.data,
                                               gates.ctypes.data, gate_p.ctypes.data, counts.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_capacity_dispatch rejected its arguments")
        return dict(ids=ids, gates=gates, gate_p=gate_p, counts=counts, cap=cap)

    def router_stats(self, ids, p):
        """Routing statistics from ids [T,k] and full softmax rows p [T,E] (binary64):
        dict(fraction[E], mean_prob[E], entropy, lb_fraction, lb_prob, fraction_std, lb_product)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        p = np.ascontiguousarray(p, dtype=np.float64)
        T, k = ids.shape
        E = p.shape[1]
        fraction = np.zeros(E, dtype=np.float64)
        mean_prob = np.zeros(E, dtype=np.float64)
        scalars = np.zeros(5, dtype=np.float64)
        rc = self.lib.oracle_router_stats(T, E, k, ids.ctypes.data, p.ctypes.data, fraction.ctypes.data,
                                          mean_prob.ctypes.data, scalars.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_router_stats rejected its arguments")
        return dict(fraction=fraction, mean_prob=mean_prob, entropy=scalars[0], lb_fraction=scalars[1],
                    lb_prob=scalars[2], fraction_std=scalars[3], lb_product=scalars[4], scalars=scalars)

    # -- experts ------------------------------------------------------------------
    def expert_ffn(self, xr, W1e, W2e, w_dtype, S1e=None, S2e=None, act=0):
        """o = W2e . act(W1e . xr) in binary64 for one float64 row xr (act 0 GeLU, 1 SiLU,
        2 SwiGLU with W1e's 2 d_ff rows interleaved in blocks of 16: gate, then up)."""
        xr = np.ascontiguousarray(xr, dtype=np.float64)
        d = xr.shape[0]
        d_ff = W1e.shape[0] // (2 if act == 2 else 1)
        W1e = np.ascontiguousarray(W1e)
        W2e = np.ascontiguousarray(W2e)
        S1e = None if S1e is None else np.ascontiguousarray(S1e)
        S2e = None if S2e is None else np.ascontiguousarray(S2e)
        o = np.zeros(d, dtype=np.float64)
        rc = self.lib.oracle_expert_ffn(d, d_ff, w_dtype, act, xr.ctypes.data, W1e.ctypes.data,
                                        None if S1e is None else S1e.ctypes.data,
                                        W2e.ctypes.data,
                                        None if S2e is None else S2e.ctypes.data, o.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_expert_ffn rejected its arguments")
        return o

    def expert_linear(self, xr, We, w_dtype, Se=None):
        """out = We . xr in binary64 for one float64 row xr of length K; We is
        [N, K] (float32, bf16 bits, or INT4 codes [N, K/2] with bf16 scales Se [N, K/128])."""
        xr = np.ascontiguousarray(xr, dtype=np.float64)
        K = xr.shape[0]
        We = np.ascontiguousarray(We)
        Se = None if Se is None else np.ascontiguousarray(Se)
        N = We.shape[0]
        out = np.zeros(N, dtype=np.float64)
        rc = self.lib.oracle_expert_linear(N, K, w_dtype, xr.ctypes.data, We.ctypes.data,
                                           None if Se is None else Se.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_expert_linear rejected its arguments")
        return out

    def forward_tokens(self, x, ids, gate_p, W1, W2, act_dtype, w_dtype, d_ff, tokens,
                       S1=None, S2=None, act=0):
        """y rows (float64) for the listed tokens.  W1/W2/S1/S2 map expert -> numpy
        array (a list of length E, entries may be None for untouched experts)."""
        x = np.ascontiguousarray(x)
        T, d = x.shape
        k = ids.shape[1]
        E = len(W1)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        gate_p = np.ascontiguousarray(gate_p, dtype=np.float64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        keep = []  # hold contiguous copies alive through the call

        def ptrs(arrs):
            if arrs is None:
                return None
            a = (ctypes.c_void_p * E)()
            for e, m in enumerate(arrs):
                if m is not None:
                    m = np.ascontiguousarray(m)
                    keep.append(m)
                    a[e] = m.ctypes.data
            keep.append(a)
            return a

        p1, p2, s1, s2 = ptrs(W1), ptrs(W2), ptrs(S1), ptrs(S2)
        y = np.zeros((len(tokens), d), dtype=np.float64)
        rc = self.lib.oracle_forward_tokens(T, d, d_ff, E, k, act_dtype, w_dtype, act, x.ctypes.data,
                                            ids.ctypes.data, gate_p.ctypes.data, p1, s1, p2, s2,
                                            len(tokens), tokens.ctypes.data, y.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_forward_tokens rejected its arguments")
        return y

    def forward(self, x, Wg, W1, W2, k, act_dtype, w_dtype, bias=None, tau=1.0,
                use_gumbel=False, seed=0, token_offset=0, S1=None, S2=None, tokens=None, act=0):
        """Whole layer: routing for every token, dispatch arrays, and y for the
        listed tokens (all tokens by default).  W1/W2 are [E, N, K] arrays or
        per-expert lists."""
        r = self.route(x, Wg, k, act_dtype, bias=bias, tau=tau, use_gumbel=use_gumbel,
                       seed=seed, token_offset=token_offset)
        E = Wg.shape[1]
        r.update(self.permute(r["ids"], E))
        T = x.shape[0]
        if tokens is None:
            tokens = np.arange(T)
        d_ff = (W1[0].shape[0] if not isinstance(W1, np.ndarray) else W1.shape[1]) // (2 if act == 2 else 1)
        as_list = (lambda a: None if a is None else [a[e] for e in range(E)])
        r["y"] = self.forward_tokens(x, r["ids"], r["gate_p"], as_list(W1), as_list(W2),
                                     act_dtype, w_dtype, d_ff, tokens,
                                     S1=as_list(S1), S2=as_list(S2), act=act)
        r["tokens"] = np.asarray(tokens)
        return r


_default = None


def get():
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
