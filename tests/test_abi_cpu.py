"""The C-ABI library on the CPU: it loads, exports every function include/moe.h
declares, and its host-side checks return the documented status codes before
anything is enqueued (no GPU is touched: every call here is rejected early or
is a pure size query)."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_synth
import sparse_mixture_experts_03_amd as moe
from sparse_mixture_experts_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run __graft_entry__.build())")
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_no_undefined_library_symbols():
    """Every symbol of the library's own namespace is defined in it: a kernel
    whose launch stub the compiler's host pass failed to emit builds and links
    (as an undefined symbol of the shared library) but cannot be loaded."""
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run __graft_entry__.build())")
    r = subprocess.run(["nm", "-D", "--undefined-only", binding.LIB_PATH], capture_output=True, text=True, check=True)
    own = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN3moe" in l or "moe_" in l]
    assert own == [], own


def test_config_struct_layout(tmp_path):
    """The ctypes mirror of moe_config matches the C compiler's layout."""
    fields = [f for f, _ in binding.MoeConfig._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"moe.h\"\nint main(void){\n"
                   f'printf("%zu\\n", sizeof(moe_config));\n'
                   + "".join(f'printf("%zu\\n", offsetof(moe_config, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(binding.MoeConfig)
    assert got[1:] == [getattr(binding.MoeConfig, f).offset for f in fields]


def test_status_strings(lib):
    for s, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                    (3, "workspace too small"), (4, "HIP launch failed")]:
        assert binding.status_string(s) == text


def _cfg(**kw):
    base = dict(T=8, d=256, d_ff=512, E=8, k=2, act_dtype=moe.BF16, w_dtype=moe.BF16)
    base.update(kw)
    c = moe.config(base["T"], base["d"], base["d_ff"], base["E"], base["k"], base["act_dtype"], base["w_dtype"])
    for key in ("tau", "use_gumbel", "gemm_path", "reserved", "capacity_factor", "capacity_policy", "gate_norm",
                "noise_std", "expert_act", "router_hidden"):
        if key in kw:
            setattr(c, key, kw[key])
    return c


BAD = [
    dict(T=-1), dict(T=(1 << 24) + 1), dict(E=0), dict(E=257), dict(k=0), dict(k=9, E=16), dict(k=5, E=4),
    dict(d=100), dict(d_ff=96), dict(d=0), dict(d=1 << 18), dict(tau=0.0), dict(tau=-1.0), dict(tau=float("nan")),
    dict(tau=float("inf")), dict(use_gumbel=2), dict(gemm_path=3), dict(reserved=1), dict(act_dtype=2),
    dict(w_dtype=3), dict(w_dtype=moe.INT4_G128, d=192), dict(w_dtype=moe.INT4_G128, d_ff=320),
    dict(capacity_factor=-1.0), dict(capacity_factor=float("nan")), dict(capacity_factor=float("inf")),
    dict(capacity_factor=-0.0 - 1e-30), dict(capacity_policy=2), dict(capacity_policy=-1),
    dict(capacity_factor=1.25, capacity_policy=7),
    dict(gate_norm=2), dict(gate_norm=-1), dict(noise_std=-0.1), dict(noise_std=float("nan")),
    dict(noise_std=float("inf")), dict(expert_act=3), dict(expert_act=-1), dict(router_hidden=-64),
    dict(router_hidden=100), dict(router_hidden=1 << 18),
]


@pytest.mark.parametrize("kw", BAD, ids=[str(b) for b in BAD])
def test_invalid_config_rejected(lib, kw):
    n = ctypes.c_size_t(12345)
    assert lib.moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert n.value == 12345


def test_unsupported_pairings(lib):
    n = ctypes.c_size_t()
    # renormalised gates are defined over the router's k choices, not over a capacity-limited dispatch
    assert lib.moe_workspace_size(ctypes.byref(_cfg(gate_norm=1, capacity_factor=1.25)), ctypes.byref(n)) == \
        binding.MOE_ERR_UNSUPPORTED
    assert lib.moe_workspace_size(ctypes.byref(_cfg(gate_norm=1, noise_std=0.1)), ctypes.byref(n)) == 0
    for a, w in [(moe.F32, moe.BF16), (moe.BF16, moe.F32), (moe.F32, moe.INT4_G128)]:
        assert lib.moe_workspace_size(ctypes.byref(_cfg(act_dtype=a, w_dtype=w)), ctypes.byref(n)) == \
            binding.MOE_ERR_UNSUPPORTED


def test_int4_tiled_needs_whole_scale_blocks(lib):
    """The tiled kernel takes INT4 weights only when d and d_ff are multiples
    of 1024; an explicit request otherwise is unsupported, the automatic
    choice falls back to the streaming kernel."""
    n = ctypes.c_size_t()
    for d, d_ff, want in [(1024, 3072, 0), (384, 768, binding.MOE_ERR_UNSUPPORTED),
                          (1024, 1536, binding.MOE_ERR_UNSUPPORTED)]:
        c = _cfg(T=512, d=d, d_ff=d_ff, w_dtype=moe.INT4_G128, gemm_path=moe.GEMM_TILED)
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == want, (d, d_ff)
        c = _cfg(T=512, d=d, d_ff=d_ff, w_dtype=moe.INT4_G128, gemm_path=moe.GEMM_AUTO)
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0, (d, d_ff)


def test_int4_tiled_scales_alignment(lib):
    c = _cfg(T=512, d=1024, d_ff=1024, w_dtype=moe.INT4_G128, gemm_path=moe.GEMM_TILED)
    wb = 1024 * 1024 // 2
    assert _forward(lib, c, s1=wb, s2=wb, S1=0xA0008, S2=0xB0000, wsb=1 << 40) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _forward(lib, c, s1=wb, s2=wb, S1=0xA0000, S2=0xB0002, wsb=1 << 40) == binding.MOE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(T=1 << 19, d=4096, k=2),            # Y: 2^19 * 2 * 4096 * 4 bytes = 32 GiB
                                dict(T=1 << 16, d=1024, d_ff=1 << 15, k=2),  # [T*k][d_ff] intermediate = 16 GiB
                                dict(T=64, d=1 << 16, d_ff=1 << 15, w_dtype=moe.BF16)])  # one expert = 4 GiB
def test_arrays_over_4gib_unsupported(lib, kw):
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n)) == binding.MOE_ERR_UNSUPPORTED


def test_workspace_size_accounts_for_buffers(lib):
    n = ctypes.c_size_t()
    c = _cfg(T=4096, d=4096, d_ff=16384, E=16)
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0
    Tk = 4096 * 2
    assert n.value >= Tk * 16384 * 2 + Tk * 4096 * 4 + 2 * Tk * 4 + 17 * 4
    assert n.value % 256 == 0
    assert lib.moe_workspace_size(ctypes.byref(_cfg(T=0)), ctypes.byref(n)) == 0 and n.value == 0
    assert lib.moe_workspace_size(ctypes.byref(c), None) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_workspace_size(None, ctypes.byref(n)) == binding.MOE_ERR_INVALID_ARGUMENT


def test_capacity_workspace(lib):
    """A capacity below T adds the [T][E] binary64 logit and probability rows
    to the workspace; a capacity of at least T (ceil(T k / E * cf) >= T)
    cannot drop anything and adds nothing."""
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    T, E = 2048, 128
    base = _cfg(T=T, d=512, d_ff=512, E=E)
    assert lib.moe_workspace_size(ctypes.byref(base), ctypes.byref(n0)) == 0
    for cf, policy, extra in [(1.25, moe.CAPACITY_DROP, True), (2.0, moe.CAPACITY_REROUTE, True),
                              (64.0, moe.CAPACITY_DROP, False), (1e30, moe.CAPACITY_REROUTE, False),
                              (0.0, moe.CAPACITY_REROUTE, False)]:
        c = _cfg(T=T, d=512, d_ff=512, E=E, capacity_factor=cf, capacity_policy=policy)
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n1)) == 0
        if extra:
            assert n1.value >= n0.value + 2 * T * E * 8, cf
        else:
            assert n1.value == n0.value, cf


def _forward(lib, c, **ptr):
    P = ctypes.c_void_p
    a = dict(x=0x10000, Wg=0x20000, bias=None, W_in=None, b_in=None, W1=0x30000, S1=None, s1=c.d * c.d_ff * 2,
             W2=0x40000, S2=None, s2=c.d * c.d_ff * 2, y=0x50000, ids=0x60000, gates=0x70000, counts=0x80000,
             ws=0x90000, wsb=1 << 40)
    a.update(ptr)
    return lib.moe_forward(ctypes.byref(c), P(a["x"]), P(a["Wg"]), P(a["bias"]), P(a["W_in"]), P(a["b_in"]),
                           P(a["W1"]), P(a["S1"]), a["s1"],
                           P(a["W2"]), P(a["S2"]), a["s2"], P(a["y"]), P(a["ids"]), P(a["gates"]), P(a["counts"]),
                           P(a["ws"]), a["wsb"], P(0))


@pytest.mark.parametrize("bad", [dict(x=None), dict(x=0x10008), dict(Wg=None), dict(y=0x50004), dict(ids=None),
                                 dict(gates=0x70002), dict(counts=None), dict(W1=None), dict(W2=0x40001),
                                 dict(s1=100), dict(s2=256 * 512 * 2 + 8), dict(ws=None), dict(ws=0x90010),
                                 dict(bias=0x1002)])
def test_forward_rejects_bad_pointers(lib, bad):
    assert _forward(lib, _cfg(), **bad) == binding.MOE_ERR_INVALID_ARGUMENT


def test_forward_rejects_small_workspace(lib):
    assert _forward(lib, _cfg(), wsb=1024) == binding.MOE_ERR_WORKSPACE_TOO_SMALL


def test_swiglu_w1_holds_gate_and_up_rows(lib):
    """SwiGLU experts read 2 d_ff rows of W1: a stride of one d_ff x d matrix is too small."""
    c = _cfg(expert_act=moe.ACT_SWIGLU)
    one = 256 * 512 * 2
    assert _forward(lib, c, s1=one) == binding.MOE_ERR_INVALID_ARGUMENT
    assert _forward(lib, c, s1=2 * one, ws=0x90000, wsb=1024) == binding.MOE_ERR_WORKSPACE_TOO_SMALL


def test_router_encoder_workspace(lib):
    """A router encoder of width d_r adds its fp32 pre-activations and act-dtype
    hidden layer [T][d_r] to the router workspace (and so to the layer's)."""
    n0, n1, r0, r1 = (ctypes.c_size_t() for _ in range(4))
    T = 512
    base, enc = _cfg(T=T, d=1024), _cfg(T=T, d=1024, router_hidden=256)
    assert lib.moe_router_workspace_size(ctypes.byref(base), ctypes.byref(r0)) == 0
    assert lib.moe_router_workspace_size(ctypes.byref(enc), ctypes.byref(r1)) == 0
    assert r1.value >= T * 256 * (4 + 2)
    assert lib.moe_workspace_size(ctypes.byref(base), ctypes.byref(n0)) == 0
    assert lib.moe_workspace_size(ctypes.byref(enc), ctypes.byref(n1)) == 0
    assert n1.value >= n0.value - r0.value + r1.value - 256
    assert _forward(lib, enc) == binding.MOE_ERR_INVALID_ARGUMENT            # no W_in
    assert _forward(lib, enc, W_in=0xA0000, wsb=1024) == binding.MOE_ERR_WORKSPACE_TOO_SMALL


def test_int4_needs_scales(lib):
    c = _cfg(w_dtype=moe.INT4_G128)
    assert _forward(lib, c, s1=256 * 512 // 2, s2=256 * 512 // 2) == binding.MOE_ERR_INVALID_ARGUMENT


def test_stage_entry_points_check_arguments(lib):
    P = ctypes.c_void_p
    c = _cfg()
    assert lib.moe_router(ctypes.byref(c), P(0), P(0x1000), None, None, None, P(0x2000), P(0x3000), P(0x4000),
                          1 << 30, P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_router(ctypes.byref(c), P(0x1000), P(0x1000), None, None, None, P(0x2000), P(0x3000), P(0x4000),
                          16, P(0)) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    # encoder weights without an encoder, and an encoder without weights
    assert lib.moe_router(ctypes.byref(c), P(0x1000), P(0x1000), None, P(0x5000), None, P(0x2000), P(0x3000),
                          P(0x4000), 1 << 30, P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    ce = _cfg(router_hidden=64)
    assert lib.moe_router(ctypes.byref(ce), P(0x1000), P(0x1000), None, None, None, P(0x2000), P(0x3000),
                          P(0x4000), 1 << 30, P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_router_encoder(ctypes.byref(c), P(0x1000), P(0x5000), None, P(0x6000), P(0x4000), 1 << 30,
                                  P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_router_encoder(ctypes.byref(ce), P(0x1000), P(0x5000), P(0x7002), P(0x6000), P(0x4000), 1 << 30,
                                  P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_router_encoder(ctypes.byref(ce), P(0x1000), P(0x5000), None, P(0x6000), P(0x4000), 64,
                                  P(0)) == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_permute(ctypes.byref(c), P(0x1000), None, P(0x2000), P(0x3000), P(0x4000),
                           P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_grouped_gemm(ctypes.byref(c), 3, P(0x1000), P(0x1000), P(0x1000), P(0x1000), None, 1 << 20,
                                P(0x1000), P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_grouped_gemm(ctypes.byref(c), 1, P(0x1000), None, P(0x1000), P(0x1000), None, 1 << 20,
                                P(0x1000), P(0)) == binding.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_combine(ctypes.byref(c), P(0x1000), P(0x1000), P(0x1000), P(0x1001),
                           P(0)) == binding.MOE_ERR_INVALID_ARGUMENT


def test_router_stats_checks_arguments(lib):
    P = ctypes.c_void_p
    c = _cfg()
    n = ctypes.c_size_t()
    assert lib.moe_router_stats_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value >= 8 * 8 * 8 + 8 * 8  # softmax rows [T][E] and entropies [T] in binary64
    good = dict(x=0x1000, Wg=0x2000, ids=0x3000, gates=0x4000, frac=0x5000, mp=0x6000, sc=0x7000, ws=0x10000)

    def call(**kw):
        a = dict(good, **kw)
        return lib.moe_router_stats(ctypes.byref(c), P(a["x"]), P(a["Wg"]), None, None, None, P(a["ids"]),
                                    P(a["gates"]),
                                    P(a["frac"]), P(a["mp"]), P(a["sc"]), P(a["ws"]), kw.get("wsb", 1 << 30), P(0))
    for bad in (dict(frac=None), dict(mp=0x6004), dict(sc=None), dict(x=None), dict(ids=0x3002), dict(ws=0x10008)):
        assert call(**bad) == binding.MOE_ERR_INVALID_ARGUMENT, bad
    assert call(wsb=64) == binding.MOE_ERR_WORKSPACE_TOO_SMALL


def test_workloads_are_valid_configs(lib):
    n = ctypes.c_size_t()
    for name in moe_synth.WORKLOADS:
        w = moe_synth.workload(name)
        c = moe.config(w["T"], w["d"], w["d_ff"], w["E"], w["k"], w["act"], w["w"], tau=w["tau"],
                       use_gumbel=w["gumbel"])
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0, name


def _ws(lib, c):
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0
    return n.value


def test_workspace_holds_two_gemm2_halves_for_small_tiled_grids(lib):
    # bf16 tiled GEMM2 over a grid short of four rounds of 256-row tiles runs in two K halves, each writing its
    # own fp32 [T*k][d] partial; the streaming path and large grids keep one
    T, d, d_ff, E = 300, 512, 1024, 8
    y_bytes = T * 2 * d * 4
    tiled = _ws(lib, _cfg(T=T, d=d, d_ff=d_ff, E=E, gemm_path=moe.GEMM_TILED))
    streaming = _ws(lib, _cfg(T=T, d=d, d_ff=d_ff, E=E, gemm_path=moe.GEMM_STREAMING))
    assert tiled - streaming == y_bytes + (-y_bytes % 256)
    # d_ff not a multiple of 128: one K range
    assert _ws(lib, _cfg(T=T, d=d, d_ff=576, E=E, gemm_path=moe.GEMM_TILED)) == \
        _ws(lib, _cfg(T=T, d=d, d_ff=576, E=E, gemm_path=moe.GEMM_STREAMING))
    # 128 experts at T=2048: (2048*2/256 + 128) m-tiles x 32 n-tiles >= 1024 workgroups, one K range
    big = dict(T=2048, d=8192, d_ff=8192, E=128)
    assert _ws(lib, _cfg(gemm_path=moe.GEMM_TILED, **big)) == _ws(lib, _cfg(gemm_path=moe.GEMM_STREAMING, **big))
    # fp32 and INT4 experts never split
    assert _ws(lib, _cfg(T=T, d=d, d_ff=d_ff, E=E, act_dtype=moe.F32, w_dtype=moe.F32)) == \
        _ws(lib, _cfg(T=T, d=d, d_ff=d_ff, E=E, act_dtype=moe.F32, w_dtype=moe.F32, gemm_path=moe.GEMM_STREAMING))
