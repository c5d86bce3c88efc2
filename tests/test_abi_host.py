"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/moe_verify.h
declares, reject invalid calls before touching the device, and size
workspaces / count bytes as documented.  No call here reaches a launch.
"""
import ctypes as C
import os
import re

import pytest

import oracle
from synth.configs import ALL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")

L = pytest.importorskip("moe_speculative_decoding_amd._lib",
                        reason="libmoe_verify.so not built")

FAKE = 0x10000  # an aligned non-null address; never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = C.CDLL(L.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def _declared_arity():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(moe_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else args.count(",") + 1
    return out


def test_binding_signatures_match_header():
    # a missing argtype would pass pointers through ctypes' int default
    arity = _declared_arity()
    assert set(L._SIG) == set(arity), set(L._SIG) ^ set(arity)
    for name, (_, args) in L._SIG.items():
        assert len(args) == arity[name], name


def test_abi_version_and_status_strings():
    assert L.moe_abi_version() == 1
    for s in range(9):
        assert L.status_str(s) and L.status_str(s) != "unknown status"
    assert L.status_str(99) == "unknown status"


def shape(**kw):
    base = dict(E=64, K=8, d=2048, f=1024, S=0, w_dtype="bf16", x_dtype="bf16")
    base.update(kw)
    return L.make_shape(**base)


@pytest.mark.parametrize("kw,expect", [
    (dict(K=0), L.MOE_ERR_ARG), (dict(K=9), L.MOE_ERR_ARG), (dict(E=7), L.MOE_ERR_ARG),
    (dict(E=257), L.MOE_ERR_ARG), (dict(S=5), L.MOE_ERR_ARG), (dict(S=-1), L.MOE_ERR_ARG),
    (dict(d=0), L.MOE_ERR_ARG), (dict(f=70000), L.MOE_ERR_ARG),
    (dict(w_dtype="bf16", x_dtype="f32"), L.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype="f32", x_dtype="bf16"), L.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype="fp8_e4m3", x_dtype="fp8_e4m3"), L.MOE_ERR_UNSUPPORTED),
    (dict(d=2044), L.MOE_ERR_UNSUPPORTED),                       # bf16 needs d % 8 == 0
    (dict(w_dtype="fp8_e4m3", d=2048, f=1000), L.MOE_ERR_UNSUPPORTED),  # fp8 needs % 128
])
def test_shape_validation(kw, expect):
    s = shape(**kw)
    ub, rb = C.c_uint64(), C.c_uint64()
    assert L.lib.moe_byte_counts(C.byref(s), 1, s.K, C.byref(ub), C.byref(rb)) == expect
    assert L.moe_workspace_size(s, 4, L.MOE_MODE_DEDUP) == 0


def _weights():
    return L.make_weights(w_gate=FAKE, w_up=FAKE, w_down=FAKE)


def test_ffn_validation_before_launch():
    s = shape()
    w = _weights()
    ws_need = L.moe_workspace_size(s, 8, L.MOE_MODE_DEDUP)
    ffn_need = 33024 + 8 * s.K * s.f * 2   # control block, hand-over flags, bf16 H
    dd = L.lib.moe_expert_ffn_dedup
    args = [C.byref(s), C.byref(w), FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
            ws_need, None]
    bad = list(args); bad[3] = 0          # n = 0
    assert dd(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[3] = 33         # n > 32
    assert dd(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[2] = FAKE + 4   # misaligned x
    assert dd(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[12] = ffn_need - 1
    assert dd(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(args); bad[11] = FAKE + 64  # workspace not 256-aligned
    assert dd(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(args); bad[4] = None       # U missing
    assert dd(*bad) == L.MOE_ERR_ARG
    w2 = L.make_weights(w_gate=FAKE, w_up=None, w_down=FAKE)
    bad = list(args); bad[1] = C.byref(w2)
    assert dd(*bad) == L.MOE_ERR_ARG
    s_sh = shape(S=2)
    bad = list(args); bad[0] = C.byref(s_sh)   # shared experts but no shared weights
    bad[12] = L.moe_workspace_size(s_sh, 8, L.MOE_MODE_DEDUP)
    assert dd(*bad) == L.MOE_ERR_ARG
    s8 = shape(w_dtype="fp8_e4m3", d=2048, f=1024)
    bad = list(args); bad[0] = C.byref(s8)     # fp8 without scales
    bad[12] = L.moe_workspace_size(s8, 8, L.MOE_MODE_DEDUP)
    assert dd(*bad) == L.MOE_ERR_ARG

    ps = L.lib.moe_expert_ffn_perslot
    assert ps(C.byref(s), C.byref(w), FAKE, 8, None, FAKE, None, None, FAKE, ws_need, None) \
        == L.MOE_ERR_ARG                                           # ids missing


def test_layer_validation_before_launch():
    s = shape()
    w = _weights()
    need = L.moe_workspace_size(s, 8, L.MOE_MODE_DEDUP)
    vl = L.lib.moe_verify_layer
    base = [C.byref(s), C.byref(w), FAKE, FAKE, 8, L.MOE_MODE_DEDUP, FAKE, L.MOE_F32,
            None, None, None, None, None, None, None, None, None, None, FAKE, need, None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return vl(*a)
    assert call(a4=0) == L.MOE_ERR_ARG                    # n = 0
    assert call(a4=33) == L.MOE_ERR_ARG                   # n > 32
    assert call(a5=7) == L.MOE_ERR_ARG                    # mode
    assert call(a2=None) == L.MOE_ERR_ARG                 # logits
    assert call(a3=FAKE + 8) == L.MOE_ERR_ARG             # misaligned x
    assert call(a6=FAKE + 4) == L.MOE_ERR_ARG             # misaligned out
    assert call(a7=L.MOE_FP8_E4M3) == L.MOE_ERR_UNSUPPORTED
    assert call(a10=FAKE) == L.MOE_ERR_ARG                # union outputs: all or none
    assert call(a15=FAKE + 4) == L.MOE_ERR_ARG            # misaligned y_slots
    assert call(a19=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(a18=FAKE + 64) == L.MOE_ERR_WORKSPACE     # workspace not 256-aligned
    # keeping the slot outputs outside the workspace shrinks the need
    r = lambda b: (b + 255) // 256 * 256
    own = need - r(8 * s.K * s.d * 4)
    assert call(a15=FAKE, a19=own - 1) == L.MOE_ERR_WORKSPACE


def test_layer_auto_validation_before_launch():
    s = shape()
    w = _weights()
    need = L.moe_workspace_size(s, 8, L.MOE_MODE_DEDUP)
    va = L.lib.moe_verify_layer_auto
    base = [C.byref(s), C.byref(w), FAKE, FAKE, 8, 0.8, FAKE, L.MOE_F32, None, None, FAKE, need,
            None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return va(*a)
    assert call(a5=-0.1) == L.MOE_ERR_ARG
    assert call(a5=float("nan")) == L.MOE_ERR_ARG
    assert call(a5=float("inf")) == L.MOE_ERR_ARG
    assert call(a4=0) == L.MOE_ERR_ARG
    assert call(a8=FAKE + 2) == L.MOE_ERR_ARG            # misaligned mode_out
    assert call(a9=FAKE + 4) == L.MOE_ERR_ARG            # misaligned bytes
    assert call(a11=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(a7=L.MOE_FP8_E4M3) == L.MOE_ERR_UNSUPPORTED


def test_budget_validation_before_launch():
    eb = L.lib.moe_expert_budget
    base = [FAKE, 4, 2, 8, 3, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return eb(*a)
    assert call(a4=0) == L.MOE_ERR_ARG                   # C < 1
    assert call(a5=2) == L.MOE_ERR_ARG                   # renorm not 0/1
    assert call(a1=33) == L.MOE_ERR_ARG                  # n
    assert call(a3=1) == L.MOE_ERR_ARG                   # E < K
    assert call(a0=None) == L.MOE_ERR_ARG
    assert call(a8=FAKE + 2) == L.MOE_ERR_ARG            # misaligned offsets
    assert call(a11=None) == L.MOE_ERR_ARG
    s = shape()
    w = _weights()
    need = L.moe_workspace_size(s, 8, L.MOE_MODE_DEDUP)
    vb = L.lib.moe_verify_layer_budget
    lb = [C.byref(s), C.byref(w), FAKE, FAKE, 8, 4, 1, FAKE, L.MOE_F32, None, None, None, None,
          None, None, None, None, None, None, FAKE, need, None]
    def lcall(**chg):
        a = list(lb)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return vb(*a)
    assert lcall(a5=0) == L.MOE_ERR_ARG                  # C < 1
    assert lcall(a6=-1) == L.MOE_ERR_ARG                 # renorm
    assert lcall(a4=0) == L.MOE_ERR_ARG                  # n
    assert lcall(a11=FAKE) == L.MOE_ERR_ARG              # union outputs: all or none
    assert lcall(a20=need - 1) == L.MOE_ERR_WORKSPACE
    assert lcall(a8=L.MOE_FP8_E4M3) == L.MOE_ERR_UNSUPPORTED


def test_bellman_validation_before_launch():
    bp = L.lib.moe_bellman_policy
    base = [FAKE, FAKE, 100, 8, FAKE, FAKE, FAKE, 256, None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return bp(*a)
    assert call(a2=0) == L.MOE_ERR_ARG                   # N
    assert call(a3=0) == L.MOE_ERR_ARG                   # L
    assert call(a3=33) == L.MOE_ERR_ARG
    assert call(a0=FAKE + 4) == L.MOE_ERR_ARG            # q must be 8-aligned
    assert call(a4=None) == L.MOE_ERR_ARG
    assert call(a5=FAKE + 2) == L.MOE_ERR_ARG
    assert call(a7=255) == L.MOE_ERR_WORKSPACE


def test_evict_validation_before_launch():
    ev = L.lib.moe_evict_select
    base = [FAKE, FAKE, FAKE, 16, FAKE, None, None, FAKE, FAKE, 256, None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return ev(*a)
    assert call(a3=0) == L.MOE_ERR_ARG
    assert call(a3=1025) == L.MOE_ERR_ARG
    assert call(a0=None) == L.MOE_ERR_ARG
    assert call(a4=FAKE + 2) == L.MOE_ERR_ARG
    assert call(a5=FAKE + 4) == L.MOE_ERR_ARG          # scores must be 8-aligned
    assert call(a7=None) == L.MOE_ERR_ARG
    assert call(a9=255) == L.MOE_ERR_WORKSPACE
    assert call(a8=FAKE + 128) == L.MOE_ERR_WORKSPACE


def test_ecospec_validation_before_launch():
    ec = L.lib.moe_ecospec_select
    base = [FAKE, FAKE, FAKE, None, 16, 4, 4, 0.1, FAKE, None, FAKE, 256, None]
    def call(**chg):
        a = list(base)
        for k, v in chg.items():
            a[int(k[1:])] = v
        return ec(*a)
    assert call(a4=0) == L.MOE_ERR_ARG                 # N
    assert call(a5=257) == L.MOE_ERR_ARG               # W
    assert call(a6=17) == L.MOE_ERR_ARG                # gamma > N
    assert call(a6=0) == L.MOE_ERR_ARG
    assert call(a4=1024, a5=9, a6=4) == L.MOE_ERR_UNSUPPORTED  # N*W beyond 64 KB of LDS
    assert call(a7=0.0) == L.MOE_ERR_ARG               # eps
    assert call(a7=float("nan")) == L.MOE_ERR_ARG
    assert call(a2=FAKE + 4) == L.MOE_ERR_ARG          # pred must be 8-aligned
    assert call(a8=None) == L.MOE_ERR_ARG
    assert call(a11=100) == L.MOE_ERR_WORKSPACE


def test_routing_and_combine_validation():
    rt = L.lib.moe_route_topk
    assert rt(FAKE, 0, 8, 2, FAKE, FAKE, None) == L.MOE_ERR_ARG
    assert rt(FAKE, 4, 8, 9, FAKE, FAKE, None) == L.MOE_ERR_ARG
    assert rt(FAKE, 4, 300, 2, FAKE, FAKE, None) == L.MOE_ERR_ARG
    assert rt(None, 4, 8, 2, FAKE, FAKE, None) == L.MOE_ERR_ARG
    bu = L.lib.moe_build_union
    assert bu(FAKE, 33, 8, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_ARG
    assert bu(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, FAKE, None) == L.MOE_ERR_ARG
    cb = L.lib.moe_combine
    assert cb(FAKE, FAKE, None, 4, 2, 1, 256, FAKE, L.MOE_F32, None) == L.MOE_ERR_ARG
    assert cb(FAKE, FAKE, None, 4, 2, 0, 256, FAKE, L.MOE_FP8_E4M3, None) == L.MOE_ERR_UNSUPPORTED
    assert cb(FAKE, FAKE, None, 4, 2, 0, 254, FAKE, L.MOE_F32, None) == L.MOE_ERR_UNSUPPORTED
    assert cb(FAKE, FAKE, None, 4, 2, 0, 256, FAKE + 8, L.MOE_BF16, None) == L.MOE_ERR_ARG
    assert cb(FAKE + 4, FAKE, None, 4, 2, 0, 256, FAKE, L.MOE_F32, None) == L.MOE_ERR_ARG
    assert L.lib.moe_decode_fp8(None, FAKE, 5, None) == L.MOE_ERR_ARG
    assert L.lib.moe_workspace_init(FAKE + 8, 1024, None) == L.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("cfg", ALL, ids=lambda c: c.name)
def test_byte_counts_match_oracle(cfg):
    s = L.make_shape(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype)
    for n in (1, 2, 8, 32):
        cap = min(n * cfg.K, cfg.E)
        for U in sorted({cfg.K, (cfg.K + cap) // 2, cap}):
            assert L.moe_byte_counts(s, n, U) == oracle.byte_counts(
                cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, n, U)
        with pytest.raises(L.MoeError):
            L.moe_byte_counts(s, n, cap + 1)
    # control block, hand-over flags, H in f32, slot outputs (one-launch pass)
    r = lambda b: (b + 255) // 256 * 256
    need = (33024 + r(32 * (cfg.K + cfg.S) * cfg.f * 4) + r(32 * cfg.K * cfg.d * 4)
            + r(32 * cfg.S * cfg.d * 4))
    assert L.moe_workspace_size(s, 32, L.MOE_MODE_DEDUP) == need
    assert L.moe_workspace_size(s, 32, L.MOE_MODE_PERSLOT) == need


def test_binding_fails_loudly_without_the_library():
    """No fallback: importing the binding with no built library raises, and so
    does every entry point of the layer helpers that imports it."""
    import subprocess
    import sys
    env = dict(os.environ, MOE_VERIFY_LIB="/nonexistent/libmoe_verify.so")
    for mod in ("moe_speculative_decoding_amd._lib", "moe_speculative_decoding_amd.layer"):
        r = subprocess.run([sys.executable, "-c", "import %s" % mod], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode != 0, mod
        assert "ImportError" in r.stderr and "not built" in r.stderr, r.stderr[-400:]


def test_noalloc_validation_before_launch():
    # every check runs before the static scratch is looked up, so no call
    # here reaches the device
    s = shape()
    w = _weights()
    fn = L.lib.moe_verify_layer_noalloc
    args = [C.byref(s), C.byref(w), FAKE, FAKE, 8, L.MOE_MODE_DEDUP, FAKE, L.MOE_F32] + \
        [None] * 10 + [None]
    bad = list(args); bad[4] = 0               # n = 0
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[5] = 2               # mode
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[7] = 5               # out dtype
    assert fn(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[10] = FAKE           # U given without the other union arrays
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[15] = FAKE + 4       # misaligned y_slots
    assert fn(*bad) == L.MOE_ERR_ARG
    # beyond the 16 MiB scratch: n*K*d*4 B of slot outputs alone exceed it
    big = shape(d=16384, f=1024)
    bad = list(args); bad[0] = C.byref(big); bad[4] = 32
    assert fn(*bad) == L.MOE_ERR_TOO_LARGE
    # the same pass with the slot outputs kept by the caller needs H only
    need = 33024 + 32 * 8 * 1024 * 4
    assert need <= 16 << 20
    need_ys = need + 32 * 8 * 16384 * 4
    assert need_ys > 16 << 20
    assert L.moe_workspace_size(big, 32, L.MOE_MODE_DEDUP) == need_ys


def test_pack_weights_validation_before_launch():
    fn = L.lib.moe_pack_weights
    s = shape()
    args = [C.byref(s), 4] + [FAKE] * 3 + [None] * 3 + [FAKE + 1024, FAKE + 2048, FAKE + 4096] + \
        [None] * 3 + [None]
    bad = list(args); bad[1] = 0            # no experts
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[1] = 257
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[8] = FAKE         # destination equals its source
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[3] = FAKE + 1     # misaligned bf16 source
    assert fn(*bad) == L.MOE_ERR_ARG
    bad = list(args); bad[4] = None
    assert fn(*bad) == L.MOE_ERR_ARG
    s8 = shape(w_dtype="fp8_e4m3", d=2048, f=1024)
    bad = list(args); bad[0] = C.byref(s8)  # fp8 without block scales
    assert fn(*bad) == L.MOE_ERR_ARG
    s_bad = shape(d=2044)
    bad = list(args); bad[0] = C.byref(s_bad)
    assert fn(*bad) == L.MOE_ERR_UNSUPPORTED
