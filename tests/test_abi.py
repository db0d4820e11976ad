"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, builds the same tables as the oracle's independent generator, lays
out planes as specified, and rejects bad arguments on the host before any
HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from kv_cache_quantization_encode_amd import turbokv as T
from oracle import turbokv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(T.LIB_PATH):
        pytest.fail("libturbokv.so is not built (run python -m kv_cache_quantization_encode_amd.build)")
    return T.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "turbokv.h")).read()
    names = sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", hdr)))
    assert len(names) == 16 and "tq_attn_decode" in names and "tq_attn_decode_noalloc" in names
    assert "tq_attn_decode_append" in names
    assert "tq_attn_prefill" in names and "tq_attn_prefill_workspace_bytes" in names and "tq_status_str" in names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_host_tables_match_oracle(lib):
    levels, bounds, signs, S = T.tq_host_tables(128, 128, 42)
    tab = O.Tables(128, seed=42)
    for b in range(1, 5):
        L = 1 << b
        assert np.max(np.abs(levels[b - 1, :L] - tab.levels[b])) < 1e-12
        assert np.max(np.abs(bounds[b - 1, :L - 1] - tab.bounds[b])) < 1e-12
    assert np.array_equal(signs.astype(np.float64), tab.signs)
    # S: fp16 bit patterns identical
    assert np.array_equal(S, tab.S.astype(np.float16).view(np.uint16))
    # another seed and another size also agree
    _, _, s2, S2 = T.tq_host_tables(64, 32, 7)
    assert np.array_equal(s2.astype(np.float64), O.random_signs(7, 64))
    assert np.array_equal(S2, O.gaussian_projection(7, 32, 64).astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("f,kind", [(T.turbo_k(2), "prod"), (T.turbo_k(3), "prod"), (T.turbo_k(4), "prod"),
                                    (T.mse(1), "mse"), (T.mse(2), "mse"), (T.mse(3), "mse"),
                                    (T.mse(4), "mse"), (T.Q8, "q8")])
@pytest.mark.parametrize("n", [0, 1, 17, 1000, 262144])
def test_layout_matches_oracle(lib, f, kind, n):
    lay = T.tq_packed_layout(f, 128, n)
    ref = O.tq_plane_layout(kind, f.bits, 128, n)
    assert lay.total_bytes == ref["total"]
    names = {"prod": ("idx", "sign", "norm"), "mse": ("idx", None, "norm"), "q8": ("q", None, "scale")}[kind]
    got = {"idx": (lay.idx_offset, lay.idx_bytes), "sign": (lay.sign_offset, lay.sign_bytes),
           "norm": (lay.norm_offset, lay.norm_bytes)}
    for ours, theirs in zip(("idx", "sign", "norm"), names):
        if theirs is None:
            assert got[ours][1] == 0
        else:
            assert got[ours] == ref["planes"][theirs]
    if n:
        assert lay.total_bytes >= n * O.bytes_per_vector(kind, f.bits)


class _FakeCtx(ctypes.Structure):
    # mirrors struct tq_ctx: only read by validation here; `dev` stays NULL so
    # nothing could ever be launched from it
    _fields_ = [("head_dim", ctypes.c_int), ("qjl_dim", ctypes.c_int), ("seed", ctypes.c_uint64),
                ("device", ctypes.c_int), ("dev", ctypes.c_void_p)]


A = 1 << 20  # a 256-byte aligned fake address; validation must reject before use


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert T.status_str(s)
    assert T.status_str(-99) == "unknown status"


def test_invalid_arguments_are_rejected_on_host(lib):
    ctx = _FakeCtx(128, 128, 42, 0, None)
    cp = ctypes.addressof(ctx)
    f3, v2 = T.turbo_k(3), T.mse(2)
    L = lib
    bad = T.tq_format(7, 3)
    # init / layout
    assert L.tq_codebook_init(None, 128, 128, 42, None) == T.TQ_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert L.tq_codebook_init(ctypes.byref(h), 100, 128, 42, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init(ctypes.byref(h), 64, 64, 42, None) == T.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_destroy(None) == T.TQ_ERR_INVALID_ARG
    d = T.tq_planes_desc()
    assert L.tq_packed_layout(bad, 128, 10, ctypes.byref(d)) == T.TQ_ERR_INVALID_ARG
    assert L.tq_packed_layout(T.tq_format(1, 4), 128, 10, ctypes.byref(d)) == T.TQ_ERR_INVALID_ARG
    assert L.tq_packed_layout(T.tq_format(0, 5), 128, 10, ctypes.byref(d)) == T.TQ_ERR_INVALID_ARG
    assert L.tq_packed_layout(f3, 64, 10, ctypes.byref(d)) == T.TQ_ERR_UNSUPPORTED
    assert L.tq_packed_layout(f3, 128, -1, ctypes.byref(d)) == T.TQ_ERR_INVALID_ARG
    # encode
    assert L.tq_encode_kv(None, A, A, 16, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(cp, None, None, 16, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(cp, A, A, -1, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(cp, A, A, 16, bad, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(cp, A, A, 16, f3, v2, None, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(cp, A + 2, A, 16, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG  # misaligned input
    assert L.tq_encode_kv(cp, A, A, 16, f3, v2, A + 16, A, None) == T.TQ_ERR_INVALID_ARG  # planes not 256-aligned
    assert L.tq_encode_kv(cp, A, A, 0, f3, v2, A, A, None) == T.TQ_OK  # nothing to do
    # append (one new row per sequence and KV head into a [B, Hkv, T_cap] cache)
    ap = L.tq_append_kv
    assert ap(None, A, A, 2, 8, 64, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 8, 64, None, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG  # no positions
    assert ap(cp, None, None, 2, 8, 64, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 0, 8, 64, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 0, 64, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 8, 0, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 8, 64, A + 2, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG  # misaligned pos
    assert ap(cp, A + 2, A, 2, 8, 64, A, f3, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 8, 64, A, f3, v2, A + 16, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 2, 8, 64, A, bad, v2, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, None, A, 2, 8, 64, A, f3, bad, None, A, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, None, 2, 8, 64, A, f3, v2, None, None, None) == T.TQ_ERR_INVALID_ARG
    assert ap(cp, A, A, 1 << 20, 8, 1 << 20, A, f3, v2, A, A, None) == T.TQ_ERR_UNSUPPORTED
    # decode
    assert L.tq_decode_kv(cp, None, f3, 16, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_decode_kv(cp, A, bad, 16, A, None) == T.TQ_ERR_INVALID_ARG
    assert L.tq_decode_kv(cp, A + 64, f3, 16, A, None) == T.TQ_ERR_INVALID_ARG
    # attention
    ws = T.tq_attn_workspace_bytes(1, 32, 8, 1024, f3, v2)
    assert ws > 0
    assert T.tq_attn_workspace_bytes(1, 32, 8, 0, f3, v2) == 0
    assert T.tq_attn_workspace_bytes(1, 30, 8, 64, f3, v2) == 0

    def attn(**kw):
        a = dict(ctx=cp, q=A, k=A, v=A, kf=f3, vf=v2, B=1, Hq=32, Hkv=8, T=1024, lens=None, tau=1e-6,
                 out=A, ws=A, wsb=ws)
        a.update(kw)
        return L.tq_attn_decode(a["ctx"], a["q"], a["k"], a["v"], a["kf"], a["vf"], a["B"], a["Hq"],
                                a["Hkv"], a["T"], a["lens"], a["tau"], a["out"], a["ws"], a["wsb"], None)

    assert attn(ctx=None) == T.TQ_ERR_INVALID_ARG
    assert attn(T=0) == T.TQ_ERR_INVALID_ARG
    assert attn(B=0) == T.TQ_ERR_INVALID_ARG
    assert attn(Hq=30) == T.TQ_ERR_INVALID_ARG
    assert attn(tau=-1.0) == T.TQ_ERR_INVALID_ARG
    assert attn(tau=float("nan")) == T.TQ_ERR_INVALID_ARG
    assert attn(q=A + 2) == T.TQ_ERR_INVALID_ARG
    assert attn(lens=A + 1) == T.TQ_ERR_INVALID_ARG
    assert attn(vf=T.turbo_k(3)) == T.TQ_ERR_UNSUPPORTED
    assert attn(Hq=24) == T.TQ_ERR_UNSUPPORTED  # GQA 3
    assert attn(ws=None) == T.TQ_ERR_WORKSPACE
    assert attn(wsb=ws - 1) == T.TQ_ERR_WORKSPACE
    assert attn(ws=A + 128) == T.TQ_ERR_WORKSPACE
    assert T.tq_attn_workspace_bytes(16384, 32, 8, 64, f3, v2) == 0  # 131072 (batch, kv head) pairs
    assert attn(B=16384) == T.TQ_ERR_UNSUPPORTED
    # prefill: Tq queries per sequence share its cache.  TurboQuant / codebook
    # K with codebook V take the prompt-scale kernels (statistics only in the
    # workspace, no limit on B * Tq * Hkv); q8 the grouped decode kernels
    pws = T.tq_attn_prefill_workspace_bytes(1, 32, 8, 1024, 16, f3, v2)
    assert pws > 0
    assert T.tq_attn_prefill_workspace_bytes(1, 32, 8, 1024, 1, f3, v2) == ws
    assert T.tq_attn_prefill_workspace_bytes(1, 32, 8, 1024, 0, f3, v2) == 0
    assert T.tq_attn_prefill_workspace_bytes(2, 32, 8, 1024, 4096, f3, v2) > 0
    assert T.tq_attn_prefill_workspace_bytes(2, 32, 8, 1024, 4096, T.Q8, T.Q8) == 0  # 65536 grid rows

    def prefill(**kw):
        a = dict(ctx=cp, q=A, k=A, v=A, kf=f3, vf=v2, B=1, Hq=32, Hkv=8, T=1024, Tq=16, lens=None, tau=1e-6,
                 out=A, ws=A, wsb=pws)
        a.update(kw)
        return L.tq_attn_prefill(a["ctx"], a["q"], a["k"], a["v"], a["kf"], a["vf"], a["B"], a["Hq"], a["Hkv"],
                                 a["T"], a["Tq"], a["lens"], a["tau"], a["out"], a["ws"], a["wsb"], None)

    assert prefill(ctx=None) == T.TQ_ERR_INVALID_ARG
    assert prefill(Tq=0) == T.TQ_ERR_INVALID_ARG
    assert prefill(Tq=-3) == T.TQ_ERR_INVALID_ARG
    assert prefill(q=A + 2) == T.TQ_ERR_INVALID_ARG
    assert prefill(lens=A + 2) == T.TQ_ERR_INVALID_ARG
    assert prefill(out=A + 4) == T.TQ_ERR_INVALID_ARG
    assert prefill(tau=float("inf")) == T.TQ_ERR_INVALID_ARG
    assert prefill(Hq=24) == T.TQ_ERR_UNSUPPORTED
    assert prefill(vf=T.turbo_k(3)) == T.TQ_ERR_UNSUPPORTED
    assert prefill(B=2, Tq=4096, kf=T.Q8, vf=T.Q8) == T.TQ_ERR_UNSUPPORTED
    assert prefill(wsb=pws - 1) == T.TQ_ERR_WORKSPACE
    assert prefill(wsb=0) == T.TQ_ERR_WORKSPACE
    # min-max
    mq = L.tq_minmax_quant
    assert mq(None, 64, 64, 3, A, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert mq(A, 65, 64, 3, A, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert mq(A, 64, 32, 3, A, A, A, None) == T.TQ_ERR_UNSUPPORTED
    assert mq(A, 64, 64, 5, A, A, A, None) == T.TQ_ERR_UNSUPPORTED
    assert mq(A, 64, 64, 0, A, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert mq(A + 8, 64, 64, 3, A, A, A, None) == T.TQ_ERR_INVALID_ARG
    assert mq(A, 0, 64, 3, A, A, A, None) == T.TQ_OK
    md = L.tq_minmax_dequant
    assert md(A, A, A, 64, 64, 3, None, None) == T.TQ_ERR_INVALID_ARG
    assert md(A, A, A, 64, 64, 1, A, None) == T.TQ_ERR_UNSUPPORTED
    assert md(A, A, A, 64, 64, 3, A + 2, None) == T.TQ_ERR_INVALID_ARG


def test_oracle_is_not_imported_by_the_product():
    pkg = os.path.join(ROOT, "kv_cache_quantization_encode_amd")
    pat = re.compile(r"^\s*(from\s+oracle\b|import\s+oracle\b)|turbokv_oracle", re.M)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, fn)).read()
                assert not pat.search(src), fn
