"""GPU parity of the encoder and the dequantiser against the CPU oracle."""
import numpy as np
import pytest

from kv_cache_quantization_encode_amd import turbokv as T
from kv_cache_quantization_encode_amd import workloads as W
from oracle import turbokv_oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

FORMATS = [("prod", 1), ("prod", 2), ("prod", 3), ("mse", 1), ("mse", 2), ("mse", 3), ("mse", 4), ("q8", 8)]


@pytest.fixture(scope="module")
def ctx():
    with G.Ctx(42) as h:
        yield h


@pytest.fixture(scope="module")
def tab(oracle_tables):
    return oracle_tables


def _rows(case, which="k"):
    x = case.k if which == "k" else case.v
    return np.ascontiguousarray(x.reshape(-1, 128))


@pytest.mark.parametrize("kind,bits", FORMATS)
def test_encode_tiny_all_formats(ctx, tab, kind, bits):
    c = W.tiny()
    for which in ("k", "v"):
        x = _rows(c, which)
        packed, _ = G.gpu_encode(ctx, x, kind, bits, as_v=(which == "v"))
        G.check_encode(x, kind, bits, packed, tab)


@pytest.mark.parametrize("kind,bits", FORMATS)
@pytest.mark.parametrize("n", [1, 15, 17, 1037])
def test_encode_ragged_sizes(ctx, tab, kind, bits, n):
    c = W.llama8b(T=600, Hkv=2)
    x = _rows(c)[:n]
    packed, _ = G.gpu_encode(ctx, x, kind, bits)
    G.check_encode(x, kind, bits, packed, tab)


def test_encode_degenerate_rows(ctx, tab):
    x = np.zeros((40, 128), np.float16)
    x[1, 5] = 1.0                                   # one-hot
    x[2] = 65504.0                                  # fp16 max everywhere
    x[3] = np.float16(6e-8)                         # subnormals
    x[4, ::2] = -3.0
    x[5:] = np.random.default_rng(0).standard_normal((35, 128)).astype(np.float16)
    for kind, bits in FORMATS:
        packed, _ = G.gpu_encode(ctx, x, kind, bits)
        if kind == "q8":
            G.check_encode(x, kind, bits, packed, tab)
            continue
        # row 2 overflows fp32 in the norm (||x||^2 > 3.4e38) -> skip it in the comparison
        rows = [r for r in range(40) if r != 2]
        # rows 1 and 4 put many coordinates exactly on a boundary (z = 0 or a
        # midpoint): only "no mismatch outside the band" applies to them
        G.check_encode(x, kind, bits, packed, tab, rows=rows, max_exempt=1.0)
        u = O.unpack_tq(packed, kind, bits, 128, 40)
        assert np.all(u["idx"][0] == (1 << (bits - 1)))   # zero vector -> z = 0 -> upper middle cell
        assert float(u["norm"][0]) == 0.0


@pytest.mark.parametrize("kind,bits", [("prod", 3), ("mse", 4)])
def test_encode_llama8b_full_size_sampled(ctx, tab, kind, bits):
    """The benchmark's workload at full size (8 KV heads x 32768 tokens); the
    oracle checks contiguous row blocks spread over the tensor, incl. the end."""
    c = W.llama8b()
    x = _rows(c, "k" if kind == "prod" else "v")
    n = x.shape[0]
    packed, _ = G.gpu_encode(ctx, x, kind, bits, as_v=(kind == "mse"))
    starts = list(np.linspace(0, n - 512, 8).astype(int)) + [n - 300]
    for s in starts:
        cnt = min(512, n - s)
        sub = G.sub_packed(packed, kind, bits, n, s, cnt)
        G.check_encode(x[s:s + cnt], kind, bits, sub, tab)


def test_encode_needle_and_70b_rows(ctx, tab):
    nd = W.slice_case(W.needle(B=2, T=512), B=2)
    x = _rows(nd)
    for kind, bits in (("prod", 3), ("mse", 2)):
        packed, _ = G.gpu_encode(ctx, x, kind, bits)
        G.check_encode(x, kind, bits, packed, tab)
    l70 = W.llama70b_layer(5, T=1024)
    x = _rows(l70)
    packed, _ = G.gpu_encode(ctx, x, "prod", 2)
    G.check_encode(x, "prod", 2, packed, tab)


def test_encode_is_deterministic(ctx, tab):
    x = _rows(W.tiny())
    a, _ = G.gpu_encode(ctx, x, "prod", 3)
    b, _ = G.gpu_encode(ctx, x, "prod", 3)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kind,bits", FORMATS)
def test_decode_matches_oracle_on_same_bytes(ctx, tab, kind, bits):
    c = W.llama8b(T=520, Hkv=2)
    x = _rows(c)
    n = x.shape[0]
    packed, _ = G.gpu_encode(ctx, x, kind, bits)
    got = G.gpu_decode(ctx, packed, kind, bits, n)
    ref = O.dequant_packed(packed, kind, bits, tab, n)
    G.check_rows_close(got, ref)


def test_decode_quality_sanity(ctx, tab):
    """Stage-1 reconstruction error of the V codec tracks the codebook MSE."""
    x = np.random.default_rng(3).standard_normal((4096, 128)).astype(np.float16)
    for bits, mse in ((2, 0.1175), (3, 0.03454), (4, 0.009497)):
        packed, _ = G.gpu_encode(ctx, x, "mse", bits)
        got = G.gpu_decode(ctx, packed, "mse", bits, 4096).astype(np.float64)
        rel = np.sum((got - x) ** 2, axis=1) / np.sum(x.astype(np.float64) ** 2, axis=1)
        assert abs(rel.mean() - mse) / mse < 0.06


@pytest.mark.parametrize("n", [1, 1037, 40000])
@pytest.mark.parametrize("kf,vf", [(("prod", 3), ("mse", 4)), (("prod", 1), ("mse", 2)), (("q8", 8), ("mse", 3))])
def test_encode_k_and_v_in_one_call_equals_separate_calls(n, kf, vf):
    """tq_encode_kv with K and V together (one joint launch for small inputs
    with a QJL K format and a codebook V format, two launches otherwise)
    writes the same bytes as two single-tensor calls."""
    rng = np.random.default_rng(615 + n)
    k16 = (rng.standard_normal((n, 128), dtype=np.float32) * 3).astype(np.float16)
    v16 = rng.standard_normal((n, 128), dtype=np.float32).astype(np.float16)
    K, V = G.tf(*kf), G.tf(*vf)
    kl, vl = T.tq_packed_layout(K, 128, n), T.tq_packed_layout(V, 128, n)
    with G.Ctx(42) as ctx:
        kb, vb = G.Guarded(int(kl.total_bytes)), G.Guarded(int(vl.total_bytes))
        G.note(f"encode K+V together n={n} kf={kf} vf={vf}")
        T.tq_encode_kv(ctx, G.to_dev_f16(k16), G.to_dev_f16(v16), n, K, V, kb.ptr, vb.ptr)
        hk, hv = kb.host(), vb.host()
        kb.check_guard(hk, G.plane_ranges(kl))
        vb.check_guard(hv, G.plane_ranges(vl))
        ek, _ = G.gpu_encode(ctx, k16, *kf)
        ev, _ = G.gpu_encode(ctx, v16, *vf, as_v=True)
    assert np.array_equal(hk[: kl.total_bytes], ek)
    assert np.array_equal(hv[: vl.total_bytes], ev)
