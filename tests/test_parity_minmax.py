"""GPU parity of the per-group min-max baseline against the oracle."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_encode_amd import turbokv as T
from kv_cache_quantization_encode_amd import workloads as W
from oracle import turbokv_oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _gpu_minmax(x16: np.ndarray, bits: int):
    n = x16.size
    x = G.to_dev_f16(x16.reshape(-1))
    codes = G.Guarded(n * bits // 8)
    scale = G.Guarded(n // 64 * 2)
    zero = G.Guarded(n // 64 * 2)
    G.note(f"minmax quant n={n} bits={bits}")
    T.tq_minmax_quant(x, n, 64, bits, codes.ptr, scale.ptr, zero.ptr)
    hc, hs, hz = codes.host(), scale.host(), zero.host()
    for buf, h in ((codes, hc), (scale, hs), (zero, hz)):
        buf.check_guard(h)
    out = G.Guarded(n * 2)
    G.note(f"minmax dequant n={n} bits={bits}")
    T.tq_minmax_dequant(codes.ptr, scale.ptr, zero.ptr, n, 64, bits, out.ptr)
    ho = out.host()
    out.check_guard(ho)
    return (hc[: n * bits // 8], hs[: n // 64 * 2].view(np.float16), hz[: n // 64 * 2].view(np.float16),
            ho[: n * 2].view(np.float16))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_minmax_one_layer_bit_exact(bits):
    x = W.minmax_tensor(layers=1)
    codes, scale, zero, deq = _gpu_minmax(x, bits)
    rc, rs, rz = O.minmax_quant(x, 64, bits)
    assert np.array_equal(scale.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(zero.view(np.uint16), rz.view(np.uint16))
    assert np.array_equal(O.unpack_minmax_codes(codes, bits, x.size), rc)
    ref = O.minmax_dequant(rc, rs, rz)
    got = deq.astype(np.float64)
    # fp16 output: within one fp16 rounding of the exact value
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -11 + 2.0 ** -24)
    q = O.quality(x, got)
    assert q["cos_flat"] > {2: 0.85, 3: 0.95, 4: 0.99}[bits]


def test_minmax_worked_example_on_gpu():
    import json, os
    gx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "minmax_worked_example.json")))
    g = np.random.default_rng(0).uniform(0.1, 0.9, 128)
    g[0], g[1] = 0.1, 0.9
    g[2:5] = gx["values"]
    g[64:] = g[:64]
    codes, scale, zero, _ = _gpu_minmax(g.astype(np.float16), 4)
    c = O.unpack_minmax_codes(codes, 4, 128)
    assert list(c[2:5]) == gx["codes"] and list(c[66:69]) == gx["codes"]


def test_minmax_degenerate_groups():
    x = np.zeros(64 * 6, np.float16)
    x[64:128] = 3.25
    x[128:192] = np.linspace(-1, 1, 64)
    x[192:256] = 65504.0
    x[256] = -65504.0
    x[320:] = np.float16(1e-7)
    for bits in (2, 3, 4):
        codes, scale, zero, deq = _gpu_minmax(x, bits)
        rc, rs, rz = O.minmax_quant(x, 64, bits)
        assert np.array_equal(scale.view(np.uint16), rs.view(np.uint16))
        assert np.array_equal(O.unpack_minmax_codes(codes, bits, x.size), rc)
        assert np.all(deq[64:128] == np.float16(3.25))


def test_minmax_full_size_sampled():
    """The min-max workload at full size (32 layers x 8 heads x 4096 x 128, one
    tensor); the oracle checks sampled groups."""
    x = W.minmax_tensor()
    bits = 3
    codes, scale, zero, deq = _gpu_minmax(x, bits)
    rng = np.random.default_rng(1)
    groups = np.concatenate([rng.choice(x.size // 64, 20000, replace=False), [x.size // 64 - 1]])
    xg = x.reshape(-1, 64)[groups]
    rc, rs, rz = O.minmax_quant(xg, 64, bits)
    assert np.array_equal(scale[groups].view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(zero[groups].view(np.uint16), rz.view(np.uint16))
    cg = codes.reshape(-1, 64 * bits // 8)[groups]
    got = O.unpack_bitstream(cg, bits, 64).reshape(-1)
    assert np.array_equal(got, rc)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_minmax_exact_ties(bits):
    """Values whose float32 quotient (v - zero)/scale is exactly k + 0.5 with a
    scale whose reciprocal is inexact (3, 5, 7, 11): the code is round half to
    even of the quotient itself, which a product with the rounded reciprocal
    misses (it lands one ulp above or below the tie)."""
    qmax = (1 << bits) - 1
    groups = []
    for s in (3.0, 5.0, 7.0, 11.0):
        for off in (0.0, -64.0, 256.0):
            g = np.empty(64)
            g[0], g[1] = off, off + s * qmax  # min and max fix zero = off and scale = s
            k = np.arange(62) % qmax
            g[2:] = off + s * (k + 0.5)
            groups.append(g)
    x = np.concatenate(groups).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), np.concatenate(groups))  # every value exact in fp16
    codes, scale, zero, _ = _gpu_minmax(x, bits)
    rc, rs, rz = O.minmax_quant(x, 64, bits)
    assert np.array_equal(scale.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(zero.view(np.uint16), rz.view(np.uint16))
    got = O.unpack_minmax_codes(codes, bits, x.size)
    assert np.array_equal(got, rc)
    # half to even: k + 0.5 goes to the even neighbour
    g2 = got.reshape(-1, 64)[:, 2:]
    k = np.arange(62) % qmax
    assert np.array_equal(g2, np.broadcast_to(np.where(k % 2 == 0, k, k + 1), g2.shape))
