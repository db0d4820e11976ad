"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test cites what fixes the expected value: a worked example or table
printed on the pages (fixtures in tests/golden/), a closed form, a textbook
table, a library routine for a special case, an invariant, or brute force on
a tiny input.
"""
import copy
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch
from scipy import stats

from oracle import turbokv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# min-max baseline (mac-code issue #1, section 2.1)
# ----------------------------------------------------------------------------
def _group_with(values, lo, hi, n=64, seed=0):
    rng = np.random.default_rng(seed)
    g = rng.uniform(lo, hi, n)
    g[0], g[1] = lo, hi
    g[2:2 + len(values)] = values
    return g


def test_minmax_worked_example():
    gx = golden("minmax_worked_example.json")
    x = _group_with(gx["values"], gx["group_min"], gx["group_max"])
    code, scale, zero = O.minmax_quant(x, 64, gx["bits"])
    assert list(code[2:5]) == gx["codes"]
    assert abs(float(scale[0]) - gx["scale_printed"]) < 5e-5
    assert float(zero[0]) == float(np.float16(gx["group_min"]))
    deq = O.minmax_dequant(code, scale, zero)[2:5]
    # the page dequantises with the scale rounded to 4 decimals
    assert np.allclose(deq, gx["dequant_printed"], atol=1e-3)


def test_minmax_global_scale_example():
    gx = golden("minmax_global_scale_example.json")
    x = _group_with(gx["values"], gx["global_min"], gx["global_max"])
    code, scale, zero = O.minmax_quant(x, 64, gx["bits"])
    assert list(code[2:4]) == gx["codes"]
    ratio = (gx["values"][0] - gx["global_min"]) / float(scale[0])
    assert abs(ratio - gx["printed_ratio"]) < 0.01


def test_minmax_overhead_bits():
    gx = golden("minmax_overhead.json")
    over = gx["per_group_fp16_values"] * 16 / gx["group_size"]
    assert over == gx["overhead_bits_per_element"]
    assert 4 + over == gx["total_bits_at_4bit"]
    assert 2 + over == gx["total_bits_at_2bit"]
    assert abs(over / (2 + over) - gx["overhead_share_at_2bit"]) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_minmax_error_bound_and_degenerate(bits):
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal(64 * 50) * np.repeat(10 ** rng.uniform(-3, 1, 50), 64))
    x[64 * 7: 64 * 8] = 0.37  # a degenerate group
    x16 = x.astype(np.float16)
    code, scale, zero = O.minmax_quant(x16, 64, bits)
    assert code.min() >= 0 and code.max() <= (1 << bits) - 1
    deq = O.minmax_dequant(code, scale, zero)
    s = np.repeat(scale.astype(np.float64), 64)
    err = np.abs(deq - x16.astype(np.float64))
    # half a step, plus the fp16 rounding of the scale accumulated over the codes
    slack = s * (1 << bits) * 2.0 ** -10 + np.abs(x16.astype(np.float64)) * 2.0 ** -20
    assert np.all(err <= s / 2 + slack)
    assert float(scale[7]) == 0.0 and np.all(code[64 * 7:64 * 8] == 0)
    assert np.all(deq[64 * 7:64 * 8] == float(np.float16(0.37)))
    # every group's extremes map to 0 and 2^b - 1
    cg = code.reshape(-1, 64)
    nz = scale.astype(np.float64) > 0
    assert np.all(cg[nz].min(axis=1) == 0) and np.all(cg[nz].max(axis=1) == (1 << bits) - 1)


def test_minmax_bitstream_roundtrip():
    rng = np.random.default_rng(5)
    for b in (2, 3, 4):
        c = rng.integers(0, 1 << b, 64 * 3)
        packed = O.pack_minmax_codes(c, b)
        assert packed.size == 64 * 3 * b // 8
        assert np.array_equal(O.unpack_minmax_codes(packed, b, c.size), c)
    # LSB-first: code 1 at element 0 sets bit 0 of byte 0; at element 1 (b=3) bit 3
    assert O.pack_minmax_codes(np.array([1, 0, 0, 0, 0, 0, 0, 0]), 3)[0] == 1
    assert O.pack_minmax_codes(np.array([0, 1, 0, 0, 0, 0, 0, 0]), 3)[0] == 8
    assert O.pack_minmax_codes(np.array([0, 0, 4, 0, 0, 0, 0, 0]), 3)[1] == 1


# ----------------------------------------------------------------------------
# random tables
# ----------------------------------------------------------------------------
def test_splitmix64_published_vectors():
    # reference outputs of splitmix64 (Vigna's splitmix64.c / Java SplittableRandom)
    assert [int(v) for v in O.splitmix64_outputs(0, 4)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [int(v) for v in O.splitmix64_outputs(1234567, 3)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_projection_matrix_is_standard_normal(oracle_tables):
    S = oracle_tables.S
    assert S.shape == (128, 128)
    assert np.array_equal(S, S.astype(np.float16).astype(np.float64))
    flat = S.reshape(-1)
    assert abs(flat.mean()) < 0.03 and abs(flat.var() - 1) < 0.03
    assert stats.kstest(flat, "norm").pvalue > 1e-3
    # rows nearly orthogonal at this size: off-diagonal correlation ~ 1/sqrt(d)
    C = np.corrcoef(S)
    assert np.max(np.abs(C - np.eye(128))) < 0.45
    sg = oracle_tables.signs
    assert set(np.unique(sg)) == {-1.0, 1.0} and abs(sg.mean()) < 0.3
    # same seed -> same tables; different seed -> different tables
    assert np.array_equal(O.gaussian_projection(42, 128, 128), S)
    assert not np.array_equal(O.gaussian_projection(43, 128, 128), S)


# ----------------------------------------------------------------------------
# Walsh-Hadamard rotation (quidproquo.cc Stage 1: orthogonal, distance-preserving)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("d", [8, 32, 128])
def test_hadamard_matches_library_and_orthogonality(d):
    H = O.hadamard(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64))
    assert np.array_equal(H @ H, d * np.eye(d))
    R = O.rotation(O.random_signs(7, d))
    assert np.max(np.abs(R @ R.T - np.eye(d))) < 1e-12
    x = np.random.default_rng(d).standard_normal((10, d))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def _fwht(v):
    """Textbook in-place fast Walsh-Hadamard transform (natural order)."""
    v = np.array(v, dtype=np.float64)
    h = 1
    n = v.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("d", [8, 128])
def test_dense_rotation_equals_fast_transform(d):
    signs = O.random_signs(3, d)
    x = np.random.default_rng(1).standard_normal((5, d))
    dense = x @ O.rotation(signs).T
    fast = _fwht(x * signs) / math.sqrt(d)
    assert np.allclose(dense, fast, atol=1e-12)


def test_rotation_gaussianises_outliers(oracle_tables):
    """yeyulingfeng.com, technical highlights: rotation drops kurtosis toward 3."""
    rng = np.random.default_rng(101)
    x = rng.standard_normal((2048, 128))
    x[:, rng.choice(128, 4, replace=False)] *= 20
    _, z = O.standardised_rotation(x, oracle_tables)
    k_before = stats.kurtosis(x.reshape(-1), fisher=False)
    k_after = stats.kurtosis(z.reshape(-1), fisher=False)
    assert k_before > 20 and 2.0 < k_after < 3.5


# ----------------------------------------------------------------------------
# Lloyd-Max Gaussian codebook (quidproquo.cc Stage 1)
# ----------------------------------------------------------------------------
# Max, "Quantizing for minimum distortion" (1960): optimal levels for N(0,1)
MAX_1960 = {
    1: [0.7979],
    2: [0.4528, 1.5104],
    3: [0.2451, 0.7560, 1.3440, 2.1520],
    4: [0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181, 2.0690, 2.7326],
}
MAX_1960_MSE = {1: 0.3634, 2: 0.1175, 3: 0.03454, 4: 0.009497}


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_textbook_levels(bits, oracle_tables):
    c = oracle_tables.levels[bits]
    t = oracle_tables.bounds[bits]
    L = 1 << bits
    assert c.shape == (L,) and np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    assert np.allclose(c[L // 2:], MAX_1960[bits], atol=2e-4)
    assert abs(O.codebook_mse(c, t) - MAX_1960_MSE[bits]) / MAX_1960_MSE[bits] < 1e-3
    # both Lloyd conditions hold at the fixed point
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    from scipy import integrate
    for k in range(L):
        m0, _ = integrate.quad(lambda z: stats.norm.pdf(z), lo[k], hi[k], epsabs=1e-15)
        m1, _ = integrate.quad(lambda z: z * stats.norm.pdf(z), lo[k], hi[k], epsabs=1e-15)
        assert abs(m1 / m0 - c[k]) < 1e-9


def test_codebook_one_bit_closed_form(oracle_tables):
    c = oracle_tables.levels[1]
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-13
    assert abs(O.codebook_mse(c, oracle_tables.bounds[1]) - (1 - 2 / math.pi)) < 1e-10


# ----------------------------------------------------------------------------
# Quantiser: nearest level (brute force at d = 8), ties, round trip
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [1, 2])
def test_quantiser_brute_force_d8(bits):
    tab = O.Tables(8, seed=11)
    c = tab.levels[bits]
    L = len(c)
    grid = np.array(np.meshgrid(*[np.arange(L)] * 8, indexing="ij")).reshape(8, -1).T
    cand = c[grid]  # every code vector of the product codebook
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((6, 8))
    x[0, 2] *= 20
    enc = O.encode(x, bits, False, tab)
    for r in range(x.shape[0]):
        best = np.argmin(np.sum((cand - enc["z"][r]) ** 2, axis=1))
        assert np.array_equal(grid[best], enc["idx"][r])
    # the library's sorted search gives the same cells
    assert np.array_equal(np.searchsorted(tab.bounds[bits], enc["z"], side="right"), enc["idx"])
    assert np.array_equal(O.nearest_level(enc["z"], c), enc["idx"])


def test_quantiser_ties_go_up_and_zero_vector(oracle_tables):
    for b in (1, 2, 3, 4):
        c = oracle_tables.levels[b]
        t = oracle_tables.bounds[b]
        assert np.array_equal(O.quantise_index(t, t), np.arange(1, len(c)))
        below = np.nextafter(t, -np.inf)
        assert np.array_equal(O.quantise_index(below, t), np.arange(0, len(c) - 1))
        # away from the boundaries the cell index is the nearest level
        zs = np.random.default_rng(b).standard_normal(20000) * 1.5
        assert np.array_equal(O.quantise_index(zs, t), O.nearest_level(zs, c))
    enc = O.encode(np.zeros((1, 128)), 3, True, oracle_tables)
    assert np.all(enc["idx"] == 4) and float(enc["norm"][0]) == 0.0
    assert float(enc["rnorm"][0]) == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_rotation_direction_and_residual(bits, oracle_tables):
    """x = R^T c (rows: c @ R) must land on z = sqrt(d) c/||c||: pins that the
    encoder rotates with R and not its transpose, and that gamma is the
    x-domain distance to the Stage-1 reconstruction."""
    tab = oracle_tables
    rng = np.random.default_rng(bits)
    idx = rng.integers(0, 1 << bits, (4, 128))
    c = tab.levels[bits][idx]
    scale = np.array([1.0, 3.5, 0.25, 10.0])
    x = scale[:, None] * (c @ tab.R)
    enc = O.encode(x, bits, True, tab)
    cn = np.linalg.norm(c, axis=1)
    assert np.allclose(enc["n64"], scale * cn, rtol=1e-13)
    assert np.allclose(enc["z"], math.sqrt(128) * c / cn[:, None], atol=1e-12)
    xhat1 = O.dequant_mse(enc["idx"], enc["n64"], bits, tab)
    assert np.allclose(enc["gamma64"], np.linalg.norm(x - xhat1, axis=1), rtol=1e-10)


# ----------------------------------------------------------------------------
# MSE codec (Stage 1 alone)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_codec_distortion_matches_codebook(bits, oracle_tables):
    tab = oracle_tables
    x = np.random.default_rng(bits).standard_normal((1500, 128))
    enc = O.encode(x, bits, False, tab)
    vhat = O.dequant_mse(enc["idx"], enc["n64"], bits, tab)
    rel = np.sum((x - vhat) ** 2, axis=1) / np.sum(x * x, axis=1)
    # isotropic x: z_i is sqrt(d) x a sphere coordinate, close to N(0,1) at d = 128
    mse = MAX_1960_MSE[bits]
    assert abs(rel.mean() - mse) / mse < 0.05


# ----------------------------------------------------------------------------
# QJL (quidproquo.cc Stage 2; chenxutan.com 2.3)
# ----------------------------------------------------------------------------
def test_qjl_unbiased_across_seeds(oracle_tables):
    base = oracle_tables
    rng = np.random.default_rng(77)
    x = rng.standard_normal((16, 128))
    x[:, :4] *= 20
    q = rng.standard_normal(128)
    bits = 2
    enc0 = O.encode(x, bits, False, base)
    xhat1 = O.dequant_mse(enc0["idx"], enc0["n64"], bits, base)
    r = x - xhat1
    true_ip = r @ q
    ests = []
    for seed in range(1000, 1500):
        tab = copy.copy(base)
        tab.S = O.gaussian_projection(seed, 128, 128)
        enc = O.encode(x, bits, True, tab)
        assert np.allclose(enc["gamma64"], np.linalg.norm(r, axis=1), rtol=1e-9)
        ests.append(O.qjl_inner_product(q, enc["bits_qjl"], enc["gamma64"], tab))
    ests = np.array(ests)  # [seeds, tokens]
    n = ests.shape[0]
    zscore = (ests.mean(axis=0) - true_ip) / (ests.std(axis=0, ddof=1) / math.sqrt(n))
    assert np.max(np.abs(zscore)) < 4.5
    # closed-form variance of the estimator for Gaussian rows:
    # Var = ||r||^2 (pi/2 ||q||^2 - <q, r/||r||>^2) / m
    rn = np.linalg.norm(r, axis=1)
    var = rn ** 2 * (math.pi / 2 * (q @ q) - (r @ q / rn) ** 2) / 128
    ratio = ests.var(axis=0, ddof=1) / var
    assert np.all((ratio > 0.7) & (ratio < 1.35))


def test_qjl_zero_residual_adds_nothing(oracle_tables):
    tab = oracle_tables
    idx = np.random.default_rng(0).integers(0, 8, (3, 128))
    bitsq = np.random.default_rng(1).integers(0, 2, (3, 128))
    n = np.array([1.0, 2.0, 3.0])
    a = O.dequant_prod(idx, bitsq, n, np.zeros(3), 3, tab)
    b = O.dequant_mse(idx, n, 3, tab)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_prod_dequant_inner_product_is_stage1_plus_qjl(oracle_tables):
    tab = oracle_tables
    x = np.random.default_rng(9).standard_normal((8, 128))
    q = np.random.default_rng(10).standard_normal(128)
    enc = O.encode(x, 2, True, tab)
    khat = O.dequant_prod(enc["idx"], enc["bits_qjl"], enc["n64"], enc["gamma64"], 2, tab)
    stage1 = O.dequant_mse(enc["idx"], enc["n64"], 2, tab)
    corr = O.qjl_inner_product(q, enc["bits_qjl"], enc["gamma64"], tab)
    assert np.allclose(khat @ q, stage1 @ q + corr, atol=1e-10)


# ----------------------------------------------------------------------------
# Packed layout
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,bits,size", [("prod", 1, 36), ("prod", 2, 52), ("prod", 3, 68),
                                            ("mse", 1, 18), ("mse", 2, 34), ("mse", 3, 50),
                                            ("mse", 4, 66), ("q8", 8, 136), ("mse32", 2, 40), ("mse32", 3, 56),
                                            ("prod32", 2, 58)])
def test_bytes_per_vector(kind, bits, size):
    assert O.bytes_per_vector(kind, bits) == size


@pytest.mark.parametrize("kind,bits", [("prod", 2), ("prod", 3), ("mse", 2), ("mse", 3), ("mse", 4)])
def test_pack_unpack_roundtrip(kind, bits, oracle_tables):
    x = np.random.default_rng(bits).standard_normal((37, 128)).astype(np.float16)
    enc = O.encode(x, bits, kind == "prod", oracle_tables)
    buf = O.pack_tq(enc, kind, bits, 128)
    u = O.unpack_tq(buf, kind, bits, 128, 37)
    assert np.array_equal(u["idx"], enc["idx"])
    assert np.array_equal(u["norm"].view(np.uint16), enc["norm"].view(np.uint16))
    if kind == "prod":
        assert np.array_equal(u["bits_qjl"], enc["bits_qjl"])
        assert np.array_equal(u["rnorm"].view(np.uint16), enc["rnorm"].view(np.uint16))


@pytest.mark.parametrize("kind,bits", [("prod32", 2), ("prod32", 1), ("mse32", 2), ("mse32", 4)])
def test_pack_unpack_roundtrip_block32(kind, bits, oracle_tables):
    """Block-32 planes: block norms of every vector, then (K) every gamma;
    the plane sizes add up to bytes_per_vector."""
    x = np.random.default_rng(bits + 7).standard_normal((37, 128)).astype(np.float16)
    enc = O.encode_block32(x, bits, kind == "prod32", oracle_tables)
    buf = O.pack_tq(enc, kind, bits, 128)
    lay = O.tq_plane_layout(kind, bits, 128, 37)
    assert sum(sz for _, sz in lay["planes"].values()) == 37 * O.bytes_per_vector(kind, bits)
    u = O.unpack_tq(buf, kind, bits, 128, 37)
    assert np.array_equal(u["idx"], enc["idx"])
    assert np.array_equal(u["bnorm"].view(np.uint16), enc["bnorm"].view(np.uint16))
    o, _ = lay["planes"]["norm"]
    first = buf[o:o + 8].copy().view(np.float16)  # vector 0: its four block norms
    assert np.array_equal(first.view(np.uint16), enc["bnorm"][0].view(np.uint16))
    if kind == "prod32":
        assert np.array_equal(u["bits_qjl"], enc["bits_qjl"])
        assert np.array_equal(u["rnorm"].view(np.uint16), enc["rnorm"].view(np.uint16))
        g0 = buf[o + 37 * 8:o + 37 * 8 + 2].copy().view(np.float16)
        assert g0.view(np.uint16)[0] == enc["rnorm"][0].view(np.uint16)


# ----------------------------------------------------------------------------
# Format arithmetic (quidproquo.cc format table; chenxutan.com 1.2 and 3.1)
# ----------------------------------------------------------------------------
def test_turbo_format_bits_and_ratios():
    gx = golden("turbo_formats.json")["formats"]
    for name, bits_cb in (("turbo2", 1), ("turbo3", 2), ("turbo4", 3)):
        f = gx[name]
        assert f["stage1_bits"] == bits_cb and f["stage1_bits"] + f["stage2_bits"] == f["total_bits"]
        # payload bits per element of our K record: codebook bits + one QJL bit
        payload = (O.bytes_per_vector("prod", bits_cb) - 4) * 8 / 128
        assert payload == f["total_bits"]
    # the printed ratios come from block-norm accounting: one fp16 per 32 (0.5 bit)
    # reproduces 6.4 and 4.57; one per 128 (0.125 bit) gives 5.12; 0.25 bit gives 3.76
    assert abs(16 / (2 + 0.5) - gx["turbo2"]["ratio_low"]) < 0.01
    assert abs(16 / (3 + 0.5) - gx["turbo3"]["ratio_low"]) < 0.05
    assert abs(16 / (3 + 0.125) - gx["turbo3"]["ratio_high"]) < 0.05
    assert abs(16 / (4 + 0.25) - gx["turbo4"]["ratio_low"]) < 0.05
    # our layout (fp16 norm + fp16 residual norm per 128-vector = 0.25 bit)
    ours = {n: 256 / O.bytes_per_vector("prod", b) for n, b in (("turbo2", 1), ("turbo3", 2), ("turbo4", 3))}
    assert abs(ours["turbo4"] - gx["turbo4"]["ratio_low"]) < 0.05
    assert gx["turbo3"]["ratio_low"] <= ours["turbo3"] <= gx["turbo3"]["ratio_high"]
    assert ours["turbo2"] > gx["turbo2"]["ratio_low"]


def test_asymmetric_ratio_arithmetic():
    gx = golden("asymmetric_ratio.json")
    for key in ("symmetric", "asymmetric"):
        v = gx[key]
        r = 2 * gx["fp16_bits"] / (v["k_bits"] + v["v_bits"])
        assert round(r, 1) == v["ratio_printed"]


def test_kv_cache_size_formula():
    gx = golden("kv_cache_size.json")
    for case in gx["cases"]:
        b = O.kv_cache_bytes_fp16(gx["layers"], gx["kv_heads"], gx["head_dim"], case["tokens"])
        assert b / 2 ** 30 == case["gib"]


def test_boundary_layer_memory_overhead():
    gx = golden("sparse_v_boundary.json")
    L = gx["example_layers"]
    prot = gx["boundary_first"] + gx["boundary_last"]
    assert prot == gx["protected_layers_printed"]
    turbo = O.bytes_per_vector("prod", 3) + O.bytes_per_vector("mse", 4)
    q8 = 2 * O.bytes_per_vector("q8", 8)
    inc = ((L - prot) * turbo + prot * q8) / (L * turbo) - 1
    assert 0 < inc < gx["memory_increase_bound"]


# ----------------------------------------------------------------------------
# q8 boundary blocks
# ----------------------------------------------------------------------------
def test_q8_invariants():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((40, 128)) * 3).astype(np.float16).astype(np.float64)
    x[5, 32:64] = 0.0
    q, sc = O.q8_quant(x)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    xh = O.q8_dequant(q, sc)
    s = np.repeat(sc.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(xh - x) <= s / 2 + np.abs(x) * 2.0 ** -9 + 1e-12)
    # the largest magnitude of each block lands on +-127
    qa = np.abs(q.astype(int)).reshape(40, 4, 32).max(axis=2)
    nz = sc.astype(np.float64) > 0
    assert np.all(qa[nz] == 127)
    assert float(sc[5, 1]) == 0.0 and np.all(q[5, 32:64] == 0)
    buf = O.pack_q8(q, sc, 128)
    u = O.unpack_q8(buf, 128, 40)
    assert np.array_equal(u["q"], q) and np.array_equal(u["scale"].view(np.uint16), sc.view(np.uint16))


# ----------------------------------------------------------------------------
# Decode attention with sparse V (chenxutan.com 1.1 / 3.3; yeyulingfeng.com item 4)
# ----------------------------------------------------------------------------
def _rand_attn(B=2, Hq=8, Hkv=2, T=40, d=16, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d)) * 2
    v = rng.standard_normal((B, Hkv, T, d))
    return q, k, v


def test_attention_tau0_equals_library_sdpa():
    q, k, v = _rand_attn()
    out, _ = O.attention_decode(q, k, v, tau=0.0)
    g = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k, g, axis=1))
    vt = torch.from_numpy(np.repeat(v, g, axis=1))
    qt = torch.from_numpy(q)[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0, :].numpy()
    assert np.allclose(out, ref, atol=1e-12)


def test_attention_sparse_v_drops_small_weights_without_renormalising():
    q, k, v = _rand_attn(seed=3)
    tau = golden("sparse_v_boundary.json")["sparse_v_threshold"]
    k[:, :, 5] *= 6.0  # make a few dominant keys so that many weights fall below tau
    dense, p = O.attention_decode(q, k, v, tau=0.0)
    sparse, _ = O.attention_decode(q, k, v, tau=tau)
    g = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            small = p[b, h] < tau
            dropped = (p[b, h] * small) @ v[b, h // g]
            assert np.allclose(sparse[b, h], dense[b, h] - dropped, atol=1e-13)
    assert np.any(p < tau)


def test_attention_special_cases():
    q, k, v = _rand_attn(T=1)
    out, _ = O.attention_decode(q, k, v, tau=1e-6)
    g = q.shape[1] // k.shape[1]
    assert np.allclose(out, np.repeat(v[:, :, 0], g, axis=1), atol=1e-15)
    q, k, v = _rand_attn(T=12)
    k[:] = k[:, :, :1]  # identical keys -> uniform weights -> mean of V
    out, _ = O.attention_decode(q, k, v, tau=1e-6)
    assert np.allclose(out, np.repeat(v.mean(axis=2), g, axis=1), atol=1e-12)
    out, _ = O.attention_decode(q, k, v, tau=0.5)  # tau above every weight
    assert np.all(out == 0)
    q, k, v = _rand_attn(T=2)
    k[:, :, 1] = k[:, :, 0]  # two equal weights of exactly 1/2: a weight equal to tau is kept
    out, _ = O.attention_decode(q, k, v, tau=0.5)
    assert np.allclose(out, np.repeat(v.mean(axis=2), g, axis=1), atol=1e-12)
    lens = np.array([3, 0])
    q, k, v = _rand_attn(T=9)
    out, _ = O.attention_decode(q, k, v, tau=0.0, seq_lens=lens)
    ref, _ = O.attention_decode(q[:1], k[:1, :, :3], v[:1, :, :3], tau=0.0)
    assert np.allclose(out[0], ref[0]) and np.all(out[1] == 0)


def test_prefill_tau0_equals_library_causal_sdpa():
    """Causal prefill at tau = 0 equals the library's attention with an explicit
    boolean mask (query i of a sequence of length L sees L - Tq + i + 1 keys)."""
    rng = np.random.default_rng(21)
    B, Tq, Hq, Hkv, T, d = 2, 5, 4, 2, 11, 16
    q = rng.standard_normal((B, Tq, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d)) * 2
    v = rng.standard_normal((B, Hkv, T, d))
    lens = np.array([T, 8])
    out = O.attention_prefill(q, k, v, tau=0.0, seq_lens=lens)
    g = Hq // Hkv
    for b in range(B):
        L = lens[b]
        mask = np.zeros((Tq, L), bool)
        for i in range(Tq):
            mask[i, :L - Tq + i + 1] = True
        kt = torch.from_numpy(np.repeat(k[b:b + 1, :, :L], g, axis=1))
        vt = torch.from_numpy(np.repeat(v[b:b + 1, :, :L], g, axis=1))
        qt = torch.from_numpy(q[b:b + 1].transpose(0, 2, 1, 3).copy())  # [1, Hq, Tq, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
        assert np.allclose(out[b], ref[0].numpy().transpose(1, 0, 2), atol=1e-12)


def test_prefill_special_cases():
    rng = np.random.default_rng(22)
    B, Tq, Hq, Hkv, T, d = 2, 4, 4, 2, 9, 8
    q = rng.standard_normal((B, Tq, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d)) * 3
    v = rng.standard_normal((B, Hkv, T, d))
    lens = np.array([9, 2])
    out = O.attention_prefill(q, k, v, tau=1e-6, seq_lens=lens)
    # the last query of each sequence is the decode step over the whole sequence
    dec, _ = O.attention_decode(q[:, -1], k, v, tau=1e-6, seq_lens=lens)
    assert np.allclose(out[:, -1], dec, atol=1e-13)
    # a sequence shorter than the query block: the first queries see nothing
    assert np.all(out[1, :2] == 0) and np.any(out[1, 2] != 0)
    # query 2 of sequence 1 sees exactly token 0: its output is that V row
    g = Hq // Hkv
    assert np.allclose(out[1, 2], np.repeat(v[1, :, 0], g, axis=0), atol=1e-14)
    # causality: keys and values after a query's position do not change it
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 7:] = rng.standard_normal(k2[0, :, 7:].shape) * 5
    v2[0, :, 7:] = 1e3
    out2 = O.attention_prefill(q, k2, v2, tau=1e-6, seq_lens=lens)
    assert np.allclose(out2[0, :2], out[0, :2], atol=1e-13)  # positions 5, 6
    assert not np.allclose(out2[0, 2:], out[0, 2:])


def test_rotated_domain_scores_equal_dense_scores(oracle_tables):
    """The score of a packed K row computed without dequantising (rotated query
    dotted with codebook values, plus the QJL term on S R q) equals the score
    against the dense dequantised row."""
    tab = oracle_tables
    rng = np.random.default_rng(12)
    x = rng.standard_normal((30, 128))
    q = rng.standard_normal(128)
    enc = O.encode(x, 3, True, tab)
    n = enc["norm"].astype(np.float64)
    gmm = enc["rnorm"].astype(np.float64)
    khat = O.dequant_prod(enc["idx"], enc["bits_qjl"], n, gmm, 3, tab)
    dense = khat @ q / math.sqrt(128)
    qrot = tab.R @ q
    qproj = tab.S @ qrot
    zhat = tab.levels[3][enc["idx"]]
    sgn = 2.0 * enc["bits_qjl"] - 1
    rotated = (n / math.sqrt(128) * (zhat @ qrot) +
               math.sqrt(math.pi / 2) / 128 * gmm * (sgn @ qproj)) / math.sqrt(128)
    assert np.allclose(dense, rotated, atol=1e-11)


# ----------------------------------------------------------------------------
# QJL projection from given codes (the checker behind every GPU sign-bit
# comparison) and the reconstruction-quality measure
# ----------------------------------------------------------------------------
def test_qjl_projection_from_codes_matches_encode_and_permutation(oracle_tables):
    """P = S (z - c[idx]) for the given codes [quidproquo.cc, Stage 2].  On the
    encoder's own codes it is the encoder's projection; with a permutation
    matrix as S it is the rotated residual permuted, where z comes from the
    textbook FWHT here (not from the oracle's rotation): (S e)_i = e_pi(i)."""
    tab = oracle_tables
    rng = np.random.default_rng(31)
    x = rng.standard_normal((12, 128))
    x[:, :3] *= 15
    perm = np.roll(np.arange(128), 5)  # a cyclic shift: not its own inverse
    tabp = copy.copy(tab)
    tabp.S = np.eye(128)[perm]
    z = _fwht(x * tab.signs) / np.linalg.norm(x, axis=1)[:, None]  # sqrt(d) R x / ||x||
    for bits in (1, 2, 3):
        enc = O.encode(x, bits, True, tab)
        P = O.qjl_projection_from_codes(x, enc["idx"], bits, tab)
        assert np.allclose(P, enc["P"], rtol=0, atol=1e-12)
        idx = rng.integers(0, 1 << bits, (12, 128))  # arbitrary codes, not the encoder's
        e = z - np.asarray(MAX_1960_LEVELS_FULL[bits])[idx]
        Pp = O.qjl_projection_from_codes(x, idx, bits, tabp)
        assert np.allclose(Pp, e[:, perm], atol=2e-4)  # printed levels carry 4 decimals
        Pe = O.qjl_projection_from_codes(x, idx, bits, tab)
        assert np.allclose(Pe, (z - tab.levels[bits][idx]) @ tab.S.T, atol=1e-9)


# all 2^b levels of Max (1960), ascending
MAX_1960_LEVELS_FULL = {b: [-v for v in reversed(MAX_1960[b])] + list(MAX_1960[b]) for b in MAX_1960}


def test_quality_closed_forms():
    """MSE and cosine [mac-code issue #1, quality measure]: a scaled copy has
    cosine 1 (or -1) and MSE (s - 1)^2 mean x^2; orthogonal rows (Hadamard rows)
    have cosine 0; a 3-4-5 example by hand."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((6, 128))
    q = O.quality(x, 2 * x)
    assert abs(q["mse"] - np.mean(x ** 2)) < 1e-12
    assert abs(q["cos_flat"] - 1) < 1e-12 and abs(q["cos_vec_mean"] - 1) < 1e-12
    q = O.quality(x, -0.5 * x)
    assert abs(q["mse"] - 2.25 * np.mean(x ** 2)) < 1e-12
    assert abs(q["cos_flat"] + 1) < 1e-12 and abs(q["cos_vec_mean"] + 1) < 1e-12
    H = scipy.linalg.hadamard(128).astype(np.float64)
    q = O.quality(H[:4], H[4:8])
    assert abs(q["cos_flat"]) < 1e-15 and abs(q["cos_vec_mean"]) < 1e-15
    assert q["mse"] == 2.0  # distinct Hadamard rows differ in exactly half the entries, by 2
    a = np.zeros((2, 128))
    b = np.zeros((2, 128))
    a[0, :2], b[0, :2] = (3, 4), (4, 3)   # cosine 24/25
    a[1, 2], b[1, 3] = 1.0, 2.0           # orthogonal row: cosine 0
    q = O.quality(a, b)
    assert abs(q["cos_vec_mean"] - (24 / 25 + 0) / 2) < 1e-15
    assert abs(q["cos_flat"] - 24 / math.sqrt(26 * 29)) < 1e-15
    assert abs(q["mse"] - (1 + 1 + 1 + 4) / 256) < 1e-15


def test_attention_decode_clamps_lengths():
    """Lengths outside [0, T] mean the nearest end (the library's convention):
    a negative length attends to nothing, a length past T to all T tokens."""
    q, k, v = _rand_attn(T=7)
    out, _ = O.attention_decode(q, k, v, tau=1e-6, seq_lens=np.array([-3, 12]))
    full, _ = O.attention_decode(q, k, v, tau=1e-6)
    assert np.all(out[0] == 0)
    assert np.array_equal(out[1], full[1])


# ----------------------------------------------------------------------------
# Block-32 norm storage (yeyulingfeng.com "TurboQuant+: 3.8x compression ...",
# technical highlights: block-32 storage; quidproquo.cc format table)
# ----------------------------------------------------------------------------
def test_block32_ratio_arithmetic():
    """One fp16 norm per 32 coordinates adds 16/32 = 0.5 bits per element: the
    pages' 6.4x for turbo2 is 16/(2+0.5) and the low end of their 4.6-5.1x for
    turbo3 is 16/(3+0.5) = 4.57.  K keeps one fp16 residual norm per vector on
    top (turbo3 K: 16/(3+0.625))."""
    def ratio(kind, bits):
        return 16.0 / (O.bytes_per_vector(kind, bits) * 8 / 128)
    assert ratio("mse32", 2) == pytest.approx(6.4, abs=1e-12)
    assert ratio("mse32", 3) == pytest.approx(16 / 3.5, abs=1e-12)
    assert round(ratio("mse32", 3), 2) == 4.57
    assert ratio("prod32", 2) == pytest.approx(16 / 3.625, abs=1e-12)
    assert ratio("prod32", 1) == pytest.approx(16 / 2.625, abs=1e-12)
    assert O.bytes_per_vector("mse32", 4) == 64 + 8


def _equal_block_norm_rows(tab, n, seed):
    """Rows x whose rotated coordinates have the same norm in every block of
    32 (x = u R with u built block by block)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((n, 128))
    ub = u.reshape(n, 4, 32)
    ub /= np.linalg.norm(ub, axis=-1, keepdims=True)
    ub *= rng.uniform(0.5, 3.0, (n, 1, 1))
    return ub.reshape(n, 128) @ tab.R


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_block32_equal_block_norms_reduce_to_per_vector_codec(bits, oracle_tables):
    """With equal block norms n_b = ||x|| / 2, the block standardisation
    sqrt(32) u_b / n_b equals the per-vector sqrt(128) u / ||x||: codes, the
    projection P, gamma and both reconstructions coincide with the per-vector
    codec (fp16(n/2) = fp16(n)/2 exactly)."""
    tab = oracle_tables
    x = _equal_block_norm_rows(tab, 40, 7 + bits)
    a = O.encode(x, bits, True, tab)
    b = O.encode_block32(x, bits, True, tab)
    np.testing.assert_allclose(b["z"], a["z"], rtol=0, atol=1e-12)
    assert (b["idx"] == a["idx"]).all()
    np.testing.assert_allclose(b["P"], a["P"], rtol=0, atol=1e-9)
    assert (b["bits_qjl"] == a["bits_qjl"]).all()
    np.testing.assert_allclose(b["gamma64"], a["gamma64"], rtol=1e-12)
    assert (b["bnorm"] == (a["norm"][:, None] / 2).astype(np.float16)).all()
    np.testing.assert_allclose(O.dequant_mse32(b["idx"], b["bnorm"], bits, tab),
                               O.dequant_mse(a["idx"], a["norm"], bits, tab), rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.dequant_prod32(b["idx"], b["bits_qjl"], b["bnorm"], b["rnorm"], bits, tab),
                               O.dequant_prod(a["idx"], a["bits_qjl"], a["norm"], a["rnorm"], bits, tab),
                               rtol=0, atol=1e-12)


def test_block32_blocks_are_independent(oracle_tables):
    """Scaling one block of the rotated vector by a > 0 scales only that
    block's norm: every code is unchanged (the per-vector codec, whose single
    norm mixes the blocks, changes codes)."""
    tab = oracle_tables
    rng = np.random.default_rng(11)
    u = rng.standard_normal((30, 128))
    x = u @ tab.R
    u2 = u.copy()
    u2[:, 32:64] *= 9.0
    x2 = u2 @ tab.R
    a, b = O.encode_block32(x, 3, False, tab), O.encode_block32(x2, 3, False, tab)
    assert (a["idx"] == b["idx"]).all()
    np.testing.assert_allclose(b["bn64"][:, 1], 9.0 * a["bn64"][:, 1], rtol=1e-12)
    np.testing.assert_allclose(b["bn64"][:, [0, 2, 3]], a["bn64"][:, [0, 2, 3]], rtol=1e-12)
    assert (O.encode(x, 3, False, tab)["idx"] != O.encode(x2, 3, False, tab)["idx"]).any()


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_block32_gamma_is_stage1_residual_norm(bits, oracle_tables):
    """gamma = ||x - x_hat_1|| with x_hat_1 the Stage-1 reconstruction from
    the exact block norms (R is orthonormal), on rows with very uneven
    blocks; and the Stage-1 reconstruction error is below ||x||."""
    tab = oracle_tables
    rng = np.random.default_rng(21 + bits)
    u = rng.standard_normal((25, 128)) * np.repeat([0.01, 1.0, 30.0, 3.0], 32)
    x = u @ tab.R
    e = O.encode_block32(x, bits, True, tab)
    x1 = O.dequant_mse32(e["idx"], e["bn64"], bits, tab)
    np.testing.assert_allclose(e["gamma64"], np.linalg.norm(x - x1, axis=1), rtol=1e-10)
    assert (np.linalg.norm(x - x1, axis=1) < np.linalg.norm(x, axis=1)).all()


def test_block32_zero_vector(oracle_tables):
    """A zero vector has zero block norms, z = 0 (the upper middle index),
    no sign bit and gamma 0, and reconstructs to zero in both formats."""
    tab = oracle_tables
    x = np.zeros((2, 128))
    e = O.encode_block32(x, 2, True, tab)
    assert (e["idx"] == 2).all() and (e["bn64"] == 0).all()
    assert e["bits_qjl"].sum() == 0 and (e["gamma64"] == 0).all()
    np.testing.assert_allclose(O.dequant_mse32(e["idx"], e["bnorm"], 2, tab), 0.0, atol=0)
    np.testing.assert_allclose(O.dequant_prod32(e["idx"], e["bits_qjl"], e["bnorm"], e["rnorm"], 2, tab), 0.0,
                               atol=0)


def test_block32_finer_norms_help_uneven_vectors(oracle_tables):
    """On rows whose energy is concentrated in one block of the rotated
    coordinates, per-block norms cut the Stage-1 error at equal code bits (the
    codebook no longer sees a mixture of scales)."""
    tab = oracle_tables
    rng = np.random.default_rng(3)
    u = rng.standard_normal((400, 128)) * np.repeat([0.05, 0.05, 1.0, 0.05], 32)
    x = u @ tab.R
    e1, e2 = O.encode(x, 2, False, tab), O.encode_block32(x, 2, False, tab)
    m1 = O.quality(x, O.dequant_mse(e1["idx"], e1["norm"], 2, tab))["mse"]
    m2 = O.quality(x, O.dequant_mse32(e2["idx"], e2["bnorm"], 2, tab))["mse"]
    assert m2 < 0.5 * m1


def test_block32_qjl_projection_from_codes(oracle_tables):
    """The block-32 projection recomputed from the encoder's own codes is the
    encoder's P; with one block's codes moved one level its block residual,
    and so P, changes."""
    tab = oracle_tables
    x = np.random.default_rng(9).standard_normal((12, 128))
    e = O.encode_block32(x, 2, True, tab)
    np.testing.assert_allclose(O.qjl_projection_from_codes_block32(x, e["idx"], 2, tab), e["P"], rtol=0, atol=1e-12)
    idx2 = e["idx"].copy()
    idx2[:, 40] = np.where(idx2[:, 40] < 3, idx2[:, 40] + 1, idx2[:, 40] - 1)
    P2 = O.qjl_projection_from_codes_block32(x, idx2, 2, tab)
    u, nb, _ = O.block_standardised_rotation(x, tab)
    step = (tab.levels[2][idx2[:, 40]] - tab.levels[2][e["idx"][:, 40]]) * nb[:, 1] / math.sqrt(32)
    zs = math.sqrt(128) / np.linalg.norm(x, axis=1)
    np.testing.assert_allclose(P2 - e["P"], -(step * zs)[:, None] * tab.S[:, 40][None, :], rtol=1e-9, atol=1e-12)
