"""GPU parity of the block-32 norm formats (one fp16 Stage-1 norm per block of
32 rotated coordinates; yeyulingfeng.com "TurboQuant+: 3.8x compression ...",
technical highlights, block-32 storage) against the CPU oracle: encode,
dequant and decode attention, alone and paired with the per-vector formats."""
import numpy as np
import pytest

from kv_cache_quantization_encode_amd import workloads as W
from oracle import turbokv_oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

B32 = [("mse32", 1), ("mse32", 2), ("mse32", 3), ("mse32", 4), ("prod32", 1), ("prod32", 2), ("prod32", 3)]


@pytest.fixture(scope="module")
def ctx():
    with G.Ctx(42) as h:
        yield h


def _uneven_rows(n, seed):
    """N(0,1) rows with 4 outlier channels x20 and per-row scales spread
    over 4 decades (the tiny workload's law, widened)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128))
    x[:, rng.choice(128, 4, replace=False)] *= 20.0
    x *= 10.0 ** rng.uniform(-2, 2, (n, 1))
    return x.astype(np.float16)


@pytest.mark.parametrize("kind,bits", B32)
@pytest.mark.parametrize("n", [1, 17, 2061])
def test_block32_encode_and_dequant(ctx, oracle_tables, kind, bits, n):
    x = _uneven_rows(n, 100 + n + bits)
    for as_v in (False, True):
        if as_v and kind == "prod32":
            continue
        packed, _ = G.gpu_encode(ctx, x, kind, bits, as_v=as_v)
        G.check_encode(x, kind, bits, packed, oracle_tables)
        got = G.gpu_decode(ctx, packed, kind, bits, n)
        ref = O.dequant_packed(packed, kind, bits, oracle_tables, n)
        G.check_rows_close(got, ref)


def test_block32_encode_llama_rows(ctx, oracle_tables):
    """The llama8b-like K law (lognormal channel scales, Student-t noise)."""
    c = W.llama8b(T=700, Hkv=2)
    x = np.ascontiguousarray(c.k.reshape(-1, 128))
    for kind, bits in (("prod32", 2), ("prod32", 3), ("mse32", 2), ("mse32", 4)):
        packed, _ = G.gpu_encode(ctx, x, kind, bits)
        G.check_encode(x, kind, bits, packed, oracle_tables)


def test_block32_degenerate_rows(ctx, oracle_tables):
    """A zero row (all block norms 0, no sign bit), a one-hot row, fp16 max
    everywhere and subnormal rows: bytes within the parity rules, and the
    zero row decodes to zeros."""
    x = np.zeros((40, 128), np.float16)
    x[1, 5] = 1.0
    x[2] = 65504.0
    x[3] = np.float16(6e-8)
    x[4, ::2] = -3.0
    x[5:] = np.random.default_rng(0).standard_normal((35, 128)).astype(np.float16)
    for kind, bits in B32:
        packed, _ = G.gpu_encode(ctx, x, kind, bits)
        u = O.unpack_tq(packed, kind, bits, 128, 40)
        assert (u["bnorm"][0] == 0).all() and (u["idx"][0] == (1 << (bits - 1))).all()
        if kind == "prod32":
            assert u["bits_qjl"][0].sum() == 0 and u["rnorm"][0] == 0
        G.check_encode(x[5:], kind, bits, G.sub_packed(packed, kind, bits, 40, 5, 35), oracle_tables)
        got = G.gpu_decode(ctx, packed, kind, bits, 40)
        assert (got[0] == 0).all()


PAIRS = [(("prod32", 2), ("mse32", 2)), (("prod32", 3), ("mse32", 3)), (("prod32", 1), ("mse32", 1)),
         (("mse32", 4), ("mse32", 4)), (("prod", 2), ("mse32", 2)), (("prod32", 2), ("mse", 2)),
         (("q8", 8), ("mse32", 2)), (("prod32", 2), ("q8", 8))]


@pytest.mark.parametrize("kf,vf", PAIRS)
def test_block32_attention_formats(ctx, oracle_tables, kf, vf):
    c = W.slice_case(W.llama8b(T=1500, Hkv=2, Hq=8), T=1333)
    k = np.ascontiguousarray(c.k.reshape(-1, 128))
    v = np.ascontiguousarray(c.v.reshape(-1, 128))
    kp, _ = G.gpu_encode(ctx, k, *kf)
    vp, _ = G.gpu_encode(ctx, v, *vf, as_v=True)
    got = G.gpu_attention(ctx, c, kp, vp, G.tf(*kf), G.tf(*vf), 1e-6)
    ref = G.oracle_attention(c, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, 1e-6)
    err = np.max(np.abs(got - ref))
    assert err <= G.ATTN_ATOL, f"max abs error {err:.3g}"


@pytest.mark.parametrize("g", [1, 2, 8])
def test_block32_attention_gqa_and_lengths(ctx, oracle_tables, g):
    """GQA ratios 1, 2, 8 and ragged, empty and over-long sequence lengths."""
    base = W.llama70b_layer(9, T=900, Hkv=2, Hq=2 * g)
    c = W.AttnCase("b32.gqa", np.concatenate([base.k, base.k[:, :, ::-1]]),
                   np.concatenate([base.v, base.v[:, :, ::-1]]), np.concatenate([base.q, base.q[:, ::-1]]))
    kf, vf = ("prod32", 2), ("mse32", 2)
    k = np.ascontiguousarray(c.k.reshape(-1, 128))
    v = np.ascontiguousarray(c.v.reshape(-1, 128))
    kp, _ = G.gpu_encode(ctx, k, *kf)
    vp, _ = G.gpu_encode(ctx, v, *vf, as_v=True)
    for lens in ([900, 900], [641, 0], [5000, 1]):
        got = G.gpu_attention(ctx, c, kp, vp, G.tf(*kf), G.tf(*vf), 1e-6, lens)
        ref = G.oracle_attention(c, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, 1e-6, lens)
        err = np.max(np.abs(got - ref))
        assert err <= G.ATTN_ATOL, f"lens {lens}: max abs error {err:.3g}"


def test_block32_attention_tau_zero_and_peaked(ctx, oracle_tables):
    """tau = 0 keeps every row; a needle-peaked softmax skips almost all."""
    n = W.needle(B=2, T=1024, Hq=16, Hkv=2)
    kf, vf = ("prod32", 3), ("mse32", 2)
    k = np.ascontiguousarray(n.k.reshape(-1, 128))
    v = np.ascontiguousarray(n.v.reshape(-1, 128))
    kp, _ = G.gpu_encode(ctx, k, *kf)
    vp, _ = G.gpu_encode(ctx, v, *vf, as_v=True)
    for tau in (0.0, 1e-6):
        got = G.gpu_attention(ctx, n, kp, vp, G.tf(*kf), G.tf(*vf), tau)
        ref = G.oracle_attention(n, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, tau)
        err = np.max(np.abs(got - ref))
        assert err <= G.ATTN_ATOL, f"tau {tau}: max abs error {err:.3g}"
