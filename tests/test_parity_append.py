"""GPU parity of the per-token append (tq_append_kv): new rows written into a
[B, Hkv, T_cap] packed cache must be byte-identical to a bulk encode of the
cache that holds them, leave every other row untouched, and serve a decode
loop (append, then attention over seq_lens = pos + 1) that matches the
oracle's attention over the same bytes."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_encode_amd import turbokv as T
from kv_cache_quantization_encode_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

FORMATS = [(("prod", 3), ("mse", 4)), (("prod", 2), ("mse", 2)), (("prod", 1), ("mse", 3)),
           (("mse", 1), ("q8", 8)), (("q8", 8), ("mse", 2)), (("prod32", 2), ("mse32", 2)),
           (("mse32", 3), ("mse32", 4))]


@pytest.fixture(scope="module")
def ctx():
    with G.Ctx(42) as h:
        yield h


def _rows(rng, shape):
    """N(0,1) rows with 4 outlier channels x20 (the tiny workload's law)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    ch = rng.choice(128, 4, replace=False)
    x[..., ch] *= 20.0
    return x.astype(np.float16)


def _bulk(ctx, cache16, f, as_v):
    """Bulk-encode [n, 128] rows into a guarded buffer (device)."""
    n = cache16.shape[0]
    lay = T.tq_packed_layout(G.tf(*f), 128, n)
    buf = G.Guarded(int(lay.total_bytes))
    x = G.to_dev_f16(cache16)
    G.note(f"bulk encode {f} n={n}")
    if as_v:
        T.tq_encode_kv(ctx, None, x, n, G.tf(*f), G.tf(*f), None, buf.ptr)
    else:
        T.tq_encode_kv(ctx, x, None, n, G.tf(*f), G.tf(*f), buf.ptr, None)
    return buf, lay


@pytest.mark.parametrize("kf,vf", FORMATS)
def test_append_equals_bulk_encode(ctx, oracle_tables, kf, vf):
    rng = np.random.default_rng(611)
    B, Hkv, Tc = 3, 5, 37  # 555 cache rows: several 16-row tiles and a ragged one
    k = _rows(rng, (B, Hkv, Tc, 128))
    v = _rows(rng, (B, Hkv, Tc, 128))
    k_new = _rows(rng, (B, Hkv, 128))
    v_new = _rows(rng, (B, Hkv, 128))
    for pos in ([5, 36, 0], [-1, Tc, 17]):  # the second: two sequences out of range
        kb, klay = _bulk(ctx, k.reshape(-1, 128), kf, False)
        vb, vlay = _bulk(ctx, v.reshape(-1, 128), vf, True)
        p = torch.tensor(pos, dtype=torch.int32, device="cuda")
        G.note(f"append kf={kf} vf={vf} pos={pos}")
        T.tq_append_kv(ctx, G.to_dev_f16(k_new), G.to_dev_f16(v_new), B, Hkv, Tc, p, G.tf(*kf), G.tf(*vf),
                       kb.ptr, vb.ptr)
        got_k, got_v = kb.host(), vb.host()
        kb.check_guard(got_k, G.plane_ranges(klay))
        vb.check_guard(got_v, G.plane_ranges(vlay))
        k_ref, v_ref = k.copy(), v.copy()
        for b, pb in enumerate(pos):
            if 0 <= pb < Tc:
                k_ref[b, :, pb] = k_new[b]
                v_ref[b, :, pb] = v_new[b]
        ek, _ = _bulk(ctx, k_ref.reshape(-1, 128), kf, False)
        ev, _ = _bulk(ctx, v_ref.reshape(-1, 128), vf, True)
        assert np.array_equal(got_k, ek.host()), "appended K cache differs from the bulk encode"
        assert np.array_equal(got_v, ev.host()), "appended V cache differs from the bulk encode"
        # the rows themselves against the oracle
        n = B * Hkv * Tc
        G.check_encode(k_ref.reshape(-1, 128), *kf, got_k[: klay.total_bytes], oracle_tables)
        G.check_encode(v_ref.reshape(-1, 128), *vf, got_v[: vlay.total_bytes], oracle_tables)
        assert n == B * Hkv * Tc


def test_decode_loop_append_then_attend(ctx, oracle_tables):
    """Prefill part of a cache, then three decode steps: append each
    sequence's new K/V at its own position and attend with seq_lens = pos+1
    (GQA 4, turbo4 K + 4-bit V, sparse V at 1e-6)."""
    rng = np.random.default_rng(612)
    B, Hq, Hkv, Tc = 2, 8, 2, 300
    kf, vf = ("prod", 3), ("mse", 4)
    k = _rows(rng, (B, Hkv, Tc, 128))
    v = _rows(rng, (B, Hkv, Tc, 128))
    start = np.array([200, 131], np.int32)
    kb, klay = _bulk(ctx, k.reshape(-1, 128), kf, False)
    vb, vlay = _bulk(ctx, v.reshape(-1, 128), vf, True)
    for step in range(3):
        pos = start + step
        k_new = _rows(rng, (B, Hkv, 128))
        v_new = _rows(rng, (B, Hkv, 128))
        q = rng.standard_normal((B, Hq, 128), dtype=np.float32).astype(np.float16)
        for b in range(B):
            k[b, :, pos[b]] = k_new[b]
            v[b, :, pos[b]] = v_new[b]
        G.note(f"decode loop step {step} pos={pos.tolist()}")
        T.tq_append_kv(ctx, G.to_dev_f16(k_new), G.to_dev_f16(v_new), B, Hkv, Tc,
                       torch.from_numpy(pos).cuda(), G.tf(*kf), G.tf(*vf), kb.ptr, vb.ptr)
        kp = kb.host()[: klay.total_bytes].copy()
        vp = vb.host()[: vlay.total_bytes].copy()
        case = W.AttnCase("decode-loop", k, v, q)
        lens = pos + 1
        got = G.gpu_attention(ctx, case, kp, vp, G.tf(*kf), G.tf(*vf), 1e-6, lens)
        ref = G.oracle_attention(case, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, 1e-6, lens)
        err = float(np.max(np.abs(got - ref)))
        assert err <= G.ATTN_ATOL, f"step {step}: max abs error {err:.3g}"
    # the rows the loop appended are the oracle's encode of the new tokens
    G.check_encode(k.reshape(-1, 128), *kf, kb.host()[: klay.total_bytes], oracle_tables)
    G.check_encode(v.reshape(-1, 128), *vf, vb.host()[: vlay.total_bytes], oracle_tables)


def test_append_many_sequences(ctx, oracle_tables):
    """64 sequences x 8 KV heads (512 new rows: several blocks per tensor in
    the joint K+V launch), each sequence at its own position of a 24-token
    cache; turbo4 K + 2-bit V as in the batched needle workload."""
    rng = np.random.default_rng(613)
    B, Hkv, Tc = 64, 8, 24
    kf, vf = ("prod", 3), ("mse", 2)
    k = _rows(rng, (B, Hkv, Tc, 128))
    v = _rows(rng, (B, Hkv, Tc, 128))
    k_new = _rows(rng, (B, Hkv, 128))
    v_new = _rows(rng, (B, Hkv, 128))
    pos = rng.integers(0, Tc, size=B).astype(np.int32)
    kb, klay = _bulk(ctx, k.reshape(-1, 128), kf, False)
    vb, vlay = _bulk(ctx, v.reshape(-1, 128), vf, True)
    G.note(f"append B={B} Hkv={Hkv} Tc={Tc}")
    T.tq_append_kv(ctx, G.to_dev_f16(k_new), G.to_dev_f16(v_new), B, Hkv, Tc, torch.from_numpy(pos).cuda(),
                   G.tf(*kf), G.tf(*vf), kb.ptr, vb.ptr)
    got_k, got_v = kb.host(), vb.host()
    kb.check_guard(got_k, G.plane_ranges(klay))
    vb.check_guard(got_v, G.plane_ranges(vlay))
    for b in range(B):
        k[b, :, pos[b]] = k_new[b]
        v[b, :, pos[b]] = v_new[b]
    ek, _ = _bulk(ctx, k.reshape(-1, 128), kf, False)
    ev, _ = _bulk(ctx, v.reshape(-1, 128), vf, True)
    assert np.array_equal(got_k, ek.host()), "appended K cache differs from the bulk encode"
    assert np.array_equal(got_v, ev.host()), "appended V cache differs from the bulk encode"
    G.check_encode(k.reshape(-1, 128), *kf, got_k[: klay.total_bytes], oracle_tables)
    G.check_encode(v.reshape(-1, 128), *vf, got_v[: vlay.total_bytes], oracle_tables)
