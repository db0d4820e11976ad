"""GPU parity of the decode step with append (tq_attn_decode_append): after
the call the caches hold exactly the bytes tq_append_kv writes, and the
outputs equal the oracle's attention over the appended cache with
seq_lens = pos + 1 (clamped), and tq_attn_decode's on the same bytes up to
the last bits.  Covers the two-pass kernels (extra block per row), the
single-launch kernel (the block owning the position encodes), GQA 1/2/4/8,
ragged and out-of-range positions, and the formats that append in a
separate launch (q8, block-32)."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_encode_amd import turbokv as T
from kv_cache_quantization_encode_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

# name, B, Hq, Hkv, T_cap, K format, V format, positions
CASES = [
    ("gqa4-two-pass", 3, 32, 8, 1500, ("prod", 3), ("mse", 4), [1499, 700, 0]),
    ("gqa8-single-launch", 2, 64, 8, 5000, ("prod", 2), ("mse", 2), [4999, 2048]),
    ("gqa8-single-launch-turbo4", 1, 64, 8, 3000, ("prod", 3), ("mse", 2), [1023]),
    ("gqa8-two-pass-v3", 2, 64, 8, 700, ("prod", 2), ("mse", 3), [699, 300]),
    ("gqa1", 2, 4, 4, 600, ("prod", 1), ("mse", 1), [599, 17]),
    ("gqa2", 1, 8, 4, 1024, ("prod", 3), ("mse", 2), [512]),
    ("out-of-range", 3, 32, 8, 300, ("prod", 3), ("mse", 4), [-1, 300, 5]),
    ("q8-separate-append", 2, 64, 8, 1000, ("q8", 8), ("q8", 8), [999, 10]),
    ("block32-separate-append", 2, 32, 8, 400, ("prod32", 2), ("mse32", 2), [399, 0]),
]


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


def _encoded(ctx, k, v, kf, vf):
    """Bulk-encoded caches of k and v ([B, Hkv, T, 128]) in guarded buffers."""
    n = k.shape[0] * k.shape[1] * k.shape[2]
    kl = T.tq_packed_layout(G.tf(*kf), 128, n)
    vl = T.tq_packed_layout(G.tf(*vf), 128, n)
    kb, vb = G.Guarded(int(kl.total_bytes)), G.Guarded(int(vl.total_bytes))
    T.tq_encode_kv(ctx, G.to_dev_f16(k.reshape(-1, 128)), G.to_dev_f16(v.reshape(-1, 128)), n, G.tf(*kf),
                   G.tf(*vf), kb.ptr, vb.ptr)
    return kb, vb, kl, vl


def _step(ctx, q, k_new, v_new, pos, kb, vb, kf, vf, B, Hq, Hkv, Tc, tau, ws, wsb):
    out = G.Guarded(B * Hq * 128 * 4)
    p = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
    T.tq_attn_decode_append(ctx, G.to_dev_f16(q), G.to_dev_f16(k_new), G.to_dev_f16(v_new), p, kb.ptr, vb.ptr,
                            G.tf(*kf), G.tf(*vf), B, Hq, Hkv, Tc, tau, out.ptr, ws, wsb)
    h = out.host()
    out.check_guard(h)
    return h[: B * Hq * 128 * 4].view(np.float32).reshape(B, Hq, 128)


@pytest.mark.parametrize("name,B,Hq,Hkv,Tc,kf,vf,pos", CASES, ids=[c[0] for c in CASES])
def test_decode_append_matches_append_then_decode(ctx, oracle_tables, name, B, Hq, Hkv, Tc, kf, vf, pos):
    rng = np.random.default_rng(711)
    k = _rows(rng, (B, Hkv, Tc, 128))
    v = _rows(rng, (B, Hkv, Tc, 128))
    k_new = _rows(rng, (B, Hkv, 128))
    v_new = _rows(rng, (B, Hkv, 128))
    q = rng.standard_normal((B, Hq, 128), dtype=np.float32).astype(np.float16)
    tau = 1e-6
    wsb = T.tq_attn_workspace_bytes(B, Hq, Hkv, Tc, G.tf(*kf), G.tf(*vf))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    # reference path: the separate append, then decode over pos + 1
    ka, va, kl, vl = _encoded(ctx, k, v, kf, vf)
    G.note(f"{name}: tq_append_kv then tq_attn_decode, pos={pos}")
    p = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
    T.tq_append_kv(ctx, G.to_dev_f16(k_new), G.to_dev_f16(v_new), B, Hkv, Tc, p, G.tf(*kf), G.tf(*vf), ka.ptr,
                   va.ptr)
    lens = np.asarray(pos, np.int64) + 1
    out_ref = G.Guarded(B * Hq * 128 * 4)
    T.tq_attn_decode(ctx, G.to_dev_f16(q), ka.ptr, va.ptr, G.tf(*kf), G.tf(*vf), B, Hq, Hkv, Tc,
                     torch.from_numpy(np.clip(lens, -1, Tc + 1).astype(np.int32)).cuda(), tau, out_ref.ptr, ws,
                     wsb)
    two = out_ref.host()[: B * Hq * 128 * 4].view(np.float32).reshape(B, Hq, 128)
    # the fused step on a second copy of the same caches
    kb, vb, _, _ = _encoded(ctx, k, v, kf, vf)
    G.note(f"{name}: tq_attn_decode_append B={B} Hq={Hq} Hkv={Hkv} T_cap={Tc} kf={kf} vf={vf}")
    got = _step(ctx, q, k_new, v_new, pos, kb, vb, kf, vf, B, Hq, Hkv, Tc, tau, ws, wsb)
    hk, hv = kb.host(), vb.host()
    kb.check_guard(hk, G.plane_ranges(kl))
    vb.check_guard(hv, G.plane_ranges(vl))
    assert np.array_equal(hk, ka.host()), "K cache differs from tq_append_kv's"
    assert np.array_equal(hv, va.host()), "V cache differs from tq_append_kv's"
    # against the oracle over the appended bytes
    k_ref, v_ref = k.copy(), v.copy()
    for b, pb in enumerate(pos):
        if 0 <= pb < Tc:
            k_ref[b, :, pb] = k_new[b]
            v_ref[b, :, pb] = v_new[b]
    case = W.AttnCase(name, k_ref, v_ref, q)
    kp, vp = hk[: kl.total_bytes].copy(), hv[: vl.total_bytes].copy()
    ref = G.oracle_attention(case, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, tau, lens)
    err = float(np.max(np.abs(got - ref)))
    assert err <= G.ATTN_ATOL, f"max abs error {err:.3g} against the oracle"
    scale = max(1.0, float(np.max(np.abs(ref))))
    gap = float(np.max(np.abs(got - two)))
    assert gap <= 1e-5 * scale, f"differs from append + decode by {gap:.3g}"
    # an out-of-range position attends over its clamped length, a negative one
    # over nothing
    for b, pb in enumerate(pos):
        if pb < 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("Hq,kf,vf", [(32, ("prod", 3), ("mse", 4)), (64, ("prod", 2), ("mse", 2))],
                         ids=["gqa4-two-pass", "gqa8-single-launch"])
def test_decode_loop_with_append(ctx, oracle_tables, Hq, kf, vf):
    """Four decode steps on one workspace: each step appends every
    sequence's new K/V at its own position inside the attention launch; each
    step's output against the oracle, and the appended rows against the
    oracle's encode at the end."""
    rng = np.random.default_rng(712)
    B, Hkv, Tc = 2, 8, 2600
    k = _rows(rng, (B, Hkv, Tc, 128))
    v = _rows(rng, (B, Hkv, Tc, 128))
    start = np.array([2044, 1535], np.int32)  # crosses 512- and 2048-token block edges
    kb, vb, kl, vl = _encoded(ctx, k, v, kf, vf)
    wsb = T.tq_attn_workspace_bytes(B, Hq, Hkv, Tc, G.tf(*kf), G.tf(*vf))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for step in range(4):
        pos = start + step
        k_new = _rows(rng, (B, Hkv, 128))
        v_new = _rows(rng, (B, Hkv, 128))
        q = rng.standard_normal((B, Hq, 128), dtype=np.float32).astype(np.float16)
        for b in range(B):
            k[b, :, pos[b]] = k_new[b]
            v[b, :, pos[b]] = v_new[b]
        G.note(f"decode loop with append, step {step}, pos={pos.tolist()}, Hq={Hq}")
        got = _step(ctx, q, k_new, v_new, pos, kb, vb, kf, vf, B, Hq, Hkv, Tc, 1e-6, ws, wsb)
        kp = kb.host()[: kl.total_bytes].copy()
        vp = vb.host()[: vl.total_bytes].copy()
        case = W.AttnCase("decode-loop-append", k, v, q)
        ref = G.oracle_attention(case, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, 1e-6, pos + 1)
        err = float(np.max(np.abs(got - ref)))
        assert err <= G.ATTN_ATOL, f"step {step}: max abs error {err:.3g}"
    # the barrier region of the workspace is back at zero after the calls
    assert int(ws[:68 * 1024].count_nonzero().item()) == 0
    G.check_encode(k.reshape(-1, 128), *kf, kb.host()[: kl.total_bytes], oracle_tables)
    G.check_encode(v.reshape(-1, 128), *vf, vb.host()[: vl.total_bytes], oracle_tables)
