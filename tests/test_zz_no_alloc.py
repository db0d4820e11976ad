"""tq_attn_decode_noalloc (the attention entry point that allocates nothing,
for callers that cannot allocate) against tq_attn_decode through the C ABI:
two calls in a row, the second on a smaller input, on the single-launch path
(8 query heads per KV head, barrier counters in the library-owned array) and
on the two-pass path (4 query heads per KV head); a shape whose workspace
exceeds the array is refused without launching."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_encode_amd import turbokv as T
from kv_cache_quantization_encode_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _packed(ctx, case, kf, vf):
    k = np.ascontiguousarray(case.k.reshape(-1, 128))
    v = np.ascontiguousarray(case.v.reshape(-1, 128))
    kp, _ = G.gpu_encode(ctx, k, *kf)
    vp, _ = G.gpu_encode(ctx, v, *vf, as_v=True)
    return kp, vp


def _both(ctx, case, kp, vp, kf, vf, lens):
    B, Hq, Hkv, Tn = case.shape
    K, V = G.tf(*kf), G.tf(*vf)
    q = G.to_dev_f16(case.q)
    kd, vd = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    ld = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    ws, wsb = T.alloc_workspace(B, Hq, Hkv, Tn, K, V)
    ref = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    G.note(f"attn_decode B={B} Hq={Hq} Hkv={Hkv} T={Tn}")
    T.tq_attn_decode(ctx, q, kd, vd, K, V, B, Hq, Hkv, Tn, ld, 1e-6, ref, ws, wsb)
    G.note(f"attn_decode_noalloc B={B} Hq={Hq} Hkv={Hkv} T={Tn}")
    T.tq_attn_decode_noalloc(ctx, q, kd, vd, K, V, B, Hq, Hkv, Tn, ld, 1e-6, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("hq,kf,vf", [(16, ("prod", 2), ("mse", 2)), (8, ("prod", 3), ("mse", 4))])
def test_noalloc_matches_decode_two_calls(oracle_tables, hq, kf, vf):
    big = W.llama70b_layer(11, T=3000, Hkv=2, Hq=hq)
    small = W.slice_case(W.llama70b_layer(12, T=700, Hkv=2, Hq=hq), T=700)
    with G.Ctx(42) as ctx:
        for case, lens in ((big, None), (small, np.array([699], np.int32))):
            case = W.slice_case(case, B=1)
            kp, vp = _packed(ctx, case, kf, vf)
            got, ref = _both(ctx, case, kp, vp, kf, vf, lens)
            assert np.isfinite(got).all()
            # fp32 atomics add block shares in any order: last bits only
            assert np.max(np.abs(got - ref)) <= 1e-5
            exp = G.oracle_attention(case, kp, vp, kf[0], kf[1], vf[0], vf[1], oracle_tables, 1e-6, lens)
            assert np.max(np.abs(got - exp)) <= G.ATTN_ATOL


def test_noalloc_refuses_workspace_beyond_the_array():
    B, Hq, Hkv, Tn = 64, 32, 8, 8192
    K, V = T.turbo_k(4), T.mse(2)
    assert T.tq_attn_workspace_bytes(B, Hq, Hkv, Tn, K, V) > 8 << 20
    with G.Ctx(42) as ctx:
        q = torch.zeros((B, Hq, 128), dtype=torch.float16, device="cuda")
        buf = torch.zeros(256, dtype=torch.uint8, device="cuda")
        out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
        with pytest.raises(T.TqError) as e:
            T.tq_attn_decode_noalloc(ctx, q, buf, buf, K, V, B, Hq, Hkv, Tn, None, 1e-6, out)
        assert e.value.status == T.TQ_ERR_WORKSPACE
