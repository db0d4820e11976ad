"""Planted-mistake sweep over the CPU oracle.

Each case replaces one oracle function with a copy that carries one plausible
mistake (a dropped term, a wrong constant, a transposed operand, a strict
comparison, a wrong index map, a different bit order) and checks that at least
one of the named pins in tests/test_oracle_pins.py then fails with an
assertion.  The pins themselves pass on the unmodified oracle (the ordinary
run of that file), so every mistake listed here is caught by something that
does not come from the oracle.
"""
import math

import numpy as np
import pytest
from scipy import special

from oracle import turbokv_oracle as O
from tests import test_oracle_pins as P

# ---------------------------------------------------------------- mistakes
_orig = {name: getattr(O, name) for name in (
    "rotation", "encode", "qjl_projection_from_codes", "dequant_mse", "dequant_prod", "qjl_inner_product",
    "quantise_index", "minmax_quant", "attention_decode", "attention_prefill", "pack_bitstream", "q8_quant",
    "quality", "lloyd_max_gaussian", "splitmix64_outputs", "standardised_rotation",
    "block_standardised_rotation", "encode_block32", "qjl_projection_from_codes_block32", "dequant_mse32",
    "dequant_prod32")}


def m_rotation_transposed(signs):
    d = signs.shape[0]
    return (O.hadamard(d) * signs[None, :] / math.sqrt(d)).T


def m_qjl_projection_S_not_ST(x, idx, bits, tab):
    _, z = _orig["standardised_rotation"](x, tab)
    return (z - tab.levels[bits][idx]) @ tab.S


def m_encode_projection_transposed(x, bits, prod, tab):
    out = _orig["encode"](x, bits, prod, tab)
    if prod:
        P_ = out["e"] @ tab.S
        out.update(P=P_, bits_qjl=(P_ > 0).astype(np.uint8))
    return out


def m_encode_gamma_without_norm(x, bits, prod, tab):
    out = _orig["encode"](x, bits, prod, tab)
    if prod:
        g = np.sqrt(np.sum(out["e"] ** 2, axis=-1)) / math.sqrt(tab.d)
        out.update(gamma64=g, rnorm=g.astype(np.float16))
    return out


def m_dequant_mse_no_norm(idx, norm16, bits, tab):
    return _orig["dequant_mse"](idx, np.ones_like(np.asarray(norm16, np.float64)), bits, tab)


def m_dequant_prod_wrong_constant(idx, bits_qjl, norm16, rnorm16, bits, tab):
    # sqrt(2/pi) in place of sqrt(pi/2)
    return _orig["dequant_prod"](idx, bits_qjl, norm16, np.asarray(rnorm16, np.float64) * (2.0 / math.pi), bits, tab)


def m_qjl_ip_wrong_constant(q, bits_qjl, gamma, tab):
    return _orig["qjl_inner_product"](q, bits_qjl, gamma, tab) * (2.0 / math.pi)


def m_quantise_strict(z, bounds):
    return np.sum(z[..., None] > bounds, axis=-1).astype(np.int64)


def _minmax_variant(x, group, bits, qmax_div, rounder):
    x16 = np.asarray(x, dtype=np.float16).reshape(-1)
    xg = x16.reshape(-1, group)
    mn = xg.min(axis=1).astype(np.float64)
    mx = xg.max(axis=1).astype(np.float64)
    qmax = (1 << bits) - 1
    scale = ((mx - mn) / qmax_div).astype(np.float16)
    zero = mn.astype(np.float16)
    s32 = scale.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xg.astype(np.float32) - zero.astype(np.float32)[:, None]) / np.where(s32 > 0, s32, 1)[:, None]
    code = np.where((s32 > 0)[:, None], np.clip(rounder(ratio), 0, qmax), 0).astype(np.int64)
    return code.reshape(-1), scale, zero


def m_minmax_floor(x, group=64, bits=3):
    return _minmax_variant(x, group, bits, (1 << bits) - 1, np.floor)


def m_minmax_divisor(x, group=64, bits=3):
    return _minmax_variant(x, group, bits, 1 << bits, np.rint)


def _attention_variant(q, k_hat, v_hat, tau=1e-6, seq_lens=None, scale=None, gqa=None, keep=None):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, T = k_hat.shape[1], k_hat.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d))
    probs = np.zeros((B, Hq, T))
    for b in range(B):
        L = T if seq_lens is None else min(max(int(seq_lens[b]), 0), T)
        for h in range(Hq):
            kv = gqa(h, g, Hkv) if gqa else h // g
            if L == 0:
                continue
            s = k_hat[b, kv, :L] @ q[b, h] * (scale(d) if scale else 1 / math.sqrt(d))
            p = special.softmax(s)
            kp = keep(p, tau) if keep else p >= tau
            out[b, h] = (p * kp) @ v_hat[b, kv, :L]
            probs[b, h, :L] = p
    return out, probs


def m_attention_no_scale(q, k, v, tau=1e-6, seq_lens=None):
    return _attention_variant(q, k, v, tau, seq_lens, scale=lambda d: 1.0)


def m_attention_gqa_modulo(q, k, v, tau=1e-6, seq_lens=None):
    return _attention_variant(q, k, v, tau, seq_lens, gqa=lambda h, g, hkv: h % hkv)


def m_attention_strict_tau(q, k, v, tau=1e-6, seq_lens=None):
    return _attention_variant(q, k, v, tau, seq_lens, keep=lambda p, t: p > t)


def m_attention_no_clamp(q, k_hat, v_hat, tau=1e-6, seq_lens=None):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, T = k_hat.shape[1], k_hat.shape[2]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = T if seq_lens is None else int(seq_lens[b])
        for h in range(Hq):
            if L == 0:
                continue
            s = k_hat[b, h // (Hq // Hkv), :L] @ q[b, h] / math.sqrt(d)
            p = special.softmax(s)
            out[b, h] = (p * (p >= tau)) @ v_hat[b, h // (Hq // Hkv), :L]
    return out, None


def m_prefill_off_by_one(q, k_hat, v_hat, tau=1e-6, seq_lens=None):
    q = np.asarray(q, dtype=np.float64)
    B, Tq, Hq, d = q.shape
    T = k_hat.shape[2]
    out = np.zeros((B, Tq, Hq, d))
    for b in range(B):
        L = T if seq_lens is None else min(max(int(seq_lens[b]), 0), T)
        for i in range(Tq):
            n = max(L - Tq + i, 0)  # a query that does not see its own token
            o, _ = _orig["attention_decode"](q[b:b + 1, i], k_hat[b:b + 1], v_hat[b:b + 1], tau, [n])
            out[b, i] = o[0]
    return out


def m_pack_msb_first(codes, bits):
    codes = np.asarray(codes, dtype=np.int64)
    n, k = codes.shape
    bitmat = ((codes[..., None] >> np.arange(bits)) & 1).reshape(n, k * bits).astype(np.uint8)
    return np.packbits(bitmat, axis=1, bitorder="big")


def m_q8_divisor_128(x, block=32):
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    xb = x.reshape(n, d // block, block)
    scale = (np.max(np.abs(xb), axis=-1) / 128.0).astype(np.float16)
    s64 = scale.astype(np.float64)
    q = np.where(s64[..., None] > 0, np.rint(xb / np.where(s64 > 0, s64, 1)[..., None]), 0)
    return np.clip(q, -127, 127).astype(np.int8).reshape(n, d), scale


def m_quality_norm_squared(x, xhat, d=128):
    x = np.asarray(x, np.float64).reshape(-1)
    xhat = np.asarray(xhat, np.float64).reshape(-1)
    mse = float(np.mean((x - xhat) ** 2))
    cos = float(x @ xhat / (x @ x + 1e-300))
    xv, hv = x.reshape(-1, d), xhat.reshape(-1, d)
    per = np.sum(xv * hv, axis=1) / np.sum(xv * xv, axis=1)
    return {"mse": mse, "cos_flat": cos, "cos_vec_mean": float(per.mean())}


def m_lloyd_cell_midpoint(bits, tol=1e-14, max_iter=2000):
    # levels at the middle of the initial equal-probability cells: no Lloyd iteration
    L = 1 << bits
    c = special.ndtri((np.arange(L) + 0.5) / L)
    return c, 0.5 * (c[:-1] + c[1:])


def m_splitmix_wrong_shift(seed, count, first_counter=1):
    i = np.arange(first_counter, first_counter + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * O._GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(31))) * O._MIX1
        z = (z ^ (z >> np.uint64(27))) * O._MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def m_standardised_no_normalise(x, tab):
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    return n, math.sqrt(tab.d) * (x @ tab.R.T)


def m_block_scale_sqrt_d(x, tab, block=32):
    u, nb, z = _orig["block_standardised_rotation"](x, tab, block)
    return u, nb, z * math.sqrt(tab.d / block)


def m_block_norms_before_rotation(x, tab, block=32):
    x = np.asarray(x, dtype=np.float64)
    u = x @ tab.R.T
    nb = np.sqrt(np.sum(x.reshape(*x.shape[:-1], tab.d // block, block) ** 2, axis=-1))
    safe = np.where(nb > 0, nb, 1.0)
    z = u.reshape(*u.shape[:-1], tab.d // block, block) / safe[..., None] * math.sqrt(block)
    return u, nb, z.reshape(u.shape)


def m_block_residual_in_block_units(x, bits, prod, tab, block=32):
    out = _orig["encode_block32"](x, bits, prod, tab, block)
    if prod:
        r = out["z"] - tab.levels[bits][out["idx"]]
        g = np.sqrt(np.sum(r * r, axis=-1))
        out.update(gamma64=g, rnorm=g.astype(np.float16))
    return out


def m_block_check_without_scale(x, idx, bits, tab, block=32):
    _, _, z = O.block_standardised_rotation(x, tab, block)
    return (z - tab.levels[bits][idx]) @ tab.S.T


def m_dequant_mse32_sqrt_d(idx, bnorm16, bits, tab, block=32):
    return _orig["dequant_mse32"](idx, np.asarray(bnorm16, np.float64) * math.sqrt(block / tab.d), bits, tab, block)


def m_dequant_prod32_no_qjl(idx, bits_qjl, bnorm16, rnorm16, bits, tab, block=32):
    return _orig["dequant_mse32"](idx, bnorm16, bits, tab, block)


# ------------------------------------------------------------------- pins
def _tab():
    return O.Tables(128, seed=42)


PINS = {
    "dense_rotation": lambda: [P.test_dense_rotation_equals_fast_transform(d) for d in (8, 128)],
    "hadamard": lambda: [P.test_hadamard_matches_library_and_orthogonality(d) for d in (8, 32, 128)],
    "rotation_direction": lambda: [P.test_rotation_direction_and_residual(b, _tab()) for b in (1, 2, 3, 4)],
    "qjl_unbiased": lambda: P.test_qjl_unbiased_across_seeds(_tab()),
    "qjl_zero_residual": lambda: P.test_qjl_zero_residual_adds_nothing(_tab()),
    "prod_inner_product": lambda: P.test_prod_dequant_inner_product_is_stage1_plus_qjl(_tab()),
    "qjl_from_codes": lambda: P.test_qjl_projection_from_codes_matches_encode_and_permutation(_tab()),
    "mse_distortion": lambda: [P.test_mse_codec_distortion_matches_codebook(b, _tab()) for b in (1, 2, 3, 4)],
    "ties": lambda: P.test_quantiser_ties_go_up_and_zero_vector(_tab()),
    "brute_force": lambda: [P.test_quantiser_brute_force_d8(b) for b in (1, 2)],
    "minmax_example": lambda: P.test_minmax_worked_example(),
    "minmax_bound": lambda: [P.test_minmax_error_bound_and_degenerate(b) for b in (2, 3, 4)],
    "bitstream": lambda: P.test_minmax_bitstream_roundtrip(),
    "sdpa": lambda: P.test_attention_tau0_equals_library_sdpa(),
    "attn_special": lambda: P.test_attention_special_cases(),
    "attn_clamp": lambda: P.test_attention_decode_clamps_lengths(),
    "prefill_sdpa": lambda: P.test_prefill_tau0_equals_library_causal_sdpa(),
    "prefill_special": lambda: P.test_prefill_special_cases(),
    "q8": lambda: P.test_q8_invariants(),
    "quality": lambda: P.test_quality_closed_forms(),
    "codebook": lambda: [P.test_codebook_textbook_levels(b, _tab()) for b in (1, 2, 3, 4)],
    "splitmix": lambda: P.test_splitmix64_published_vectors(),
    "rotated_scores": lambda: P.test_rotated_domain_scores_equal_dense_scores(_tab()),
    "block32_equal_norms": lambda: [P.test_block32_equal_block_norms_reduce_to_per_vector_codec(b, _tab())
                                    for b in (1, 2, 3, 4)],
    "block32_independent": lambda: P.test_block32_blocks_are_independent(_tab()),
    "block32_gamma": lambda: [P.test_block32_gamma_is_stage1_residual_norm(b, _tab()) for b in (1, 2, 3)],
    "block32_from_codes": lambda: P.test_block32_qjl_projection_from_codes(_tab()),
}

# mistake -> (oracle function replaced, replacement, pins expected to catch it)
MUTATIONS = {
    "rotation transposed": ("rotation", m_rotation_transposed, ["dense_rotation", "rotation_direction"]),
    "QJL check projects with S, not S^T": ("qjl_projection_from_codes", m_qjl_projection_S_not_ST,
                                           ["qjl_from_codes"]),
    "encoder projects with S^T": ("encode", m_encode_projection_transposed, ["qjl_unbiased", "qjl_from_codes"]),
    "residual norm without the vector norm": ("encode", m_encode_gamma_without_norm, ["qjl_unbiased"]),
    "V dequant drops the norm": ("dequant_mse", m_dequant_mse_no_norm, ["qjl_zero_residual", "prod_inner_product"]),
    "K dequant with sqrt(2/pi)": ("dequant_prod", m_dequant_prod_wrong_constant, ["prod_inner_product"]),
    "QJL estimator with sqrt(2/pi)": ("qjl_inner_product", m_qjl_ip_wrong_constant, ["qjl_unbiased"]),
    "ties go down": ("quantise_index", m_quantise_strict, ["ties"]),
    "min-max floor instead of round": ("minmax_quant", m_minmax_floor, ["minmax_example", "minmax_bound"]),
    "min-max scale over 2^b": ("minmax_quant", m_minmax_divisor, ["minmax_example", "minmax_bound"]),
    "scores without 1/sqrt(d)": ("attention_decode", m_attention_no_scale, ["sdpa"]),
    "GQA head map h mod Hkv": ("attention_decode", m_attention_gqa_modulo, ["sdpa"]),
    "sparse V keeps only p > tau": ("attention_decode", m_attention_strict_tau, ["attn_special"]),
    "lengths not clamped": ("attention_decode", m_attention_no_clamp, ["attn_clamp"]),
    "prefill query misses its own token": ("attention_prefill", m_prefill_off_by_one,
                                           ["prefill_sdpa", "prefill_special"]),
    "bitstream MSB-first": ("pack_bitstream", m_pack_msb_first, ["bitstream"]),
    "q8 scale over 128": ("q8_quant", m_q8_divisor_128, ["q8"]),
    "cosine over ||x||^2": ("quality", m_quality_norm_squared, ["quality"]),
    "codebook without Lloyd iterations": ("lloyd_max_gaussian", m_lloyd_cell_midpoint, ["codebook"]),
    "splitmix64 first shift 31": ("splitmix64_outputs", m_splitmix_wrong_shift, ["splitmix"]),
    "rotation not normalised by the norm": ("standardised_rotation", m_standardised_no_normalise,
                                            ["rotation_direction", "mse_distortion"]),
    "block standardised with sqrt(d)": ("block_standardised_rotation", m_block_scale_sqrt_d,
                                        ["block32_equal_norms"]),
    "block norms taken before the rotation": ("block_standardised_rotation", m_block_norms_before_rotation,
                                              ["block32_equal_norms", "block32_independent"]),
    "block-32 K residual in block z-units": ("encode_block32", m_block_residual_in_block_units,
                                             ["block32_gamma", "block32_equal_norms"]),
    "block-32 QJL check without block scales": ("qjl_projection_from_codes_block32", m_block_check_without_scale,
                                                ["block32_from_codes"]),
    "block-32 V dequant with sqrt(d)": ("dequant_mse32", m_dequant_mse32_sqrt_d,
                                        ["block32_equal_norms", "block32_gamma"]),
    "block-32 K dequant without the QJL term": ("dequant_prod32", m_dequant_prod32_no_qjl,
                                                ["block32_equal_norms"]),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, fn, pins = MUTATIONS[name]
    monkeypatch.setattr(O, target, fn)
    caught = []
    for pin in pins:
        try:
            PINS[pin]()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin catches the planted mistake '{name}' (tried {pins})"
