"""Plain, slow CPU oracle for the TurboQuant / TurboQuant+ KV-cache codec.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code, tables or constants with the library: the
random tables, the codebook, the bit packing and every formula below are
written here a second time, from the method's description, in float64 NumPy
with dense matrices.

Sources (web pages; cited by title and section):
  [QPQ]  quidproquo.cc, "TurboQuant+ KV cache compression":
         "Stage 1: PolarQuant" (norm, random Walsh-Hadamard rotation,
         Lloyd-Max Gaussian codebook, per-coordinate quantisation),
         "Stage 2: QJL" (residual, residual norm, 1-bit sign projection),
         the format table (turbo2/3/4 bits per element), and
         "K/V asymmetric strategy" (K = two stages, V = Stage 1 only).
  [CXT]  chenxutan.com, "TurboQuant+ deep dive": section 1.2 (KV-cache size
         formula), 2.3 (QJL: one fixed-seed matrix shared by encoder and
         decoder, bit = projection > 0), 3.3 (sparse V: weights are not
         renormalised after the skip), and the cached-attention sketch of 1.1.
  [YYL]  yeyulingfeng.com, "TurboQuant+: 3.8x compression ...": core item 3
         (Boundary V: first 2 and last 2 layers at q8_0) and item 4 (Sparse V:
         skip V dequant where the attention weight is below 1e-6).
  [MAC]  GitHub issue #1 of the mac-code project, "technical analysis",
         section 2.1 (per-group asymmetric min-max quantisation, group 64,
         worked example 0.1/0.5/0.9 at 4 bits) and its storage-overhead note.

Readings where the pages are silent (each is listed in the design notes):
  * R = H diag(D) / sqrt(d): Sylvester Hadamard in natural order, one random
    sign diagonal applied before H.
  * Standardised rotated coordinates z = sqrt(d) R x / ||x||, quantised with
    the N(0,1) Lloyd-Max levels.
  * Nearest level, ties to the upper index; n = 0 gives z = 0.
  * K residual is taken in the rotated domain, e = z - c[idx]; its x-domain
    norm is gamma = n ||e|| / sqrt(d); the QJL sketch is sign(S e) > 0 with S
    an m x d matrix of N(0,1) draws rounded to fp16, m = d.
  * QJL inner-product estimator: sqrt(pi/2)/m * gamma * <S R q, 2 bit - 1>.
  * Norms n and gamma stored as fp16 (round to nearest even).
  * Random tables: splitmix64 (Steele, Lea, Flood 2014) in counter form,
    state_i = seed + i * 0x9E3779B97F4A7C15 for i = 1, 2, ...; the first d
    outputs give the signs (top bit set -> -1), the next m*d outputs feed the
    Box-Muller transform (Box & Muller 1958) pairwise, row-major into S.
  * q8 boundary blocks: symmetric absmax int8, blocks of 32, fp16 scale.
  * Block-32 norm storage (formats 'mse32', 'prod32'): the rotation stays
    over all d coordinates; the Stage-1 norm is kept per block of 32 rotated
    coordinates (n_b = ||(R x)_b||, fp16), each block standardised by its own
    norm, z = sqrt(32) (R x)_b / n_b.  K's residual r = R x - x_hat_1 (x
    units, rotated) keeps one fp16 norm gamma per vector; its QJL sketch is
    sign(S r).
  * min-max: fp16 scale = (max - min)/(2^b - 1) and fp16 zero = min, codes
    decided in float32 (the kernel's precision, the pages fix none).

Parity pins for this module live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special

# --------------------------------------------------------------------------
# Random tables: splitmix64 counter stream + Box-Muller
# --------------------------------------------------------------------------
_GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


def splitmix64_outputs(seed: int, count: int, first_counter: int = 1) -> np.ndarray:
    """Outputs of splitmix64 for counters first_counter .. first_counter+count-1.

    Counter form of the published generator: state_i = seed + i*gamma (mod
    2^64), output_i = mix(state_i) with the two xor-shift-multiply rounds.
    """
    i = np.arange(first_counter, first_counter + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def random_signs(seed: int, d: int) -> np.ndarray:
    """The diagonal D of the random-sign Hadamard rotation [QPQ Stage 1]."""
    w = splitmix64_outputs(seed, d, 1)
    return np.where((w >> np.uint64(63)) == 1, -1.0, 1.0)


def gaussian_projection(seed: int, m: int, d: int) -> np.ndarray:
    """The QJL matrix S (m x d), N(0,1) draws rounded to fp16 [QPQ Stage 2].

    Box-Muller on pairs of 53-bit uniforms; u1 is offset by half a step so
    it never reaches 0.  Returned as float64 holding fp16-exact values.
    """
    n = m * d
    assert n % 2 == 0
    w = splitmix64_outputs(seed, n, 1 + d)
    top53 = (w >> np.uint64(11)).astype(np.float64)
    u1 = (top53[0::2] + 0.5) * 2.0 ** -53
    u2 = top53[1::2] * 2.0 ** -53
    r = np.sqrt(-2.0 * np.log(u1))
    g = np.empty(n, dtype=np.float64)
    g[0::2] = r * np.cos(2.0 * np.pi * u2)
    g[1::2] = r * np.sin(2.0 * np.pi * u2)
    return g.astype(np.float16).astype(np.float64).reshape(m, d)


# --------------------------------------------------------------------------
# Lloyd-Max codebook for N(0,1)  [QPQ Stage 1: "Lloyd's algorithm precomputes
# the optimal Gaussian codebook"]
# --------------------------------------------------------------------------
def _phi(t):
    return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _interval_mass(lo, hi):
    """P(lo < Z < hi) for Z ~ N(0,1), using the upper tail where it is exact."""
    upper = lo >= 0.0
    return np.where(upper, special.ndtr(-lo) - special.ndtr(-hi),
                    special.ndtr(hi) - special.ndtr(lo))


def lloyd_max_gaussian(bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Levels c (ascending) and decision boundaries t of the b-bit Lloyd-Max
    quantiser for a standard normal.

    Lloyd's two conditions, alternated until the levels move less than tol:
    boundaries at midpoints, levels at the conditional mean of their cell,
    E[Z | lo<Z<hi] = (phi(lo) - phi(hi)) / (Phi(hi) - Phi(lo)).  The levels
    are kept symmetric about zero.
    """
    L = 1 << bits
    c = special.ndtri((np.arange(L) + 0.5) / L)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], t))
        hi = np.concatenate((t, [np.inf]))
        num = _phi(lo) - _phi(hi)
        c_new = num / _interval_mass(lo, hi)
        c_new = 0.5 * (c_new - c_new[::-1])
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def codebook_mse(c, t):
    """E[(Z - Q(Z))^2] for Z ~ N(0,1), by numerical quadrature per cell."""
    from scipy import integrate
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    total = 0.0
    for k in range(len(c)):
        f = lambda z, ck=c[k]: (z - ck) ** 2 * _phi(z)
        val, _ = integrate.quad(f, edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-12)
        total += val
    return total


# --------------------------------------------------------------------------
# Rotation  [QPQ Stage 1: random Walsh-Hadamard rotation, orthogonal]
# --------------------------------------------------------------------------
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix, natural order: H[i,j] = (-1)^popcount(i&j)."""
    i = np.arange(d)
    pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def rotation(signs: np.ndarray) -> np.ndarray:
    """Orthonormal R = H diag(D) / sqrt(d)."""
    d = signs.shape[0]
    return hadamard(d) * signs[None, :] / math.sqrt(d)


class Tables:
    """Everything the codec fixes once from (head_dim, seed)."""

    def __init__(self, d: int = 128, m: int | None = None, seed: int = 42):
        self.d = d
        self.m = d if m is None else m
        self.seed = seed
        self.signs = random_signs(seed, d)
        self.S = gaussian_projection(seed, self.m, d)
        self.R = rotation(self.signs)
        self.levels = {}
        self.bounds = {}
        for b in range(1, 5):
            self.levels[b], self.bounds[b] = lloyd_max_gaussian(b)


# --------------------------------------------------------------------------
# Encode  [QPQ Stage 1 + Stage 2, K/V asymmetric strategy]
# --------------------------------------------------------------------------
def quantise_index(z: np.ndarray, bounds: np.ndarray) -> np.ndarray:
    """Cell index of the Lloyd-Max partition: idx = #{k : t_k <= z}.

    Cell k is [t_{k-1}, t_k), so a value on a boundary takes the upper cell;
    away from boundaries this is the nearest level.
    """
    return np.sum(z[..., None] >= bounds, axis=-1).astype(np.int64)


def nearest_level(z: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level by exhaustive distance (used by the pins)."""
    dist = np.abs(z[..., None] - levels)
    L = levels.shape[0]
    return (L - 1 - np.argmin(dist[..., ::-1], axis=-1)).astype(np.int64)


def standardised_rotation(x: np.ndarray, tab: Tables):
    """n = ||x||, z = sqrt(d) R x / n (z = 0 for a zero vector)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where((n > 0)[..., None], x / safe[..., None], 0.0)
    z = math.sqrt(tab.d) * (u @ tab.R.T)
    return n, z


def encode(x: np.ndarray, bits: int, prod: bool, tab: Tables) -> dict:
    """Encode rows of x ([n, d]).

    MSE codec (V): idx, fp16 norm.  PROD codec (K): additionally the QJL sign
    bits of S e and the fp16 residual norm gamma.  Also returns the fp64
    intermediates (z, and for K the projection P) used to find coordinates
    that sit on a decision boundary.
    """
    n, z = standardised_rotation(x, tab)
    c = tab.levels[bits]
    idx = quantise_index(z, tab.bounds[bits])
    out = {"idx": idx, "norm": n.astype(np.float16), "n64": n, "z": z}
    if prod:
        e = z - c[idx]
        gamma = n * np.sqrt(np.sum(e * e, axis=-1)) / math.sqrt(tab.d)
        P = e @ tab.S.T
        out.update(bits_qjl=(P > 0).astype(np.uint8), rnorm=gamma.astype(np.float16),
                   gamma64=gamma, P=P, e=e)
    return out


def qjl_projection_from_codes(x: np.ndarray, idx: np.ndarray, bits: int, tab: Tables):
    """P = S (z - c[idx]) with z from x and the given codes (for checking a
    producer's sign bits against its own codes)."""
    _, z = standardised_rotation(x, tab)
    e = z - tab.levels[bits][idx]
    return e @ tab.S.T


# --------------------------------------------------------------------------
# Block-32 norm storage  [yeyulingfeng.com "TurboQuant+: 3.8x compression
# ...", technical highlights: block-32 storage; quidproquo.cc format table:
# 6.4x for turbo2, 4.6-5.1x for turbo3]
# --------------------------------------------------------------------------
BLOCK = 32


def block_standardised_rotation(x: np.ndarray, tab: Tables, block: int = BLOCK):
    """u = R x; per block of `block` rotated coordinates n_b = ||u_b|| and
    z = sqrt(block) u_b / n_b (z = 0 in a zero block).  Returns (u, n_b, z)."""
    x = np.asarray(x, dtype=np.float64)
    u = x @ tab.R.T
    ub = u.reshape(*u.shape[:-1], tab.d // block, block)
    nb = np.sqrt(np.sum(ub * ub, axis=-1))
    safe = np.where(nb > 0, nb, 1.0)
    z = np.where((nb > 0)[..., None], ub / safe[..., None], 0.0) * math.sqrt(block)
    return u, nb, z.reshape(u.shape)


def _per_coordinate(nb, block: int = BLOCK):
    """Block values [.., d/block] -> per-coordinate values [.., d]."""
    return np.repeat(np.asarray(nb, dtype=np.float64), block, axis=-1)


def encode_block32(x: np.ndarray, bits: int, prod: bool, tab: Tables, block: int = BLOCK) -> dict:
    """Block-32 encode of rows of x ([n, d]).

    'mse32': idx and the fp16 block norms.  'prod32': additionally the QJL
    sign bits of S r, r = u - (n_b / sqrt(block)) c[idx] the rotated
    Stage-1 residual (exact n_b), and its fp16 norm gamma = ||r||.  P is
    returned in z-units of the whole vector, sqrt(d) (S r) / ||x||, for the
    near-zero exemption of the parity checks (its sign is that of S r)."""
    u, nb, z = block_standardised_rotation(x, tab, block)
    c = tab.levels[bits]
    idx = quantise_index(z, tab.bounds[bits])
    out = {"idx": idx, "bnorm": nb.astype(np.float16), "bn64": nb, "z": z}
    if prod:
        r = u - _per_coordinate(nb / math.sqrt(block), block) * c[idx]
        gamma = np.sqrt(np.sum(r * r, axis=-1))
        n = np.sqrt(np.sum(u * u, axis=-1))
        zs = np.where(n > 0, math.sqrt(tab.d) / np.where(n > 0, n, 1.0), 0.0)
        P = (r @ tab.S.T) * zs[..., None]
        out.update(bits_qjl=(P > 0).astype(np.uint8), rnorm=gamma.astype(np.float16),
                   gamma64=gamma, P=P, r=r)
    return out


def qjl_projection_from_codes_block32(x: np.ndarray, idx: np.ndarray, bits: int, tab: Tables,
                                      block: int = BLOCK):
    """P (as in encode_block32) for the given codes."""
    u, nb, _ = block_standardised_rotation(x, tab, block)
    r = u - _per_coordinate(nb / math.sqrt(block), block) * tab.levels[bits][idx]
    n = np.sqrt(np.sum(u * u, axis=-1))
    zs = np.where(n > 0, math.sqrt(tab.d) / np.where(n > 0, n, 1.0), 0.0)
    return (r @ tab.S.T) * zs[..., None]


def dequant_mse32(idx, bnorm16, bits, tab: Tables, block: int = BLOCK) -> np.ndarray:
    """v_hat = R^T ( (n_b / sqrt(block)) c[idx] ) per block."""
    zhat = tab.levels[bits][idx]
    return (_per_coordinate(np.asarray(bnorm16, np.float64) / math.sqrt(block), block) * zhat) @ tab.R


def dequant_prod32(idx, bits_qjl, bnorm16, rnorm16, bits, tab: Tables, block: int = BLOCK) -> np.ndarray:
    """k_hat = R^T ( (n_b / sqrt(block)) c[idx] + sqrt(pi/2)/m * gamma * S^T (2 bit - 1) )."""
    zhat = tab.levels[bits][idx]
    g = np.asarray(rnorm16, dtype=np.float64)
    sgn = 2.0 * np.asarray(bits_qjl, dtype=np.float64) - 1.0
    rot = _per_coordinate(np.asarray(bnorm16, np.float64) / math.sqrt(block), block) * zhat + \
        (math.sqrt(math.pi / 2.0) / tab.m) * g[..., None] * (sgn @ tab.S)
    return rot @ tab.R


# --------------------------------------------------------------------------
# Dequant  [QPQ: Stage-1 reconstruction; QJL estimate of the residual]
# --------------------------------------------------------------------------
def dequant_mse(idx, norm16, bits, tab: Tables) -> np.ndarray:
    """v_hat = n R^T c[idx] / sqrt(d)."""
    zhat = tab.levels[bits][idx]
    n = np.asarray(norm16, dtype=np.float64)
    return n[..., None] * (zhat @ tab.R) / math.sqrt(tab.d)


def dequant_prod(idx, bits_qjl, norm16, rnorm16, bits, tab: Tables) -> np.ndarray:
    """k_hat = R^T ( n c[idx]/sqrt(d) + sqrt(pi/2)/m * gamma * S^T (2 bit - 1) )."""
    zhat = tab.levels[bits][idx]
    n = np.asarray(norm16, dtype=np.float64)
    g = np.asarray(rnorm16, dtype=np.float64)
    sgn = 2.0 * np.asarray(bits_qjl, dtype=np.float64) - 1.0
    rot = n[..., None] * zhat / math.sqrt(tab.d) + \
        (math.sqrt(math.pi / 2.0) / tab.m) * g[..., None] * (sgn @ tab.S)
    return rot @ tab.R


def qjl_inner_product(q, bits_qjl, gamma, tab: Tables):
    """QJL estimate of <q, r> from the sign bits of S R r and gamma = ||r||."""
    sgn = 2.0 * np.asarray(bits_qjl, dtype=np.float64) - 1.0
    sq = (np.asarray(q, dtype=np.float64) @ tab.R.T) @ tab.S.T
    return math.sqrt(math.pi / 2.0) / tab.m * np.asarray(gamma) * np.sum(sq * sgn, axis=-1)


# --------------------------------------------------------------------------
# Packed byte layout (independent of the library's packer)
# --------------------------------------------------------------------------
def pack_bitstream(codes: np.ndarray, bits: int) -> np.ndarray:
    """Rows of b-bit codes -> bytes, LSB-first: bit j of code i at stream bit
    i*b + j.  codes: [n, k] -> uint8 [n, k*b/8]."""
    codes = np.asarray(codes, dtype=np.int64)
    n, k = codes.shape
    assert (k * bits) % 8 == 0
    shifts = np.arange(bits)
    bitmat = ((codes[..., None] >> shifts) & 1).reshape(n, k * bits).astype(np.uint8)
    return np.packbits(bitmat, axis=1, bitorder="little")


def unpack_bitstream(data: np.ndarray, bits: int, k: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.uint8)
    n = data.shape[0]
    bitmat = np.unpackbits(data, axis=1, bitorder="little")[:, : k * bits]
    bitmat = bitmat.reshape(n, k, bits).astype(np.int64)
    return np.sum(bitmat << np.arange(bits), axis=-1)


def _align256(x: int) -> int:
    return (x + 255) // 256 * 256


def tq_plane_layout(kind: str, bits: int, d: int, n_vec: int, m: int | None = None) -> dict:
    """Byte offsets/sizes of the planes of one packed tensor.

    kind 'mse': [IDX n_vec*(b*d/8)] [NORM n_vec*2]
    kind 'prod': [IDX] [SIGN n_vec*m/8] [NORM n_vec*4: fp16 n then fp16 gamma]
    kind 'mse32': [IDX] [NORM n_vec*(d/32)*2: fp16 block norms]
    kind 'prod32': [IDX] [SIGN] [NORM n_vec*(d/32)*2 block norms, then
                   n_vec*2 fp16 gamma]
    kind 'q8':   [Q n_vec*d int8] [SCALE n_vec*(d/32)*2]
    Each plane starts on a 256-byte boundary.
    """
    m = d if m is None else m
    planes = {}
    off = 0
    if kind == "q8":
        planes["q"] = (off, n_vec * d)
        off = _align256(off + n_vec * d)
        planes["scale"] = (off, n_vec * (d // 32) * 2)
        off = _align256(off + n_vec * (d // 32) * 2)
        return {"planes": planes, "total": off}
    ib = n_vec * bits * d // 8
    planes["idx"] = (off, ib)
    off = _align256(off + ib)
    if kind in ("prod", "prod32"):
        planes["sign"] = (off, n_vec * m // 8)
        off = _align256(off + n_vec * m // 8)
    nb = {"mse": 2, "prod": 4, "mse32": 2 * (d // BLOCK), "prod32": 2 * (d // BLOCK) + 2}[kind]
    planes["norm"] = (off, n_vec * nb)
    off = _align256(off + n_vec * nb)
    return {"planes": planes, "total": off}


def pack_tq(enc: dict, kind: str, bits: int, d: int, m: int | None = None) -> np.ndarray:
    n_vec = enc["idx"].shape[0]
    lay = tq_plane_layout(kind, bits, d, n_vec, m)
    buf = np.zeros(lay["total"], dtype=np.uint8)
    o, s = lay["planes"]["idx"]
    buf[o:o + s] = pack_bitstream(enc["idx"], bits).reshape(-1)
    if kind in ("prod", "prod32"):
        o, s = lay["planes"]["sign"]
        buf[o:o + s] = pack_bitstream(enc["bits_qjl"], 1).reshape(-1)
    o, s = lay["planes"]["norm"]
    if kind == "prod":
        pair = np.stack([enc["norm"], enc["rnorm"]], axis=1).astype(np.float16)
        buf[o:o + s] = pair.view(np.uint8).reshape(-1)
    elif kind == "mse":
        buf[o:o + s] = enc["norm"].astype(np.float16).view(np.uint8).reshape(-1)
    else:
        blk = np.ascontiguousarray(enc["bnorm"], dtype=np.float16).view(np.uint8).reshape(-1)
        buf[o:o + blk.size] = blk
        if kind == "prod32":
            buf[o + blk.size:o + s] = np.ascontiguousarray(enc["rnorm"], dtype=np.float16).view(np.uint8).reshape(-1)
    return buf


def unpack_tq(buf: np.ndarray, kind: str, bits: int, d: int, n_vec: int, m: int | None = None) -> dict:
    m = d if m is None else m
    lay = tq_plane_layout(kind, bits, d, n_vec, m)
    buf = np.asarray(buf, dtype=np.uint8)
    o, s = lay["planes"]["idx"]
    out = {"idx": unpack_bitstream(buf[o:o + s].reshape(n_vec, bits * d // 8), bits, d)}
    if kind in ("prod", "prod32"):
        o, s = lay["planes"]["sign"]
        out["bits_qjl"] = unpack_bitstream(buf[o:o + s].reshape(n_vec, m // 8), 1, m)
    o, s = lay["planes"]["norm"]
    if kind == "prod":
        pair = buf[o:o + s].copy().view(np.float16).reshape(n_vec, 2)
        out["norm"], out["rnorm"] = pair[:, 0].copy(), pair[:, 1].copy()
    elif kind == "mse":
        out["norm"] = buf[o:o + s].copy().view(np.float16)
    else:
        nbk = d // BLOCK
        out["bnorm"] = buf[o:o + n_vec * nbk * 2].copy().view(np.float16).reshape(n_vec, nbk)
        if kind == "prod32":
            out["rnorm"] = buf[o + n_vec * nbk * 2:o + s].copy().view(np.float16)
    return out


def dequant_packed(buf, kind: str, bits: int, tab: Tables, n_vec: int) -> np.ndarray:
    """Dense fp64 reconstruction of every vector held in a packed buffer."""
    if kind == "q8":
        qd = unpack_q8(buf, tab.d, n_vec)
        return q8_dequant(qd["q"], qd["scale"])
    u = unpack_tq(buf, kind, bits, tab.d, n_vec, tab.m)
    if kind == "prod":
        return dequant_prod(u["idx"], u["bits_qjl"], u["norm"], u["rnorm"], bits, tab)
    if kind == "prod32":
        return dequant_prod32(u["idx"], u["bits_qjl"], u["bnorm"], u["rnorm"], bits, tab)
    if kind == "mse32":
        return dequant_mse32(u["idx"], u["bnorm"], bits, tab)
    return dequant_mse(u["idx"], u["norm"], bits, tab)


# --------------------------------------------------------------------------
# q8 boundary-layer blocks  [YYL core item 3: boundary layers kept at q8_0]
# --------------------------------------------------------------------------
def q8_quant(x: np.ndarray, block: int = 32):
    """Symmetric absmax int8 per block of 32: fp16 scale = max|x|/127,
    q = clamp(rint(x/scale), -127, 127); an all-zero block has scale 0, q 0."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    xb = x.reshape(n, d // block, block)
    amax = np.max(np.abs(xb), axis=-1)
    scale = (amax / 127.0).astype(np.float16)
    s64 = scale.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    q = np.where(s64[..., None] > 0, np.rint(xb / safe[..., None]), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(n, d)
    return q, scale


def q8_dequant(q, scale, block: int = 32):
    q = np.asarray(q, dtype=np.float64)
    n, d = q.shape
    s = np.asarray(scale, dtype=np.float64).reshape(n, d // block)
    return (q.reshape(n, d // block, block) * s[..., None]).reshape(n, d)


def pack_q8(q, scale, d: int) -> np.ndarray:
    n_vec = q.shape[0]
    lay = tq_plane_layout("q8", 8, d, n_vec)
    buf = np.zeros(lay["total"], dtype=np.uint8)
    o, s = lay["planes"]["q"]
    buf[o:o + s] = np.asarray(q, dtype=np.int8).view(np.uint8).reshape(-1)
    o, s = lay["planes"]["scale"]
    buf[o:o + s] = np.asarray(scale, dtype=np.float16).view(np.uint8).reshape(-1)
    return buf


def unpack_q8(buf, d: int, n_vec: int) -> dict:
    lay = tq_plane_layout("q8", 8, d, n_vec)
    buf = np.asarray(buf, dtype=np.uint8)
    o, s = lay["planes"]["q"]
    q = buf[o:o + s].copy().view(np.int8).reshape(n_vec, d)
    o, s = lay["planes"]["scale"]
    sc = buf[o:o + s].copy().view(np.float16).reshape(n_vec, d // 32)
    return {"q": q, "scale": sc}


# --------------------------------------------------------------------------
# Decode attention  [CXT 1.1 cached attention; YYL item 4 / CXT 3.3 sparse V]
# --------------------------------------------------------------------------
def attention_decode(q, k_hat, v_hat, tau: float = 1e-6, seq_lens=None):
    """One query token per (batch, q-head) against dense dequantised K/V.

    q: [B, Hq, d]; k_hat, v_hat: [B, Hkv, T, d].  Scores <q, k>/sqrt(d), full
    softmax over the first seq_len tokens, then V rows whose normalised weight
    is below tau are dropped without renormalising.  q head h reads kv head
    floor(h / (Hq/Hkv)).  seq_lens[b] is clamped to [0, T].  Returns
    (out [B, Hq, d] float64, p [B, Hq, T]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, T = k_hat.shape[1], k_hat.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d))
    probs = np.zeros((B, Hq, T))
    for b in range(B):
        # a length outside [0, T] means the nearest end of that range
        L = T if seq_lens is None else min(max(int(seq_lens[b]), 0), T)
        for h in range(Hq):
            kv = h // g
            if L == 0:
                continue
            s = k_hat[b, kv, :L] @ q[b, h] / math.sqrt(d)
            p = special.softmax(s)
            keep = p >= tau
            out[b, h] = (p * keep) @ v_hat[b, kv, :L]
            probs[b, h, :L] = p
    return out, probs


def attention_prefill(q, k_hat, v_hat, tau: float = 1e-6, seq_lens=None):
    """Causal attention of the last Tq positions of each sequence over dense
    dequantised K/V (the prompt-processing counterpart of the decode step of
    [CXT] 1.1, whose prefill speed the pages report).

    q: [B, Tq, Hq, d]; k_hat, v_hat: [B, Hkv, T, d].  With L_b = seq_lens[b]
    (or T), query i of sequence b sits at position L_b - Tq + i and sees the
    first L_b - Tq + i + 1 tokens (none when that is <= 0); for each query the
    computation is the decode step above with that length: scores
    <q, k>/sqrt(d), full softmax, V rows below tau dropped, no
    renormalisation.  Returns out [B, Tq, Hq, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Tq, Hq, d = q.shape
    T = k_hat.shape[2]
    out = np.zeros((B, Tq, Hq, d))
    for b in range(B):
        L = T if seq_lens is None else min(max(int(seq_lens[b]), 0), T)
        for i in range(Tq):
            n = max(L - Tq + i + 1, 0)
            o, _ = attention_decode(q[b:b + 1, i], k_hat[b:b + 1], v_hat[b:b + 1], tau, [n])
            out[b, i] = o[0]
    return out


# --------------------------------------------------------------------------
# Per-group asymmetric min-max baseline  [MAC section 2.1]
# --------------------------------------------------------------------------
def minmax_quant(x: np.ndarray, group: int = 64, bits: int = 3):
    """Per group of `group` consecutive elements: fp16 scale =
    (max-min)/(2^b-1), fp16 zero = min, code = clamp(round((x-zero)/scale)).

    Scale comes from the exact fp16 extremes in float64 and is rounded to
    fp16 once.  The code (an integer decided by floating point) is taken in
    float32 from the stored fp16 scale and zero, round half to even; a group
    with max == min gets scale 0 and codes 0.
    """
    x16 = np.asarray(x, dtype=np.float16).reshape(-1)
    assert x16.size % group == 0
    xg = x16.reshape(-1, group)
    mn = xg.min(axis=1).astype(np.float64)
    mx = xg.max(axis=1).astype(np.float64)
    qmax = (1 << bits) - 1
    scale = ((mx - mn) / qmax).astype(np.float16)
    zero = mn.astype(np.float16)
    s32 = scale.astype(np.float32)
    diff = xg.astype(np.float32) - zero.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = diff / np.where(s32 > 0, s32, np.float32(1.0))[:, None]
    code = np.clip(np.rint(ratio), 0, qmax)
    code = np.where((s32 > 0)[:, None], code, 0).astype(np.int64)
    return code.reshape(-1), scale, zero


def minmax_dequant(code, scale, zero, group: int = 64):
    c = np.asarray(code, dtype=np.float64).reshape(-1, group)
    return (c * np.asarray(scale, np.float64)[:, None] +
            np.asarray(zero, np.float64)[:, None]).reshape(-1)


def pack_minmax_codes(code: np.ndarray, bits: int) -> np.ndarray:
    """One LSB-first bitstream over the flattened tensor."""
    code = np.asarray(code, dtype=np.int64).reshape(1, -1)
    return pack_bitstream(code, bits).reshape(-1)


def unpack_minmax_codes(data: np.ndarray, bits: int, n: int) -> np.ndarray:
    return unpack_bitstream(np.asarray(data, np.uint8).reshape(1, -1), bits, n).reshape(-1)


def quality(x, xhat, d: int = 128):
    """MSE, cosine of the flattened tensors, and mean per-vector cosine
    [MAC section 2.2 quality measure]."""
    x = np.asarray(x, np.float64).reshape(-1)
    xhat = np.asarray(xhat, np.float64).reshape(-1)
    mse = float(np.mean((x - xhat) ** 2))
    cos = float(x @ xhat / (np.linalg.norm(x) * np.linalg.norm(xhat) + 1e-300))
    xv, hv = x.reshape(-1, d), xhat.reshape(-1, d)
    num = np.sum(xv * hv, axis=1)
    den = np.linalg.norm(xv, axis=1) * np.linalg.norm(hv, axis=1)
    per = np.where(den > 0, num / np.where(den > 0, den, 1.0), 1.0)
    return {"mse": mse, "cos_flat": cos, "cos_vec_mean": float(per.mean())}


# --------------------------------------------------------------------------
# Format arithmetic  [QPQ format table; CXT 1.2 size formula]
# --------------------------------------------------------------------------
def kv_cache_bytes_fp16(layers, kv_heads, head_dim, tokens, batch=1):
    """2 (K and V) x batch x tokens x layers x kv_heads x head_dim x 2 bytes."""
    return 2 * batch * tokens * layers * kv_heads * head_dim * 2


def bytes_per_vector(kind: str, bits: int, d: int = 128, m: int | None = None) -> int:
    m = d if m is None else m
    if kind == "q8":
        return d + (d // 32) * 2
    if kind in ("mse32", "prod32"):
        base = bits * d // 8 + 2 * (d // BLOCK)
        if kind == "prod32":
            base += m // 8 + 2
        return base
    base = bits * d // 8 + 2
    if kind == "prod":
        base += m // 8 + 2
    return base
