"""Plain, slow, float64 CPU oracle for rotation-preconditioned KV-cache compression.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library (``kv_cache_vector_encode_amd``); the only
common dependency is the seeded input generator module, which holds none of
the method's arithmetic.

Every function states what it computes and which passage of the source pages
it follows.  Page shorthands (titles as printed on the pages):

  [P1] "TurboQuant: KV Cache Vector Quantization" (llm-engineer.pages.dev card)
  [P2] "TurboQuant: KV Cache Compression" (Bit-Axon documentation page)
  [P3] "OCTOPUS: Optimized KV Cache for Transformers via Octahedral
       Parametrization Under optimal Squared error quantization" (aitrends.kr
       summary)
  [P4] TurboQuant deep-dive blog post (cell-devlog.tistory.com), sections
       "Step 1: Randomized Hadamard Transform", "Step 2: PolarQuant",
       "Step 3: QJL", "실전 2" (KIVI vs TurboQuant)

Readings taken where the pages are silent or disagree (each one is listed,
with its reason, in the design notes of the repository):
  * sign generator: SplitMix64 (counter based) replaces torch's seeded RNG;
  * R = H diag(s) / sqrt(d), H in Sylvester (natural) order;
  * codebook: Lloyd-Max for the exact coordinate marginal of a uniformly
    random unit vector in R^d, rounded to fp32; thresholds are the fp32
    midpoints of adjacent fp32 centroids;
  * nearest codeword with ties to the lower (more negative) index;
  * fp16 round-to-nearest-even norm, saturating at 65504;
  * QJL residual taken in the rotated unit-direction frame with estimator
    constant sqrt(pi/2)/sqrt(d) and an independent sign-Hadamard R';
  * logit scale 1/sqrt(d); query head h reads KV head h // (Hq / Hkv);
  * triplet codec: the last of ceil(d/3) triplets padded with zeros; the
    octahedral map is the equal-area one (the glossary calls it equal-area),
    so C_xi is the uniform quantiser; rho takes Lloyd-Max for its exact
    marginal; B_tri = 2 b_dir + b_nrm with (b_dir, b_nrm) = (b+1, b-1); the
    3x3 joint rounding scans the nearest cell and its neighbours in xi and
    eta and, per candidate direction, the norm code nearest the projection;
    a zero triplet takes the direction (0, 0, 1).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, textbook limits or brute force.
"""

from __future__ import annotations

import math

import numpy as np
from scipy import special

__all__ = [
    "splitmix64", "rotation_signs", "hadamard", "rotation_matrix",
    "coord_density", "coord_cdf", "coord_partial_mean",
    "coord_partial_second_moment", "lloyd_max",
    "codebook_fp32", "codebook_distortion", "fp16_norm", "encode",
    "reconstruct", "qjl_encode", "qjl_dot_estimate", "logits",
    "attention", "bits_per_vector", "LayoutV1", "pack_codes",
    "unpack_codes", "pack_signs", "unpack_signs", "write_cache",
    "read_cache", "unpack_pool", "SQRT_HALF_PI", "fp16_sat",
    "minmax_encode", "minmax_decode", "octo_bits", "octo_triplets",
    "oct_map", "oct_unmap", "octo_dir_codebook", "rho_cdf",
    "rho_partial_mean", "rho_lloyd_max", "octo_codebooks", "octo_encode",
    "octo_encode_triplets", "octo_triplet_error", "octo_decode",
    "octo_record_bytes", "octo_pack", "octo_unpack", "octo_qjl_encode",
]

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


# ---------------------------------------------------------------------------
# E0: seeded random signs  ([P4] Step 1: a diagonal of random signs drawn
# from a seed; [P3] Method step 2: the Walsh-Hadamard rotation after a sign
# flip; a fixed seed for reproducibility in the [P4] TurboQuantConfig
# example).
# ---------------------------------------------------------------------------

def splitmix64(seed: int, n: int) -> list[int]:
    """First ``n`` outputs of SplitMix64 seeded with ``seed``.

    Published generator (Steele, Lea & Flood 2014; Vigna's ``splitmix64.c``):
    state += 0x9E3779B97F4A7C15; z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
    output z ^ (z >> 31)   (all arithmetic modulo 2^64).
    """
    out = []
    state = seed & _MASK64
    for _ in range(n):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def rotation_signs(seed: int, d: int) -> np.ndarray:
    """s_j = +1 if the top bit of the j-th SplitMix64 output is 0, else -1."""
    return np.array([1 if (z >> 63) == 0 else -1 for z in splitmix64(seed, d)],
                    dtype=np.int8)


def hadamard(d: int) -> np.ndarray:
    """Dense Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j).

    This is the matrix that the in-place butterfly loop of [P4] Step 1
    (fast_hadamard_transform, strides h = 1, 2, 4, ...) applies; d must be a
    power of two ([P4] Step 1 asserts it).
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    a = i[:, None] & i[None, :]
    parity = np.zeros_like(a)
    while np.any(a):
        parity ^= a & 1
        a >>= 1
    return np.where(parity == 0, 1.0, -1.0)


def rotation_matrix(seed: int, d: int) -> np.ndarray:
    """R = H diag(s) / sqrt(d): sign flip first, then Hadamard, then 1/sqrt(d).

    [P4] Step 1 applies x*signs, then the Hadamard transform, then divides by
    sqrt(d); [P3] Method step 2 writes R = H diag(s).  The 1/sqrt(d) makes R
    orthogonal, which [P1] (the rotation keeps vector lengths) and [P4] Step 1
    (the transform is orthogonal, so inner products survive it) require.
    """
    s = rotation_signs(seed, d).astype(np.float64)
    return hadamard(d) * s[None, :] / math.sqrt(d)


# ---------------------------------------------------------------------------
# E0: Lloyd-Max codebook for the coordinate marginal of a uniform unit vector
# ([P3] glossary entry for Lloyd-Max quantization: alternate centroid updates that
# minimise MSE for a given 1-D density, used per coordinate; [P3] key idea:
# rotation codecs approximate the marginals with per-coordinate Lloyd-Max).
# ---------------------------------------------------------------------------

def _log_kd(d: int) -> float:
    # normalising constant K_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2))
    return special.gammaln(d / 2.0) - special.gammaln((d - 1) / 2.0) - 0.5 * math.log(math.pi)


def coord_density(x, d: int):
    """f_d(x) = K_d (1 - x^2)^((d-3)/2) on [-1, 1]: density of one coordinate
    of a uniformly random unit vector in R^d."""
    x = np.asarray(x, dtype=np.float64)
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    out[inside] = np.exp(_log_kd(d) + (d - 3) / 2.0 * np.log1p(-x[inside] ** 2))
    return out


def coord_cdf(x, d: int):
    """F(x) = 1/2 + sgn(x)/2 * I_{x^2}(1/2, (d-1)/2)  (x^2 ~ Beta(1/2, (d-1)/2))."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(x) * special.betainc(0.5, (d - 1) / 2.0, x * x)


def coord_partial_mean(a, b, d: int):
    """Integral of x f_d(x) over [a, b]:
    K_d/(d-1) * [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)]."""
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    kd = math.exp(_log_kd(d))
    e = (d - 1) / 2.0
    return kd / (d - 1) * ((1.0 - a * a) ** e - (1.0 - b * b) ** e)


def lloyd_max(d: int, bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Float64 Lloyd-Max quantiser with 2^bits levels for f_d.

    Alternates the two optimality conditions until the centroids move by less
    than ``tol`` times the largest centroid magnitude: thresholds at midpoints of adjacent centroids, centroids at
    the conditional means of their cells.  Starts from the quantiles at
    (i + 1/2) / 2^bits.  The density is even, so the centroids are
    symmetrised exactly (c_{n-1-i} = -c_i) after every step.
    Returns (centroids, thresholds) sorted ascending, float64.
    """
    n = 1 << bits
    if n < 2:
        raise ValueError("bits must be >= 1")
    q = (np.arange(n) + 0.5) / n
    # inverse CDF through the inverse regularised incomplete beta function
    z = special.betaincinv(0.5, (d - 1) / 2.0, np.abs(2.0 * q - 1.0))
    c = np.sign(q - 0.5) * np.sqrt(z)
    c = 0.5 * (c - c[::-1])
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-1.0], t))
        hi = np.concatenate((t, [1.0]))
        mass = coord_cdf(hi, d) - coord_cdf(lo, d)
        new = coord_partial_mean(lo, hi, d) / mass
        new = 0.5 * (new - new[::-1])
        moved = np.max(np.abs(new - c))
        c = new
        if moved < tol * np.max(np.abs(c)):
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    return c, 0.5 * (c[:-1] + c[1:])


def codebook_fp32(d: int, bits: int):
    """The codebook as stored: c32 = fp32(c) (round to nearest), and
    t32_i = fp32((c32_i + c32_{i+1}) / 2) (the midpoint is exact in float64).
    Returned as float64 arrays holding fp32 values."""
    c, _ = lloyd_max(d, bits)
    c32 = c.astype(np.float32).astype(np.float64)
    t32 = (0.5 * (c32[:-1] + c32[1:])).astype(np.float32).astype(np.float64)
    return c32, t32


def coord_partial_second_moment(a, b, d: int):
    """Integral of x^2 f_d(x) over [a, b], by parts:
    [-x K_d (1-x^2)^((d-1)/2) / (d-1)]_a^b + (F_{d+2}(b) - F_{d+2}(a)) / d,
    using K_d / ((d-1) K_{d+2}) = 1/d.  Over [-1, 1] it gives E[X^2] = 1/d."""
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    kd = math.exp(_log_kd(d))
    e = (d - 1) / 2.0
    boundary = (-b * (1.0 - b * b) ** e + a * (1.0 - a * a) ** e) * kd / (d - 1)
    return boundary + (coord_cdf(b, d + 2) - coord_cdf(a, d + 2)) / d


def codebook_distortion(d: int, bits: int, c=None) -> float:
    """Per-coordinate MSE E[(X - Q(X))^2] of codebook ``c`` (default: the
    float64 Lloyd-Max one) under f_d with nearest-codeword cells:
    sum over cells of (E[X^2; cell] - 2 c E[X; cell] + c^2 P(cell))."""
    if c is None:
        c, _ = lloyd_max(d, bits)
    c = np.asarray(c, dtype=np.float64)
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    mass = coord_cdf(hi, d) - coord_cdf(lo, d)
    m1 = coord_partial_mean(lo, hi, d)
    m2 = coord_partial_second_moment(lo, hi, d)
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))


# ---------------------------------------------------------------------------
# E1-E5: encode  ([P1] three stages Split / Rotate / Codebook; [P3] Method
# steps 1-2 and 6; [P2] quantisation function Q(K) = argmin ||K - K'||;
# [P4] Step 2 stores the magnitude as fp16 and the direction as indices).
# ---------------------------------------------------------------------------

def fp16_norm(gamma) -> np.ndarray:
    """fp16 round-to-nearest-even of the norm, saturating at 65504 ([P4]
    Step 2 keeps the magnitude as an fp16 value; saturation is this build's
    reading)."""
    g = np.minimum(np.asarray(gamma, dtype=np.float64), 65504.0)
    return g.astype(np.float16)


def encode(x, seed: int, c32):
    """Encode vectors ``x`` (..., d) with rotation seed ``seed`` and codebook
    ``c32`` (ascending, float64 holding fp32 values).

    gamma = ||x||_2; u = x / gamma (u = 0 when gamma = 0); y = R u;
    idx_j = argmin_i (y_j - c_i)^2, first index on ties (numpy argmin).
    Returns dict(idx=int64 (..., d), gamma=float64, gamma16=float16, y=float64).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    gamma = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(gamma > 0, gamma, 1.0)
    u = np.where((gamma > 0)[..., None], x / safe[..., None], 0.0)
    R = rotation_matrix(seed, d)
    y = u @ R.T
    c = np.asarray(c32, dtype=np.float64)
    dist = (y[..., None] - c) ** 2
    idx = np.argmin(dist, axis=-1)
    return {"idx": idx, "gamma": gamma, "gamma16": fp16_norm(gamma), "y": y}


def reconstruct(idx, gamma16, seed: int, c32):
    """x_hat = float64(gamma16) * R^T c32[idx]  ([P2] dequantisation
    K_hat = DQ(K_q); [P4] Step 2 decompress_key = magnitude * direction,
    with the rotation undone by R^T because R is orthogonal)."""
    idx = np.asarray(idx)
    d = idx.shape[-1]
    R = rotation_matrix(seed, d)
    yhat = np.asarray(c32, dtype=np.float64)[idx]
    return np.asarray(gamma16, dtype=np.float64)[..., None] * (yhat @ R)


# ---------------------------------------------------------------------------
# Comparison codec: the per-vector affine (min/max) uniform quantiser after
# the same rotation ([P4] Step 3's value path): 2^b equally spaced levels
# spanning [min_j y_j, max_j y_j] of the rotated vector, each coordinate
# sent to its nearest level; step and lowest level kept as fp16; decoded by
# the inverse rotation.
# ---------------------------------------------------------------------------

def fp16_sat(v) -> np.ndarray:
    """fp16 round-to-nearest-even, saturating at +-65504 (this build's reading:
    a plain fp16 conversion, as the page's listing does, would give
    infinities past the fp16 range)."""
    return np.clip(np.asarray(v, dtype=np.float64), -65504.0, 65504.0).astype(np.float16)


def minmax_encode(x, seed: int, bits: int):
    """Min/max codes of vectors ``x`` (..., d): y = R x (no norm split);
    the levels are lo + k * scale, k = 0 .. 2^bits - 1, with lo = min_j y_j
    and scale = (max_j y_j - lo) / (2^bits - 1); q_j is the nearest level's
    k (ties to the even k).  A vector whose rotated coordinates are
    all equal (scale = 0, e.g. zero) takes every code 0 (the page divides by
    zero there; this build's reading).  scale16 = fp16(scale), zero16 =
    fp16(lo).  Returns dict(codes, scale, zero, scale16, zero16, u, y)."""
    x = np.asarray(x, dtype=np.float64)
    R = rotation_matrix(seed, x.shape[-1])
    y = x @ R.T
    lo, hi = y.min(axis=-1), y.max(axis=-1)
    scale = (hi - lo) / ((1 << bits) - 1)
    safe = np.where(scale > 0, scale, 1.0)
    u = np.where((scale > 0)[..., None], (y - lo[..., None]) / safe[..., None], 0.0)
    q = np.clip(np.rint(u), 0, (1 << bits) - 1).astype(np.int64)
    return {"codes": q, "scale": scale, "zero": lo, "scale16": fp16_sat(scale), "zero16": fp16_sat(lo),
            "u": u, "y": y}


def minmax_decode(codes, scale16, zero16, seed: int):
    """x_hat = R^T (codes * scale16 + zero16), in float64 from the stored
    fp16 scale and zero point (each code's level, rotated back; the inverse
    is R^T, not a second forward rotation)."""
    codes = np.asarray(codes, dtype=np.float64)
    R = rotation_matrix(seed, codes.shape[-1])
    yhat = codes * np.asarray(scale16, dtype=np.float64)[..., None] + np.asarray(zero16, dtype=np.float64)[..., None]
    return yhat @ R


# ---------------------------------------------------------------------------
# E6: optional 1-bit QJL residual sketch  ([P3] Contributions, the optional
# one-bit QJL residual that makes the inner-product estimate unbiased: sketch
# the signs of the rotated-frame residual through an independent R', store
# them, add a correction to q^T k).
# ---------------------------------------------------------------------------

def qjl_encode(y, idx, c32, seed_qjl: int):
    """r = y - c32[idx]; rho16 = fp16(||r||); z = R' r; bit_j = [z_j < 0].
    Returns dict(bits=uint8 (..., d) of 0/1, rho=float64, rho16=float16, z)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    r = y - np.asarray(c32, dtype=np.float64)[np.asarray(idx)]
    rho = np.sqrt(np.sum(r * r, axis=-1))
    Rq = rotation_matrix(seed_qjl, d)
    z = r @ Rq.T
    return {"bits": (z < 0).astype(np.uint8), "rho": rho,
            "rho16": fp16_norm(rho), "z": z}


def qjl_dot_estimate(bits, rho16, w_rot, seed_qjl: int):
    """Estimate <w_rot, r> from the sketch: sqrt(pi/2)/sqrt(d) * rho16 *
    sum_j sgn_j (R' w_rot)_j with sgn_j = +1 (bit 0) or -1 (bit 1).

    For a Gaussian sketch row g, E[sign(g.r) (g.w)] = sqrt(2/pi) <r,w>/||r||;
    the rows of R' are unit vectors (g/sqrt(d) in distribution), which gives
    the constant above.
    """
    bits = np.asarray(bits)
    d = bits.shape[-1]
    sgn = 1.0 - 2.0 * bits.astype(np.float64)
    Rq = rotation_matrix(seed_qjl, d)
    wq = np.asarray(w_rot, dtype=np.float64) @ Rq.T
    return SQRT_HALF_PI / math.sqrt(d) * np.asarray(rho16, np.float64) * np.sum(sgn * wq, axis=-1)


# ---------------------------------------------------------------------------
# D0-D6: decode  ([P2] attention under quantisation:
# Attn(Q, K_hat, V_hat) = softmax(Q K_hat^T / sqrt(d_h)) V_hat).
# The oracle works in the ORIGINAL frame (reconstructs K_hat, V_hat); it never
# uses the rotated-frame shortcut, so that shortcut is tested, not assumed.
# ---------------------------------------------------------------------------

def logits(q, khat, scale=None, qjl=None):
    """score_t = scale * <q, khat_t>, scale = 1/sqrt(d) by default.

    ``qjl`` (optional) = dict(bits, rho16, gamma16, seed, seed_qjl): adds
    scale * gamma16_t * estimate(<R q, r_t>) for every key t.
    q: (d,), khat: (T, d).  Returns (T,) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    s = tau * (np.asarray(khat, np.float64) @ q)
    if qjl is not None:
        qrot = rotation_matrix(qjl["seed"], d) @ q
        est = qjl_dot_estimate(qjl["bits"], qjl["rho16"], qrot[None, :], qjl["seed_qjl"])
        s = s + tau * np.asarray(qjl["gamma16"], np.float64) * est
    return s


def attention(q, khat, vhat, scale=None):
    """Exact softmax attention of one query over T reconstructed keys/values:
    p = softmax(scores) (max subtracted), o = sum_t p_t vhat_t.
    Returns (o, scores)."""
    s = logits(q, khat, scale)
    p = np.exp(s - np.max(s))
    p /= np.sum(p)
    return p @ np.asarray(vhat, np.float64), s


def bits_per_vector(d: int, bits: int, qjl: bool = False) -> int:
    """d*b index bits + 16 norm bits ([P4] Step 2 bit budget: 128*4+16 = 528,
    128*3+16 = 400); the QJL sidecar adds d sign bits + a 16-bit residual norm."""
    return d * bits + 16 + ((d + 16) if qjl else 0)


# ---------------------------------------------------------------------------
# Paged cache layout, version 1 (the pages fix none of it: [P4] stores int8
# indices unpacked, its bit budget implies packing; [P2] cites PagedAttention
# for cache management).  Spec:
#   pool = [num_blocks][num_kv_heads][block_bytes], 16 tokens per block;
#   block = K codes [16][d*bk/8] | V codes [16][d*bv/8] (if bv > 0)
#           | gammaK [16] fp16 | gammaV [16] fp16 (if bv > 0)
#           | (QJL) rho [16] fp16 | sign bits [16][d/8];
#   a token's code record: code j at bits [j*b, j*b + b) of the record read
#   as a little-endian bit string; codes are ascending ranks (0 = most
#   negative centroid); QJL sign bit j at bit j (1 = negative).
# ---------------------------------------------------------------------------

class LayoutV1:
    BLOCK = 16

    def __init__(self, d: int, num_kv_heads: int, bits_k: int, bits_v: int,
                 qjl: bool, num_blocks: int):
        self.d, self.hkv, self.bk, self.bv = d, num_kv_heads, bits_k, bits_v
        self.qjl, self.num_blocks = bool(qjl), num_blocks
        B = self.BLOCK
        self.k_rec = d * bits_k // 8
        self.v_rec = d * bits_v // 8
        self.off_k = 0
        self.off_v = B * self.k_rec
        self.off_gk = self.off_v + B * self.v_rec
        self.off_gv = self.off_gk + 2 * B
        self.off_rho = self.off_gv + (2 * B if bits_v > 0 else 0)
        self.off_sig = self.off_rho + 2 * B
        self.block_bytes = self.off_rho + ((2 * B + B * d // 8) if qjl else 0)
        self.pool_bytes = num_blocks * num_kv_heads * self.block_bytes

    def base(self, block: int, head: int) -> int:
        return (block * self.hkv + head) * self.block_bytes


def pack_codes(codes, bits: int) -> bytes:
    """One record: code j occupies bits [j*bits, (j+1)*bits), LSB first."""
    v = 0
    for j, cj in enumerate(np.asarray(codes, dtype=np.int64).tolist()):
        if not 0 <= cj < (1 << bits):
            raise ValueError("code out of range")
        v |= cj << (j * bits)
    return v.to_bytes(len(codes) * bits // 8, "little")


def unpack_codes(rec: bytes, bits: int, d: int) -> np.ndarray:
    v = int.from_bytes(bytes(rec), "little")
    m = (1 << bits) - 1
    return np.array([(v >> (j * bits)) & m for j in range(d)], dtype=np.int64)


def pack_signs(bits01) -> bytes:
    return pack_codes(bits01, 1)


def unpack_signs(rec: bytes, d: int) -> np.ndarray:
    return unpack_codes(rec, 1, d)


def write_cache(pool: bytearray, lay: LayoutV1, slot: int, head: int,
                k_idx, k_g16, v_idx=None, v_g16=None, qjl_bits=None, rho16=None):
    """Store one token-head of encoded data at ``slot`` (block = slot // 16,
    row = slot % 16) following layout version 1."""
    blk, row = divmod(slot, lay.BLOCK)
    b = lay.base(blk, head)
    o = b + lay.off_k + row * lay.k_rec
    pool[o:o + lay.k_rec] = pack_codes(k_idx, lay.bk)
    o = b + lay.off_gk + 2 * row
    pool[o:o + 2] = np.float16(k_g16).tobytes()
    if lay.bv > 0:
        o = b + lay.off_v + row * lay.v_rec
        pool[o:o + lay.v_rec] = pack_codes(v_idx, lay.bv)
        o = b + lay.off_gv + 2 * row
        pool[o:o + 2] = np.float16(v_g16).tobytes()
    if lay.qjl:
        o = b + lay.off_rho + 2 * row
        pool[o:o + 2] = np.float16(rho16).tobytes()
        o = b + lay.off_sig + row * (lay.d // 8)
        pool[o:o + lay.d // 8] = pack_signs(qjl_bits)


def read_cache(pool, lay: LayoutV1, slot: int, head: int) -> dict:
    """Inverse of ``write_cache`` for one token-head (spec unpacker)."""
    pool = bytes(pool) if not isinstance(pool, (bytes, bytearray)) else pool
    blk, row = divmod(slot, lay.BLOCK)
    b = lay.base(blk, head)
    o = b + lay.off_k + row * lay.k_rec
    out = {"k_idx": unpack_codes(pool[o:o + lay.k_rec], lay.bk, lay.d)}
    o = b + lay.off_gk + 2 * row
    out["k_g16"] = np.frombuffer(pool[o:o + 2], dtype=np.float16)[0]
    if lay.bv > 0:
        o = b + lay.off_v + row * lay.v_rec
        out["v_idx"] = unpack_codes(pool[o:o + lay.v_rec], lay.bv, lay.d)
        o = b + lay.off_gv + 2 * row
        out["v_g16"] = np.frombuffer(pool[o:o + 2], dtype=np.float16)[0]
    if lay.qjl:
        o = b + lay.off_rho + 2 * row
        out["rho16"] = np.frombuffer(pool[o:o + 2], dtype=np.float16)[0]
        o = b + lay.off_sig + row * (lay.d // 8)
        out["qjl_bits"] = unpack_signs(pool[o:o + lay.d // 8], lay.d)
    return out


def unpack_pool(pool, lay: LayoutV1, blocks=None) -> dict:
    """Vectorised form of ``read_cache`` for whole blocks (same spec): returns
    arrays indexed [block, head, row, ...] for the selected physical blocks.
    Pinned against the per-token unpacker in the oracle tests."""
    buf = np.frombuffer(bytes(pool) if not isinstance(pool, np.ndarray) else pool.tobytes(), dtype=np.uint8)
    arr = buf.reshape(lay.num_blocks, lay.hkv, lay.block_bytes)
    if blocks is not None:
        arr = arr[np.asarray(blocks)]
    B, d = lay.BLOCK, lay.d

    def codes(off, rec, bits):
        raw = arr[:, :, off:off + B * rec].reshape(arr.shape[0], lay.hkv, B, rec)
        bitv = np.unpackbits(raw, axis=-1, bitorder="little").reshape(arr.shape[0], lay.hkv, B, d, bits)
        return np.sum(bitv.astype(np.int64) << np.arange(bits), axis=-1)

    def halves(off):
        return arr[:, :, off:off + 2 * B].copy().view(np.float16).reshape(arr.shape[0], lay.hkv, B)

    out = {"k_idx": codes(lay.off_k, lay.k_rec, lay.bk), "k_g16": halves(lay.off_gk)}
    if lay.bv > 0:
        out["v_idx"] = codes(lay.off_v, lay.v_rec, lay.bv)
        out["v_g16"] = halves(lay.off_gv)
    if lay.qjl:
        out["rho16"] = halves(lay.off_rho)
        raw = arr[:, :, lay.off_sig:lay.off_sig + B * d // 8].reshape(arr.shape[0], lay.hkv, B, d // 8)
        out["qjl_bits"] = np.unpackbits(raw, axis=-1, bitorder="little").astype(np.int64)
    return out


# ---------------------------------------------------------------------------
# Triplet codec ([P3] Contributions, the triplet direction quantizer with
# norm marginals, and the Method list, steps 1-7): the rotated unit direction is
# cut into ceil(d/3) triplets t_i (the last padded with zeros); each triplet
# is rho_i = ||t_i|| times a unit direction n_i; n_i goes through an
# equal-area octahedral map to (xi, eta) in [-1, 1]^2 ([P3] glossary
# entry for the octahedral map); xi and eta take b_dir-bit codebooks, rho takes a
# b_nrm-bit codebook, with (b_dir, b_nrm) = (b + 1, b - 1) ([P3] Contributions,
# the MSE-driven uneven split of bits: B_tri = 2 b_dir + b_nrm); a 3x3 joint rounding
# picks the final codes; the state is (gamma, I_dir, I_nrm).
# ---------------------------------------------------------------------------

def octo_bits(b: int) -> tuple[int, int]:
    """(b_dir, b_nrm) = (b + 1, b - 1) for a budget of b bits per coordinate."""
    if b < 2:
        raise ValueError("the triplet codec needs b >= 2 (b_nrm = b - 1 >= 1)")
    return b + 1, b - 1


def octo_triplets(d: int) -> int:
    """n_tri = ceil(d / 3)."""
    return -(-d // 3)


def oct_map(n):
    """Equal-area octahedral map of unit vectors n (..., 3) to (xi, eta).

    Upper hemisphere (z >= 0): L1 radius r = sqrt(1 - z) (the cap z' >= z has
    area 2 pi (1 - z), the diamond |xi| + |eta| <= r has area 2 r^2, ratio pi
    everywhere); along the diamond edge the azimuth phi = atan2(|y|, |x|) in
    [0, pi/2] moves linearly: |eta| = r * phi / (pi/2), |xi| = r - |eta|,
    signs of x and y.  Lower hemisphere: the same point reflected across the
    diamond edge, (|xi|, |eta|) -> (1 - |eta|, 1 - |xi|), which preserves area.
    """
    n = np.asarray(n, dtype=np.float64)
    x, y, z = n[..., 0], n[..., 1], n[..., 2]
    r = np.sqrt(np.maximum(1.0 - np.abs(z), 0.0))
    phi = np.arctan2(np.abs(y), np.abs(x))
    ae = r * phi / (np.pi / 2.0)
    ax = r - ae
    lower = z < 0
    ax, ae = np.where(lower, 1.0 - ae, ax), np.where(lower, 1.0 - ax, ae)
    sx = np.where(x < 0, -1.0, 1.0)
    sy = np.where(y < 0, -1.0, 1.0)
    return sx * ax, sy * ae


def oct_unmap(xi, eta):
    """Inverse of oct_map: (xi, eta) in [-1, 1]^2 to unit vectors (..., 3)."""
    xi = np.asarray(xi, dtype=np.float64)
    eta = np.asarray(eta, dtype=np.float64)
    ax, ae = np.abs(xi), np.abs(eta)
    lower = ax + ae > 1.0
    ax, ae = np.where(lower, 1.0 - ae, ax), np.where(lower, 1.0 - ax, ae)
    r = ax + ae
    z = 1.0 - r * r
    phi = np.where(r > 0, (np.pi / 2.0) * ae / np.where(r > 0, r, 1.0), 0.0)
    s = r * np.sqrt(np.maximum(2.0 - r * r, 0.0))          # sqrt(1 - z^2)
    x = np.where(xi < 0, -1.0, 1.0) * s * np.cos(phi)
    y = np.where(eta < 0, -1.0, 1.0) * s * np.sin(phi)
    return np.stack([x, y, np.where(lower, -z, z)], axis=-1)


def octo_dir_codebook(b_dir: int) -> np.ndarray:
    """Codebook C_xi of xi and eta.  For a uniformly random unit vector in
    R^d every triplet direction is uniform on S^2 (the triplet's law is
    invariant under rotations of R^3), so through an equal-area map xi and eta
    are uniform on [-1, 1]; the Lloyd-Max quantiser of the uniform density is
    the uniform one: c_j = -1 + (2j + 1) / 2^b_dir."""
    n = 1 << b_dir
    return -1.0 + (2.0 * np.arange(n) + 1.0) / n


def rho_cdf(r, d: int):
    """P(rho <= r) for the norm of one triplet of a uniformly random unit
    vector in R^d: rho^2 ~ Beta(3/2, (d - 3)/2)."""
    r = np.clip(np.asarray(r, dtype=np.float64), 0.0, 1.0)
    return special.betainc(1.5, (d - 3) / 2.0, r * r)


def rho_partial_mean(a, b, d: int):
    """Integral of r f_rho(r) over [a, b] = E[X^(1/2); a^2 <= X <= b^2] for
    X ~ Beta(3/2, beta): B(2, beta) / B(3/2, beta) * (I_{b^2}(2, beta) -
    I_{a^2}(2, beta)), beta = (d - 3)/2."""
    a = np.clip(np.asarray(a, dtype=np.float64), 0.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), 0.0, 1.0)
    be = (d - 3) / 2.0
    ratio = math.exp(special.betaln(2.0, be) - special.betaln(1.5, be))
    return ratio * (special.betainc(2.0, be, b * b) - special.betainc(2.0, be, a * a))


def rho_lloyd_max(d: int, bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Float64 Lloyd-Max quantiser of rho with 2^bits levels: thresholds at
    midpoints, centroids at cell conditional means, from quantile start."""
    n = 1 << bits
    q = (np.arange(n) + 0.5) / n
    c = np.sqrt(special.betaincinv(1.5, (d - 3) / 2.0, q))
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([0.0], t))
        hi = np.concatenate((t, [1.0]))
        new = rho_partial_mean(lo, hi, d) / (rho_cdf(hi, d) - rho_cdf(lo, d))
        moved = np.max(np.abs(new - c))
        c = new
        if moved < tol * np.max(c):
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    return c, 0.5 * (c[:-1] + c[1:])


def octo_codebooks(d: int, b: int):
    """Tables as stored (fp32 values held in float64):
    dirs[a, c] = fp32(oct_unmap(C_xi[a], C_xi[c])), shape (2^b_dir, 2^b_dir, 3);
    crho = fp32(Lloyd-Max centroids of rho)."""
    b_dir, b_nrm = octo_bits(b)
    cx = octo_dir_codebook(b_dir)
    dirs = oct_unmap(cx[:, None], cx[None, :]).astype(np.float32).astype(np.float64)
    c, _ = rho_lloyd_max(d, b_nrm)
    return dirs, c.astype(np.float32).astype(np.float64)


def _rotated_triplets(x, seed: int):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    gamma = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(gamma > 0, gamma, 1.0)
    u = np.where((gamma > 0)[..., None], x / safe[..., None], 0.0)
    y = u @ rotation_matrix(seed, d).T
    nt = octo_triplets(d)
    pad = np.zeros(y.shape[:-1] + (3 * nt - d,))
    return gamma, np.concatenate([y, pad], axis=-1).reshape(y.shape[:-1] + (nt, 3))


def octo_encode(x, seed: int, b: int, dirs, crho):
    """Triplet codes of vectors x (..., d).

    gamma = ||x||, u = x / gamma (0 when gamma = 0), y = R u cut into
    triplets t_i; rho_i = ||t_i||, n_i = t_i / rho_i (n_i = (0, 0, 1) when
    rho_i = 0); (xi, eta) = oct_map(n_i); the nearest codes j_xi, j_eta on the
    uniform grid (cell floor((v + 1) 2^(b_dir - 1)), clamped).  Joint rounding:
    for every (a, c) with a in {j_xi - 1, j_xi, j_xi + 1} and c in
    {j_eta - 1, j_eta, j_eta + 1} inside the grid (a-major, ascending), with
    n_hat = dirs[a, c] and p = t_i . n_hat, the norm code k minimising
    (p - crho_k)^2 (first on ties) and the error ||t_i - crho_k n_hat||^2; the
    first candidate of least error wins.
    Returns dict(a, c, k: int64 (..., n_tri), gamma, gamma16, err, t)."""
    gamma, t = _rotated_triplets(x, seed)
    out = octo_encode_triplets(t, b, dirs, crho)
    out.update(gamma=gamma, gamma16=fp16_norm(gamma), t=t)
    return out


def octo_encode_triplets(t, b: int, dirs, crho):
    """The per-triplet stage of octo_encode on triplets t (..., 3): returns
    dict(a, c, k, err)."""
    b_dir, _ = octo_bits(b)
    nd = 1 << b_dir
    t = np.asarray(t, dtype=np.float64)
    rho = np.sqrt(np.sum(t * t, axis=-1))
    n = np.where((rho > 0)[..., None], t / np.where(rho > 0, rho, 1.0)[..., None], np.array([0.0, 0.0, 1.0]))
    xi, eta = oct_map(n)
    jx = np.clip(np.floor((xi + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    je = np.clip(np.floor((eta + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    best = np.full(rho.shape, np.inf)
    A = np.zeros(rho.shape, np.int64)
    C = np.zeros(rho.shape, np.int64)
    K = np.zeros(rho.shape, np.int64)
    crho = np.asarray(crho, dtype=np.float64)
    for da in (-1, 0, 1):
        for dc in (-1, 0, 1):
            a, c = jx + da, je + dc
            ok = (a >= 0) & (a < nd) & (c >= 0) & (c < nd)
            nh = dirs[np.clip(a, 0, nd - 1), np.clip(c, 0, nd - 1)]
            p = np.sum(t * nh, axis=-1)
            k = np.argmin((p[..., None] - crho) ** 2, axis=-1)
            err = np.sum((t - crho[k][..., None] * nh) ** 2, axis=-1)
            take = ok & (err < best)
            best = np.where(take, err, best)
            A, C, K = np.where(take, a, A), np.where(take, c, C), np.where(take, k, K)
    return {"a": A, "c": C, "k": K, "err": best}


def octo_triplet_error(t, a, c, k, dirs, crho):
    """||t - crho[k] dirs[a, c]||^2 for given codes (the quantity the joint
    rounding minimises)."""
    nh = dirs[a, c]
    return np.sum((np.asarray(t) - np.asarray(crho)[k][..., None] * nh) ** 2, axis=-1)


def octo_decode(a, c, k, gamma16, seed: int, d: int, dirs, crho):
    """x_hat = gamma16 * R^T y_hat, y_hat the first d entries of the
    concatenated crho[k_i] * dirs[a_i, c_i] ([P3] Method step 7: each triplet
    rebuilt from its norm and direction codes)."""
    yh = np.asarray(crho)[k][..., None] * dirs[a, c]
    yh = yh.reshape(yh.shape[:-2] + (-1,))[..., :d]
    return np.asarray(gamma16, dtype=np.float64)[..., None] * (yh @ rotation_matrix(seed, d))


def octo_qjl_encode(x, seed: int, seed_qjl: int, b: int, dirs, crho):
    """OCTOPUS-QJL ([P3] Method step 8, the optional residual sketch that
    makes the dot-product estimate unbiased): the triplet codes of
    octo_encode, plus the one-bit sketch of what they leave out, taken as in
    qjl_encode.  y = R u is the rotated unit direction (the first d entries
    of the triplets), y_hat its reconstruction from the codes (octo_decode
    before the inverse rotation); r = y - y_hat, rho16 = fp16(||r||),
    z = R' r with R' the independent rotation of seed_qjl, bit_j = [z_j < 0].
    The logits then add scale * gamma16 * qjl_dot_estimate(bits, rho16, R q)
    to scale * q . x_hat (logits(..., qjl=...)).
    Returns octo_encode's dict plus qjl_bits (uint8 0/1, (..., d)), qjl_rho,
    qjl_rho16, qjl_z."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    e = octo_encode(x, seed, b, dirs, crho)
    y = e["t"].reshape(e["t"].shape[:-2] + (-1,))[..., :d]
    yh = np.asarray(crho)[e["k"]][..., None] * dirs[e["a"], e["c"]]
    yh = yh.reshape(yh.shape[:-2] + (-1,))[..., :d]
    r = y - yh
    rho = np.sqrt(np.sum(r * r, axis=-1))
    z = r @ rotation_matrix(seed_qjl, d).T
    e.update(qjl_bits=(z < 0).astype(np.uint8), qjl_rho=rho, qjl_rho16=fp16_norm(rho), qjl_z=z)
    return e


def octo_record_bytes(d: int, b: int) -> int:
    """Bytes of one vector's code record: n_tri fields of B_tri = 2 b_dir +
    b_nrm bits, triplet i at bit i * B_tri, fields xi | eta << b_dir |
    rho << 2 b_dir, LSB first; rounded up to whole 32-bit words (this build's
    layout; the page fixes none)."""
    b_dir, b_nrm = octo_bits(b)
    bits = octo_triplets(d) * (2 * b_dir + b_nrm)
    return 4 * (-(-bits // 32))


def octo_pack(a, c, k, b: int, d: int) -> np.ndarray:
    """Records (..., octo_record_bytes) of uint8 from codes (..., n_tri)."""
    b_dir, b_nrm = octo_bits(b)
    bt = 2 * b_dir + b_nrm
    a, c, k = (np.asarray(v, dtype=np.int64) for v in (a, c, k))
    field = a | (c << b_dir) | (k << (2 * b_dir))
    nt = field.shape[-1]
    bits = ((field[..., :, None] >> np.arange(bt)) & 1).reshape(field.shape[:-1] + (nt * bt,))
    nb = octo_record_bytes(d, b)
    full = np.zeros(field.shape[:-1] + (8 * nb,), np.int64)
    full[..., :nt * bt] = bits
    return (full.reshape(field.shape[:-1] + (nb, 8)) << np.arange(8)).sum(axis=-1).astype(np.uint8)


def octo_unpack(rec, b: int, d: int):
    """Codes (a, c, k), each (..., n_tri), from records."""
    b_dir, b_nrm = octo_bits(b)
    bt = 2 * b_dir + b_nrm
    nt = octo_triplets(d)
    rec = np.asarray(rec, dtype=np.uint8)
    bits = ((rec[..., :, None].astype(np.int64) >> np.arange(8)) & 1).reshape(rec.shape[:-1] + (-1,))
    f = (bits[..., :nt * bt].reshape(rec.shape[:-1] + (nt, bt)) << np.arange(bt)).sum(axis=-1)
    return f & ((1 << b_dir) - 1), (f >> b_dir) & ((1 << b_dir) - 1), f >> (2 * b_dir)
