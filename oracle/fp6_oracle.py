"""Plain CPU oracle of the weight-only FP6 (W6A16) linear layer.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg.  Shares nothing with the HIP library.

What is computed, and where it comes from
-----------------------------------------
* FP6-LLM (arXiv 2401.14112), abstract: six-bit floating-point weights with
  16-bit activations; the two costs are irregular-width weight access and
  weight de-quantisation.
* TC-FPx explainer (duicuo.cn/w/184.html), section "redesigning the kernel
  solution": FP6 weights are de-quantised to FP16 ("disguised" as FP16) and the
  matrix product is then done in FP16; weights are re-ordered and packed
  offline into power-of-two-aligned pieces (6 = 2 + 4 bits).

The pages do not give the FP6 bit format, the scale granularity, rounding or a
packed layout.  The readings used here (each one stated where it is used):

* FP6 = e3m2: 1 sign, 3 exponent, 2 mantissa bits, exponent bias 3,
  subnormals, no inf/NaN, largest magnitude 28 (the OCP MX FP6 E3M2 element
  format).  Code bits (MSB..LSB): s e2 e1 e0 m1 m0.
* One fp16 scale per output row n: s_n = fp16_RNE(max_k |W[n,k]| / 28).
* Quantisation rounds |W/s_n| to the nearest e3m2 magnitude, ties to the even
  code, saturating at 28; the sign bit is copied from W (so -0 is kept).
* Dequantised weight Wdq[n,k] = fp16_RNE(v(c[n,k]) * s_n): the product is
  formed exactly in float64 and rounded once (IEEE round-to-nearest-even,
  gradual underflow, signed zero kept).
* Y_ref = X . Wdq^T accumulated in float64 (nn.Linear convention: X is
  [M,K], W is [N,K], Y is [M,N]).
* Packed layout v3 (the library's private offline format; any bijection is
  correct, this oracle checks the round trip): see :func:`unpack_scalar`.

Other widths (FP6-LLM abstract: one Tensor-Core kernel scheme for float weights
of several bit widths; TC-FPx explainer, section "redesigning the kernel
solution": a unified kernel for quantised weights of different widths up to
6 bits).  The pages name no formats; the reading used here is the plainest set
of small IEEE-like float formats (sign, exponent with bias 2^(E-1)-1,
subnormals, no inf/NaN), each with the same per-row fp16 scale, rounding and
de-quantisation rules as e3m2:
  e2m3 (6 bits, bias 1, max 7.5; the OCP MX FP6 E2M3 element format),
  e2m2 (5 bits, bias 1, max 7),
  e2m1 (4 bits, bias 1, max 6; the OCP MX FP4 E2M1 element format).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# O1: explicit e3m2 decode table (64 entries, index = 6-bit code).
# Codes 0..31 are the non-negative values (e = code>>2, m = code&3):
#   e = 0 (subnormal): m * 2^-4          -> 0, 0.0625, 0.125, 0.1875
#   e >= 1 (normal):   2^(e-3) * (1+m/4)
# Codes 32..63 are the same magnitudes with the sign bit set.
# ---------------------------------------------------------------------------
E3M2_VALUES = (
    0.0, 0.0625, 0.125, 0.1875,      # e=0 (subnormal)
    0.25, 0.3125, 0.375, 0.4375,     # e=1
    0.5, 0.625, 0.75, 0.875,         # e=2
    1.0, 1.25, 1.5, 1.75,            # e=3
    2.0, 2.5, 3.0, 3.5,              # e=4
    4.0, 5.0, 6.0, 7.0,              # e=5
    8.0, 10.0, 12.0, 14.0,           # e=6
    16.0, 20.0, 24.0, 28.0,          # e=7
    -0.0, -0.0625, -0.125, -0.1875,
    -0.25, -0.3125, -0.375, -0.4375,
    -0.5, -0.625, -0.75, -0.875,
    -1.0, -1.25, -1.5, -1.75,
    -2.0, -2.5, -3.0, -3.5,
    -4.0, -5.0, -6.0, -7.0,
    -8.0, -10.0, -12.0, -14.0,
    -16.0, -20.0, -24.0, -28.0,
)
# e2m3 (OCP MX FP6 E2M3): 1 sign, 2 exponent bits (bias 1), 3 mantissa bits,
# subnormals, no inf/NaN, max 7.5.  Index = e*8 + m:
#   e = 0 (subnormal): m / 8;   e >= 1: 2^(e-1) * (1 + m/8).
E2M3_VALUES = (
    0.0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,               # e=0 (subnormal)
    1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,               # e=1
    2.0, 2.25, 2.5, 2.75, 3.0, 3.25, 3.5, 3.75,                     # e=2
    4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0, 7.5,                         # e=3
    -0.0, -0.125, -0.25, -0.375, -0.5, -0.625, -0.75, -0.875,
    -1.0, -1.125, -1.25, -1.375, -1.5, -1.625, -1.75, -1.875,
    -2.0, -2.25, -2.5, -2.75, -3.0, -3.25, -3.5, -3.75,
    -4.0, -4.5, -5.0, -5.5, -6.0, -6.5, -7.0, -7.5,
)
# e2m2 (5 bits): 1 sign, 2 exponent bits (bias 1), 2 mantissa bits, max 7.
#   e = 0 (subnormal): m / 4;   e >= 1: 2^(e-1) * (1 + m/4).
E2M2_VALUES = (
    0.0, 0.25, 0.5, 0.75,            # e=0 (subnormal)
    1.0, 1.25, 1.5, 1.75,            # e=1
    2.0, 2.5, 3.0, 3.5,              # e=2
    4.0, 5.0, 6.0, 7.0,              # e=3
    -0.0, -0.25, -0.5, -0.75,
    -1.0, -1.25, -1.5, -1.75,
    -2.0, -2.5, -3.0, -3.5,
    -4.0, -5.0, -6.0, -7.0,
)
# e2m1 (OCP MX FP4 E2M1): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit,
# max 6.   e = 0 (subnormal): m / 2;   e >= 1: 2^(e-1) * (1 + m/2).
E2M1_VALUES = (
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
)


class Format:
    """One small float weight format.

    bits: code width (sign = top bit); table: value of every code (explicit);
    max: largest magnitude (the quantiser divides the row maximum by it);
    scale_limit: rows must have |s| below it (the library's exactness range,
    see quantize_rows); ebits, mbits, bias: the field widths and exponent bias
    the table follows.
    """

    def __init__(self, name, bits, ebits, mbits, bias, values, vmax, scale_limit):
        self.name = name
        self.bits = bits
        self.ebits = ebits
        self.mbits = mbits
        self.bias = bias
        self.table = np.array(values, dtype=np.float64)
        if self.table.size != 1 << bits:
            raise AssertionError("table size does not match the code width")
        self.nmag = 1 << (bits - 1)
        self.mags = self.table[: self.nmag]
        self.mids = (self.mags[:-1] + self.mags[1:]) / 2.0   # exact (short dyadics)
        self.max = vmax
        self.scale_limit = scale_limit


FORMATS = {
    "e3m2": Format("e3m2", 6, 3, 2, 3, E3M2_VALUES, 28.0, 16.0),
    "e2m3": Format("e2m3", 6, 2, 3, 1, E2M3_VALUES, 7.5, 4.0),
    "e2m2": Format("e2m2", 5, 2, 2, 1, E2M2_VALUES, 7.0, 4.0),
    "e2m1": Format("e2m1", 4, 2, 1, 1, E2M1_VALUES, 6.0, math.inf),
}
_TABLE = FORMATS["e3m2"].table
_MAGS = FORMATS["e3m2"].mags
_MIDS = FORMATS["e3m2"].mids
E3M2_MAX = 28.0


def _fmt(fmt) -> Format:
    if isinstance(fmt, Format):
        return fmt
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}")
    return FORMATS[fmt]


def decode(codes, fmt="e3m2") -> np.ndarray:
    """v(c) for an array of codes of the format, as float64 (table lookup)."""
    f = _fmt(fmt)
    c = np.asarray(codes)
    if c.size and (c.min() < 0 or c.max() >= (1 << f.bits)):
        raise ValueError(f"{f.bits}-bit codes must lie in 0..{(1 << f.bits) - 1}")
    return f.table[c.astype(np.int64)]


def encode_rne(x, fmt="e3m2") -> np.ndarray:
    """Nearest code for float64 values, ties to the even code.

    The magnitude |x| is mapped to the closest of the format's magnitudes; an
    exact midpoint goes to the even code (lowest mantissa bit 0); |x| at or
    beyond the largest magnitude saturates to it.  The sign bit (the code's top
    bit) is the IEEE sign bit of x, so -0.0 and small negatives that round to
    zero give the negative-zero code.  NaN is rejected.
    """
    f = _fmt(fmt)
    mids = f.mids
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN cannot be encoded (no NaN codes)")
    a = np.abs(x)
    # below = number of midpoints strictly below a: mids[below-1] < a <= mids[below]
    below = np.searchsorted(mids, a, side="left")
    idx = below.copy()
    # exact midpoint: a == mids[below]; choose the even one of (below, below+1)
    at_mid = np.zeros(a.shape, dtype=bool)
    inb = below < mids.size
    at_mid[inb] = a[inb] == mids[below[inb]]
    tie_idx = np.where(below % 2 == 0, below, below + 1)
    idx = np.where(at_mid, tie_idx, idx)
    idx = np.minimum(idx, f.nmag - 1)                 # saturate (also +inf)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << (f.bits - 1)) | idx).astype(np.uint8)


def fp16_rne(x) -> np.ndarray:
    """Round float64 values once to IEEE binary16 (RNE, subnormals kept;
    magnitudes beyond the largest binary16 round to infinity, as IEEE does)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


# ---------------------------------------------------------------------------
# O2: per-row quantiser (input preparation, not part of the timed path).
# ---------------------------------------------------------------------------
def quantize_rows(W, fmt="e3m2") -> tuple[np.ndarray, np.ndarray]:
    """W fp32 [N,K] -> (codes uint8 [N,K], scales fp16 [N]).

    s_n = fp16_RNE(float64(max_k |W[n,k]|) / vmax) (vmax: the format's largest
    magnitude); x = float64(W)/float64(s_n); codes = encode_rne(x).  A row
    whose scale is 0 gets all-zero codes.  Rows whose scale is not finite or
    reaches the format's limit are rejected (16 for e3m2, 4 for e2m3 and e2m2:
    the library folds s * 2^12 or s * 2^14 as one fp16, exact only below it;
    e2m1 has no limit beyond finiteness).
    """
    f = _fmt(fmt)
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise ValueError("W must be a 2-D float32 array")
    if not np.isfinite(W).all():
        raise ValueError("W must be finite")
    amax = np.abs(W).max(axis=1).astype(np.float64) if W.shape[1] else np.zeros(W.shape[0])
    scales = fp16_rne(amax / f.max)
    s64 = scales.astype(np.float64)
    if not np.isfinite(s64).all() or (np.abs(s64) >= f.scale_limit).any():
        raise ValueError("row scale out of the exact range")
    codes = np.zeros(W.shape, dtype=np.uint8)
    nz = s64 != 0.0
    if nz.any():
        q = W[nz].astype(np.float64) / s64[nz][:, None]
        codes[nz] = encode_rne(q, f)
    return codes, scales


def quantize_rows_sampled(W_rows, fmt="e3m2") -> tuple[np.ndarray, np.ndarray]:
    """Quantise a subset of rows (rows are independent); same as quantize_rows."""
    return quantize_rows(W_rows, fmt)


# ---------------------------------------------------------------------------
# O3: packed layout v3.
#
# Codes c[n][k] with N % 16 == 0 and K % 256 == 0.  The buffer holds
# N*K*bits/8 bytes in tiles of 16 rows x 256 k.  Tile (nb, kb) starts at byte
# (kb*(N/16) + nb) * tile_bytes (k-block major, row-block minor).  Inside a
# tile, local row r in 0..15 and local k = 32*j + 8*g + i (j: k-step 0..7,
# g: lane group 0..3, i: element 0..7) belong to lane L = 16*g + r.
#
# FP6 e3m2 (tile 3072 bytes).  Each code splits into a 2-bit piece (bits s,e2
# = c>>4) and a 4-bit piece (bits e1,e0,m1,m0 = c&15).
#   * 2-bit plane: bytes [0,1024) of the tile.  Lane L owns the 16 bytes at
#     16*L, as 4 little-endian 32-bit words; word j//2 holds k-steps j and
#     j+1.  Element i of k-step j belongs to group G = i//4 at byte E = i%4;
#     with rho = 4*(j%2) + 2*G, bit e2 sits at position (4 + 8*E + rho) mod
#     32 and bit s at (7 + 8*E + rho) mod 32 (the four rho values put the 16
#     elements of a word on the 16 even and the 16 odd positions).
#   * 4-bit plane: bytes [1024,3072).  k-steps 0..3 in [1024,2048), 4..7 in
#     [2048,3072); lane L owns 16 bytes at 16*L in each half, word j%4 is
#     k-step j.  Element i occupies nibble slot 2*(i%4) + i//4, i.e. bits
#     4*slot .. 4*slot+3 (elements 0..3 in the low nibbles of bytes 0..3,
#     elements 4..7 in the high nibbles).
# FP6 e2m3 (tile 3072 bytes): 2-bit piece = s,e1; 4-bit piece = e0,m2,m1,m0.
#   With pair p = 4*(j%2) + i//2 and half h = i%2, b = [0,1,2,3,8,9,10,
#   11][p]: bit e1 sits at b + 16*h and bit s at b + 4 + 16*h of the 2-bit
#   word; element i occupies nibble slot (i//2) + 4*(i%2) of the 4-bit word.
# FP5 e2m2 (tile 2560 bytes): 4-bit piece (e1,e0,m1,m0 = c&15) in a 4-bit
#   plane at bytes [0,2048) laid out as the e3m2 one (element i in nibble
#   slot 2*(i%4) + i//4); the sign (c>>4) in a 1-bit plane at [2048,2560):
#   lane L owns the 8 bytes at 2048 + 8*L as two words; word j//4 holds
#   k-steps 4*(j//4)..+3, and the sign of element i of k-step j sits at bit
#   (7 + 8*(i%4) + 2*(j%4) + i//4) mod 32 (layout v3; v1 and v2 put it at
#   4*(j%4) + i//2 + 16*(i%2) with the e2m3 nibble order).
# FP4 e2m1 (tile 2048 bytes): one 4-bit plane at [0,2048) laid out as the FP6
#   one, holding the whole code, element i in nibble slot i (natural order).
# ---------------------------------------------------------------------------
TILE_N = 16
TILE_K = 256
TILE_BYTES = 3072
_E2M3_BASE = (0, 1, 2, 3, 8, 9, 10, 11)


def tile_bytes(fmt="e3m2") -> int:
    """Bytes of one 16 x 256 tile: 4096 codes of the format's width."""
    return 4096 * _fmt(fmt).bits // 8


def packed_bytes(N: int, K: int, fmt="e3m2") -> int:
    return N * K * _fmt(fmt).bits // 8


def _check_shape(N: int, K: int) -> None:
    if N <= 0 or K <= 0 or N % TILE_N or K % TILE_K:
        raise ValueError("layout v3 needs N % 16 == 0 and K % 256 == 0, both > 0")


def _locate(N: int, K: int, n: int, k: int):
    """e3m2: byte offset of the 2-bit word, bit positions, and 4-bit word + shift for (n,k)."""
    nb, r = divmod(n, TILE_N)
    kb, kk = divmod(k, TILE_K)
    j, rem = divmod(kk, 32)
    g, i = divmod(rem, 8)
    lane = 16 * g + r
    base = (kb * (N // TILE_N) + nb) * TILE_BYTES
    grp, e = divmod(i, 4)
    rho = 4 * (j % 2) + 2 * grp
    w2 = base + 16 * lane + 4 * (j // 2)
    bit_e2 = (4 + 8 * e + rho) % 32
    bit_s = (7 + 8 * e + rho) % 32
    w4 = base + 1024 + 1024 * (j // 4) + 16 * lane + 4 * (j % 4)
    nib = 4 * (2 * e + grp)
    return w2, bit_e2, bit_s, w4, nib


def _slots(fmt, N: int, K: int, n: int, k: int):
    """Where each bit of code (n, k) lives: a list of (byte offset of its
    little-endian 32-bit word, bit in that word, bit of the code)."""
    f = _fmt(fmt)
    nb, r = divmod(n, TILE_N)
    kb, kk = divmod(k, TILE_K)
    j, rem = divmod(kk, 32)
    g, i = divmod(rem, 8)
    lane = 16 * g + r
    tb = tile_bytes(f)
    base = (kb * (N // TILE_N) + nb) * tb
    p = 4 * (j % 2) + i // 2
    h = i % 2
    if f.name == "e3m2":
        w2, b_e2, b_s, w4, nib = _locate(N, K, n, k)
        return [(w2, b_e2, 4), (w2, b_s, 5)] + [(w4, nib + b, b) for b in range(4)]
    if f.name == "e2m3":
        w2 = base + 16 * lane + 4 * (j // 2)
        b = _E2M3_BASE[p] + 16 * h
        w4 = base + 1024 + 1024 * (j // 4) + 16 * lane + 4 * (j % 4)
        nib = 4 * ((i // 2) + 4 * (i % 2))
        return [(w2, b, 4), (w2, b + 4, 5)] + [(w4, nib + q, q) for q in range(4)]
    if f.name == "e2m2":
        w4 = base + 1024 * (j // 4) + 16 * lane + 4 * (j % 4)
        nib = 4 * (2 * (i % 4) + i // 4)
        w1 = base + 2048 + 8 * lane + 4 * (j // 4)
        b1 = (7 + 8 * (i % 4) + 2 * (j % 4) + i // 4) % 32
        return [(w4, nib + q, q) for q in range(4)] + [(w1, b1, 4)]
    if f.name == "e2m1":
        w4 = base + 1024 * (j // 4) + 16 * lane + 4 * (j % 4)
        return [(w4, 4 * i + q, q) for q in range(4)]
    raise AssertionError(f.name)


def _get_word(buf, off: int) -> int:
    return buf[off] | (buf[off + 1] << 8) | (buf[off + 2] << 16) | (buf[off + 3] << 24)


def _set_word(buf, off: int, val: int) -> None:
    for b in range(4):
        buf[off + b] = (val >> (8 * b)) & 0xFF


def pack_scalar(codes, fmt="e3m2") -> np.ndarray:
    """Scalar packer of layout v3 (pure Python; small inputs only).

    Used only to pin :func:`unpack_scalar` (bijection checks); the library has
    its own packer.
    """
    f = _fmt(fmt)
    c = np.asarray(codes, dtype=np.uint8)
    N, K = c.shape
    _check_shape(N, K)
    if c.max(initial=0) >= (1 << f.bits):
        raise ValueError(f"codes must lie in 0..{(1 << f.bits) - 1}")
    buf = bytearray(packed_bytes(N, K, f))
    for n in range(N):
        for k in range(K):
            code = int(c[n, k])
            for off, wbit, cbit in _slots(f, N, K, n, k):
                _set_word(buf, off, _get_word(buf, off) | (((code >> cbit) & 1) << wbit))
    return np.frombuffer(bytes(buf), dtype=np.uint8).copy()


def unpack_scalar(packed, N: int, K: int, fmt="e3m2") -> np.ndarray:
    """Scalar unpacker of layout v3 (pure Python loop over every code)."""
    f = _fmt(fmt)
    _check_shape(N, K)
    buf = bytes(np.asarray(packed, dtype=np.uint8).ravel())
    if len(buf) != packed_bytes(N, K, f):
        raise ValueError("packed buffer has the wrong size")
    out = np.zeros((N, K), dtype=np.uint8)
    for n in range(N):
        for k in range(K):
            code = 0
            for off, wbit, cbit in _slots(f, N, K, n, k):
                code |= ((_get_word(buf, off) >> wbit) & 1) << cbit
            out[n, k] = code
    return out


def _tile_map(fmt):
    """For one tile: byte index and bit in byte of every (row, k, code bit)."""
    f = _fmt(fmt)
    byte_idx = np.zeros((f.bits, TILE_N, TILE_K), dtype=np.int64)
    bit_idx = np.zeros((f.bits, TILE_N, TILE_K), dtype=np.int64)
    for r in range(TILE_N):
        for k in range(TILE_K):
            for off, wbit, cbit in _slots(f, TILE_N, TILE_K, r, k):
                byte_idx[cbit, r, k] = off + wbit // 8
                bit_idx[cbit, r, k] = wbit % 8
    return byte_idx, bit_idx


def unpack_tiles(packed, N: int, K: int, fmt="e3m2") -> np.ndarray:
    """Vectorised unpacker of any format: one tile's bit map applied to all tiles."""
    f = _fmt(fmt)
    _check_shape(N, K)
    p = np.asarray(packed, dtype=np.uint8).ravel()
    if p.size != packed_bytes(N, K, f):
        raise ValueError("packed buffer has the wrong size")
    nbk, kbk = N // TILE_N, K // TILE_K
    # the buffer's tiles are in (kb, nb) order
    tiles = p.reshape(kbk, nbk, tile_bytes(f)).transpose(1, 0, 2).astype(np.int64)
    byte_idx, bit_idx = _tile_map(f)
    out = np.zeros((nbk, kbk, TILE_N, TILE_K), dtype=np.int64)
    for b in range(f.bits):
        out |= ((tiles[:, :, byte_idx[b]] >> bit_idx[b]) & 1) << b
    return out.transpose(0, 2, 1, 3).reshape(N, K).astype(np.uint8)


def unpack_np(packed, N: int, K: int) -> np.ndarray:
    """Vectorised unpacker of layout v3 (e3m2; same definition, NumPy indexing)."""
    _check_shape(N, K)
    p = np.asarray(packed, dtype=np.uint8).ravel()
    if p.size != N * K * 3 // 4:
        raise ValueError("packed buffer has the wrong size")
    nbk, kbk = N // TILE_N, K // TILE_K
    tiles = p.reshape(kbk, nbk, TILE_BYTES).transpose(1, 0, 2)  # buffer in (kb, nb) order
    # words: 2-bit plane [nbk,kbk,lane=64,word=4]; 4-bit [nbk,kbk,half=2,lane=64,word=4]
    w2 = tiles[:, :, :1024].copy().view("<u4").reshape(nbk, kbk, 64, 4).astype(np.int64)
    w4 = tiles[:, :, 1024:].copy().view("<u4").reshape(nbk, kbk, 2, 64, 4).astype(np.int64)
    out = np.zeros((nbk, kbk, TILE_N, 8, 4, 8), dtype=np.int64)  # [nb,kb,r,j,g,i]
    for j in range(8):
        for i in range(8):
            grp, e = divmod(i, 4)
            rho = 4 * (j % 2) + 2 * grp
            b_e2 = (4 + 8 * e + rho) % 32
            b_s = (7 + 8 * e + rho) % 32
            nib = 4 * (2 * e + grp)
            for g in range(4):
                lanes = slice(16 * g, 16 * g + 16)
                v2 = w2[:, :, lanes, j // 2]
                v4 = w4[:, :, j // 4, lanes, j % 4]
                out[:, :, :, j, g, i] = (((v2 >> b_s) & 1) << 5) | (((v2 >> b_e2) & 1) << 4) | ((v4 >> nib) & 0xF)
    # [nb,kb,r,j,g,i] -> [nb,r,kb,j,g,i] -> [N,K]
    return out.transpose(0, 2, 1, 3, 4, 5).reshape(N, K).astype(np.uint8)


# ---------------------------------------------------------------------------
# O4: dequantisation.
# ---------------------------------------------------------------------------
def dequant_ref(codes, scales, fmt="e3m2") -> np.ndarray:
    """Wdq[n,k] = fp16_RNE(v(c[n,k]) * s_n), product exact in float64, one rounding."""
    v = decode(codes, fmt)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if v.ndim != 2 or s.shape != (v.shape[0],):
        raise ValueError("codes [N,K] and scales [N] expected")
    return fp16_rne(v * s[:, None])


# ---------------------------------------------------------------------------
# O5: GEMM in float64.
# ---------------------------------------------------------------------------
def gemm_ref(X, Wdq) -> np.ndarray:
    """Y_ref[m,n] = sum_k X[m,k] * Wdq[n,k], float64 accumulation (BLAS dgemm)."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    W64 = np.asarray(Wdq, dtype=np.float16).astype(np.float64)
    return X64 @ W64.T


def gemm_naive(X, Wdq) -> np.ndarray:
    """Triple loop in plain Python floats (tiny shapes only)."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    W64 = np.asarray(Wdq, dtype=np.float16).astype(np.float64)
    M, K = X64.shape
    N = W64.shape[0]
    Y = np.zeros((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(X64[m, k]) * float(W64[n, k])
            Y[m, n] = acc
    return Y


# ---------------------------------------------------------------------------
# Acceptance: fp16 output with fp32 accumulation is correct when every element
# satisfies |Y - Y_ref| <= 2e-3 (|Y_ref| + rms(Y_ref)) and the relative
# Frobenius error is <= 5e-4.
# ---------------------------------------------------------------------------
TOL_ELEM = 2e-3
TOL_FROB = 5e-4


def tolerance_report(Y, Y_ref, rms=None) -> dict:
    """Compare a device result with Y_ref.  ``rms`` may be given when Y_ref is a
    sample of a larger output (then it is the rms of the whole output)."""
    Y64 = np.asarray(Y, dtype=np.float64)
    R = np.asarray(Y_ref, dtype=np.float64)
    if Y64.shape != R.shape:
        raise ValueError("shape mismatch")
    if R.size == 0:
        return {"ok": True, "max_ratio": 0.0, "frob": 0.0, "rms": 0.0}
    if rms is None:
        rms = math.sqrt(float(np.mean(R * R)))
    err = np.abs(Y64 - R)
    bound = TOL_ELEM * (np.abs(R) + rms)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    nref = math.sqrt(float(np.sum(R * R)))
    nerr = math.sqrt(float(np.sum((Y64 - R) ** 2)))
    frob = nerr / nref if nref > 0 else (0.0 if nerr == 0 else math.inf)
    finite = bool(np.isfinite(Y64).all())
    max_ratio = float(ratio.max())
    return {
        "ok": finite and max_ratio <= 1.0 and frob <= TOL_FROB,
        "max_ratio": max_ratio,
        "frob": frob,
        "rms": rms,
    }
