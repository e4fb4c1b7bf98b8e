"""Plain CPU oracle of the 2:4-sparse FP6 (e3m2) weight-only linear layer.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg.  Shares nothing with the HIP library.

What is computed, and where it comes from
-----------------------------------------
* Sparse-Marlin (first page, the post on quantised-weight kernels, points on
  2:4 sparsity): weights that are both quantised and 2:4 structured-sparse (of
  every 4 consecutive weights along the reduction dimension at most 2 are
  non-zero), run on sparse matrix units, with the quantised values, the
  sparsity metadata and the quantisation statistics laid out together.
* The same fused FP6 linear layer as :mod:`oracle.fp6_oracle` otherwise:
  Wdq[n,k] = fp16_RNE(v(c) * s_n) at kept positions and 0 elsewhere,
  Y_ref = X . Wdq^T in float64.

The pages give no pruning rule, metadata format or layout.  Readings used:

* Pruning (input preparation): in every aligned group of 4 weights along k,
  keep the 2 of largest magnitude; equal magnitudes keep the lower index.
  Exactly 2 positions are kept per group (a kept weight may be zero).
* Compressed form: codes[n, 2t+s] and pos[n, 2t+s] (s = 0, 1) are the code
  and the position (0..3) inside dense group t of the s-th kept weight, with
  pos[n, 2t] < pos[n, 2t+1].
* Quantisation: :func:`oracle.fp6_oracle.quantize_rows` applied to the kept
  values (so s_n = fp16_RNE(max|kept| / 28) = fp16_RNE(max|W_pruned| / 28)).
* Packed 2:4 layout (the library's private offline format), see
  :func:`_sparse_slots`.
"""

from __future__ import annotations

import numpy as np

from . import fp6_oracle as fo

TILE_N = 16
TILE_K = 512          # dense k per tile
TILE_BYTES = 4096     # 3072 bytes of FP6 codes + 1024 bytes of positions


# ---------------------------------------------------------------------------
# S1: pruning and compression (input preparation).
# ---------------------------------------------------------------------------
def prune_2of4(W) -> np.ndarray:
    """Boolean keep-mask [N, K]: in each group of 4 along k, the 2 entries of
    largest |W|, the lower index first among equal magnitudes."""
    W = np.asarray(W)
    if W.ndim != 2 or W.shape[1] % 4:
        raise ValueError("W must be [N, K] with K % 4 == 0")
    N, K = W.shape
    g = np.abs(W.astype(np.float64)).reshape(N, K // 4, 4)
    # stable sort on -|w| keeps the lower index first among ties
    order = np.argsort(-g, axis=2, kind="stable")
    mask = np.zeros_like(g, dtype=bool)
    np.put_along_axis(mask, order[:, :, :2], True, axis=2)
    return mask.reshape(N, K)


def compress(W, mask):
    """(values [N, K/2], pos [N, K/2] uint8) of the kept entries, ascending
    position inside each group."""
    W = np.asarray(W)
    mask = np.asarray(mask, dtype=bool)
    N, K = W.shape
    m4 = mask.reshape(N, K // 4, 4)
    if not (m4.sum(axis=2) == 2).all():
        raise ValueError("mask must keep exactly 2 of every 4")
    pos = np.nonzero(m4)[2].reshape(N, K // 4, 2).astype(np.uint8)   # ascending by construction
    vals = np.take_along_axis(W.reshape(N, K // 4, 4), pos.astype(np.int64), axis=2)
    return vals.reshape(N, K // 2), pos.reshape(N, K // 2)


def expand(vals, pos, K: int, fill=0):
    """Dense [N, K] from a compressed pair (zeros, or `fill`, elsewhere)."""
    vals = np.asarray(vals)
    pos = np.asarray(pos, dtype=np.int64)
    N = vals.shape[0]
    if vals.shape != (N, K // 2) or pos.shape != (N, K // 2):
        raise ValueError("compressed arrays must be [N, K/2]")
    out = np.full((N, K // 4, 4), fill, dtype=vals.dtype)
    np.put_along_axis(out, pos.reshape(N, K // 4, 2), vals.reshape(N, K // 4, 2), axis=2)
    return out.reshape(N, K)


def quantize_sparse(W):
    """W fp32 [N, K] -> (codes [N, K/2], pos [N, K/2], scales fp16 [N]) after
    2:4 magnitude pruning; the kept values are quantised per row."""
    W = np.asarray(W)
    if W.dtype != np.float32:
        raise ValueError("W must be float32")
    mask = prune_2of4(W)
    vals, pos = compress(W, mask)
    codes, scales = fo.quantize_rows(np.ascontiguousarray(vals, dtype=np.float32))
    return codes, pos, scales


def dequant_ref(codes, pos, scales, K: int) -> np.ndarray:
    """Dense Wdq fp16 [N, K]: fp16_RNE(v(c) * s_n) at kept positions, +0 elsewhere."""
    wk = fo.dequant_ref(codes, scales)                 # [N, K/2] fp16
    return expand(wk, pos, K, fill=np.float16(0.0))


# ---------------------------------------------------------------------------
# S2: packed 2:4 layout.
#
# N % 16 == 0 and K % 512 == 0; N*K/2 bytes in tiles of 16 rows x 512 dense
# k (4096 bytes) at (nb*(K/512) + kb) * 4096.  A tile holds 8 k-steps of 64
# dense k, each the operand of one v_smfmac_f32_16x16x64_f16 (16 rows x 64 k
# with 2 of every 4 kept).  For step j and wave lane L = 16*g + r (row r),
# element i (0..7) of the lane is kept weight s = i%2 of the dense group at
# k-offset 64*j + 32*(g%2) + 16*(i/4) + 8*(g/2) + 4*((i%4)/2) of the tile:
#   * its 6-bit code sits where the dense FP6 e3m2 packing puts the code of
#     lane L, k-step j, element i in bytes [0, 3072) of the tile;
#   * its position inside the group (0..3) is the 2-bit field at bit
#     16*(j%2) + 2*i of the little-endian word at byte 3072 + 16*L + 4*(j/2).
# ---------------------------------------------------------------------------
def _check_shape(N: int, K: int) -> None:
    if N <= 0 or K <= 0 or N % TILE_N or K % TILE_K:
        raise ValueError("the 2:4 layout needs N % 16 == 0 and K % 512 == 0, both > 0")


def packed_bytes(N: int, K: int) -> int:
    return N * K // 2


def _element_of(kk: int):
    """Dense k-offset kk (0..511) inside a tile -> (j, g_lo, g_hi, i_no_s):
    the step, the lane-group bits and the element without its s bit."""
    j, u = divmod(kk, 64)
    u //= 4                       # dense group inside the step, 0..15
    # offset 4u = 32*(g%2) + 16*(i/4) + 8*(g/2) + 4*((i%4)/2)
    g = (u >> 3) + 2 * ((u >> 1) & 1)
    i_base = 4 * ((u >> 2) & 1) + 2 * (u & 1)
    return j, g, i_base


def _sparse_slots(N: int, K: int, n: int, t2: int):
    """Where kept weight t2 = 2t + s of row n lives: a list of (byte offset of
    a little-endian 32-bit word, bit in that word, what) with `what` = ('c', b)
    for code bit b or ('p', b) for position bit b."""
    nb, r = divmod(n, TILE_N)
    t, s = divmod(t2, 2)
    kb, tt = divmod(t, TILE_K // 4)          # dense group inside the tile
    j, g, i_base = _element_of(4 * tt)
    i = i_base + s
    lane = 16 * g + r
    base = (nb * (K // TILE_K) + kb) * TILE_BYTES
    # code bits: dense FP6 e3m2 tile positions of (lane, k-step j, element i)
    w2, b_e2, b_s, w4, nib = fo._locate(16, 256, r, 32 * j + 8 * g + i)
    out = [(base + w2, b_e2, ("c", 4)), (base + w2, b_s, ("c", 5))]
    out += [(base + w4, nib + b, ("c", b)) for b in range(4)]
    wp = base + 3072 + 16 * lane + 4 * (j // 2)
    out += [(wp, 16 * (j % 2) + 2 * i, ("p", 0)), (wp, 16 * (j % 2) + 2 * i + 1, ("p", 1))]
    return out


def pack_scalar(codes, pos, K: int) -> np.ndarray:
    """Scalar packer of the 2:4 layout (pure Python; small inputs only)."""
    codes = np.asarray(codes, dtype=np.uint8)
    pos = np.asarray(pos, dtype=np.uint8)
    N = codes.shape[0]
    _check_shape(N, K)
    if codes.shape != (N, K // 2) or pos.shape != (N, K // 2):
        raise ValueError("codes and pos must be [N, K/2]")
    if codes.max(initial=0) > 63 or pos.max(initial=0) > 3:
        raise ValueError("codes must be < 64 and positions < 4")
    p2 = pos.reshape(N, K // 4, 2)
    if not (p2[:, :, 0] < p2[:, :, 1]).all():
        raise ValueError("positions inside a group must be increasing")
    buf = bytearray(packed_bytes(N, K))
    for n in range(N):
        for t2 in range(K // 2):
            vals = {"c": int(codes[n, t2]), "p": int(pos[n, t2])}
            for off, bit, (what, b) in _sparse_slots(N, K, n, t2):
                fo._set_word(buf, off, fo._get_word(buf, off) | (((vals[what] >> b) & 1) << bit))
    return np.frombuffer(bytes(buf), dtype=np.uint8).copy()


def unpack_scalar(packed, N: int, K: int):
    """Scalar unpacker: (codes [N, K/2], pos [N, K/2])."""
    _check_shape(N, K)
    buf = bytes(np.asarray(packed, dtype=np.uint8).ravel())
    if len(buf) != packed_bytes(N, K):
        raise ValueError("packed buffer has the wrong size")
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    pos = np.zeros((N, K // 2), dtype=np.uint8)
    for n in range(N):
        for t2 in range(K // 2):
            v = {"c": 0, "p": 0}
            for off, bit, (what, b) in _sparse_slots(N, K, n, t2):
                v[what] |= ((fo._get_word(buf, off) >> bit) & 1) << b
            codes[n, t2] = v["c"]
            pos[n, t2] = v["p"]
    return codes, pos


def _tile_map():
    """Byte and bit of every (row, kept index, bit) of one tile; bits 0..5 are
    code bits, 6..7 position bits."""
    byte_idx = np.zeros((8, TILE_N, TILE_K // 2), dtype=np.int64)
    bit_idx = np.zeros((8, TILE_N, TILE_K // 2), dtype=np.int64)
    for r in range(TILE_N):
        for t2 in range(TILE_K // 2):
            for off, bit, (what, b) in _sparse_slots(TILE_N, TILE_K, r, t2):
                q = b if what == "c" else 6 + b
                byte_idx[q, r, t2] = off + bit // 8
                bit_idx[q, r, t2] = bit % 8
    return byte_idx, bit_idx


def unpack_tiles(packed, N: int, K: int):
    """Vectorised unpacker (one tile's bit map applied to every tile)."""
    _check_shape(N, K)
    p = np.asarray(packed, dtype=np.uint8).ravel()
    if p.size != packed_bytes(N, K):
        raise ValueError("packed buffer has the wrong size")
    nbk, kbk = N // TILE_N, K // TILE_K
    tiles = p.reshape(nbk, kbk, TILE_BYTES).astype(np.int64)
    byte_idx, bit_idx = _tile_map()
    v = np.zeros((8, nbk, kbk, TILE_N, TILE_K // 2), dtype=np.int64)
    for q in range(8):
        v[q] = (tiles[:, :, byte_idx[q]] >> bit_idx[q]) & 1
    codes = sum(v[b] << b for b in range(6))
    pos = v[6] | (v[7] << 1)
    def to_rows(a):
        return a.transpose(0, 2, 1, 3).reshape(N, K // 2).astype(np.uint8)
    return to_rows(codes), to_rows(pos)
