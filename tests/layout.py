"""The library's physical storage layouts, written out as plain index rules (test side only).

The oracle keeps every cache and weight array in its logical order: a KV pool is [P][Hkv][S][D]
(element (page, kv head, slot, dim)), INT4/FP8 weight codes are [N][K] with scales [N][K/128].  The
library stores the same values in layouts chosen for its kernels' loads (documented in
include/kvfp8.h and include/wgemm.h).  Byte-exact comparisons of a device pool or device codes with the
oracle go through the functions here, which map between the two orders.  Nothing here is used by the
oracle or by the library; the hand-worked offsets and bijection checks in tests/test_layout.py pin it.

KV pools (element = one e4m3 byte or one bf16 value; a 16-byte chunk holds E = 16/elt elements).
Every (page, head) block is contiguous, blocks ordered page-major:
  K       the block is S/16 sub-page blocks of 16 tokens x D elements.  Inside one, a token's row is
          cut into 16-byte chunks c = q*NI + k (NI = D*elt/64, q in 0..3); token t = 4s + i of the
          sub-page keeps chunk c at chunk position ((s*NI + k)*4 + q)*4 + i.
  V       the block is V transposed: element (slot, d) at d*S + slot.
  latent  the block is row-major: element (slot, d) at slot*D + d (the logical order itself).

Weight codes (N output channels x K input channels, groups of 128 input channels):
  tiles of 16 output channels x 128 input channels, tile (t, g) at index t*(K/128) + g; lane
  l = 16*qq + nn of a tile holds output channel 16t + nn and input channels 128g + 32j + 8qq + e
  (j in 0..3, e in 0..7).  INT4: 16 bytes per lane, dword j holds the 8 codes of (j, e) as nibbles
  q + 8 with e = 2*(s%4) + s//4 in nibble slot s.  FP8: 32 bytes per lane, byte 8j + e.
  Scales: [N/16][K/128][16], element (t, g, nn) = scale of channel 16t + nn in group g.
"""
from __future__ import annotations

import numpy as np

KINDS = ("k", "v", "latent")


# ----------------------------------------------------------------------------- KV pools

def k_block_offsets(S: int, D: int, elt: int) -> np.ndarray:
    """int64 [S][D]: element offset of (slot, d) inside one (page, head) block of a K pool."""
    if S % 16 or (D * elt) % 64:
        raise ValueError(f"K layout needs S % 16 == 0 and a row of a multiple of 64 bytes (S={S}, D={D}, elt={elt})")
    E = 16 // elt
    NI = D * elt // 64
    slot = np.arange(S, dtype=np.int64)[:, None]
    d = np.arange(D, dtype=np.int64)[None, :]
    sub, tok = slot // 16, slot % 16
    grp, i = tok // 4, tok % 4
    chunk = d // E
    q, k = chunk // NI, chunk % NI
    pos = ((grp * NI + k) * 4 + q) * 4 + i
    return sub * 16 * D + pos * E + d % E


def v_block_offsets(S: int, Dv: int) -> np.ndarray:
    """int64 [S][Dv]: element offset of (slot, d) inside one (page, head) block of a V pool."""
    slot = np.arange(S, dtype=np.int64)[:, None]
    d = np.arange(Dv, dtype=np.int64)[None, :]
    return d * S + slot


def block_offsets(kind: str, S: int, D: int, elt: int) -> np.ndarray:
    if kind == "k":
        return k_block_offsets(S, D, elt)
    if kind == "v":
        return v_block_offsets(S, D)
    if kind == "latent":
        return np.arange(S * D, dtype=np.int64).reshape(S, D)
    raise ValueError(kind)


def to_device(pool: np.ndarray, kind: str, elt: int) -> np.ndarray:
    """Logical pool [P][H][S][D] -> the flat array the library stores."""
    P, H, S, D = pool.shape
    off = block_offsets(kind, S, D, elt).ravel()
    out = np.empty((P * H, S * D), dtype=pool.dtype)
    out[:, off] = pool.reshape(P * H, S * D)
    return out.reshape(-1)


def from_device(flat: np.ndarray, kind: str, shape, elt: int) -> np.ndarray:
    """The flat array the library stores -> logical pool [P][H][S][D]."""
    P, H, S, D = shape
    off = block_offsets(kind, S, D, elt).ravel()
    return np.asarray(flat).reshape(P * H, S * D)[:, off].reshape(P, H, S, D)


def element_offset(kind: str, page: int, head: int, slot: int, d: int, H: int, S: int, D: int, elt: int) -> int:
    """Flat element offset of one logical element in the library's layout."""
    return (page * H + head) * S * D + int(block_offsets(kind, S, D, elt)[slot, d])


# ----------------------------------------------------------------------------- weight codes

TILE_N = 16
GROUP = 128


def _lanes(N: int, K: int):
    """For every (n, k): (tile index, lane, j, e)."""
    if N % TILE_N or K % GROUP:
        raise ValueError(f"N = {N} must be a multiple of {TILE_N} and K = {K} of {GROUP}")
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    t, nn = n // TILE_N, n % TILE_N
    g, kk = k // GROUP, k % GROUP
    j, qq, e = kk // 32, (kk % 32) // 8, kk % 8
    return np.broadcast_arrays(t * (K // GROUP) + g, 16 * qq + nn, j, e)


def _w4_byte_shift(N: int, K: int):
    tile, lane, j, e = _lanes(N, K)
    slot = (e % 2) * 4 + e // 2            # the nibble slot s with e = 2*(s%4) + s//4
    return (tile * 64 + lane) * 16 + 4 * j + slot // 2, 4 * (slot % 2)


def pack_w4(q: np.ndarray) -> np.ndarray:
    """int8 codes [N][K] in [-8, 7] -> the library's packed INT4 bytes (N*K/2)."""
    N, K = q.shape
    byte, shift = _w4_byte_shift(N, K)
    nib = (q.astype(np.int64) + 8) & 0xF
    out = np.zeros(N * K // 2, dtype=np.int64)
    np.add.at(out, byte.ravel(), (nib << shift).ravel())
    return out.astype(np.uint8)


def unpack_w4(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    byte, shift = _w4_byte_shift(N, K)
    nib = (np.asarray(packed, dtype=np.uint8)[byte].astype(np.int64) >> shift) & 0xF
    return (nib - 8).astype(np.int8)


def _w8_index(N: int, K: int):
    tile, lane, j, e = _lanes(N, K)
    return (tile * 64 + lane) * 32 + 8 * j + e


def pack_w8(codes: np.ndarray) -> np.ndarray:
    N, K = codes.shape
    out = np.zeros(N * K, dtype=np.uint8)
    out[_w8_index(N, K).ravel()] = np.asarray(codes, dtype=np.uint8).ravel()
    return out


def unpack_w8(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    return np.asarray(packed, dtype=np.uint8)[_w8_index(N, K)]


def pack_scales(s_bits: np.ndarray) -> np.ndarray:
    """bf16 bits [N][K/128] -> [N/16][K/128][16]."""
    N, KG = s_bits.shape
    return np.ascontiguousarray(np.asarray(s_bits, dtype=np.uint16).reshape(N // TILE_N, TILE_N, KG)
                                .transpose(0, 2, 1))


def unpack_scales(s_packed: np.ndarray, N: int, K: int) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(s_packed, dtype=np.uint16).reshape(N // TILE_N, K // GROUP, TILE_N)
                                .transpose(0, 2, 1).reshape(N, K // GROUP))
