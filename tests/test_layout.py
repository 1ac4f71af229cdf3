"""Pins of the test-side mapping to the library's storage layouts (tests/layout.py): hand-worked offsets,
bijections and round trips.  The oracle holds pools and weight codes in logical order; every byte-exact
comparison with device memory goes through this mapping, so it is pinned here on its own (CPU only)."""
import numpy as np
import pytest

from tests import layout


def _k(page, head, slot, d, H, S, D, elt):
    return layout.element_offset("k", page, head, slot, d, H, S, D, elt)


def test_k_offsets_by_hand():
    # e4m3 K, Hkv=2, S=16, D=64 (one 64-byte slice per row, NI=1): element (page 2, head 1, slot 13, d 37)
    #   block (2*2+1)*16*64 = 5120; token 13 = 4*3+1 (s=3, i=1); chunk 37//16 = 2 (q=2, k=0)
    #   chunk position ((3*1+0)*4+2)*4+1 = 57 -> 5120 + 57*16 + 37%16 = 6037
    assert _k(2, 1, 13, 37, 2, 16, 64, 1) == 6037
    # e4m3 K, Hkv=1, S=32, D=64: (page 1, head 0, slot 17, d 0) -> 2048 + sub-page 1 (1024) + chunk 1 (16)
    assert _k(1, 0, 17, 0, 1, 32, 64, 1) == 3088
    # bf16 K, Hkv=1, S=16, D=128 (8 elements a chunk, NI=4): (page 0, head 0, slot 5, d 100)
    #   token 5 (s=1, i=1); chunk 100//8 = 12 (q=3, k=0); position ((1*4+0)*4+3)*4+1 = 77 -> 77*8 + 4
    assert _k(0, 0, 5, 100, 1, 16, 128, 2) == 620
    # e4m3 K, D=128 (NI=2): the 32 bytes lane group q reads of token 4s+i start at 512s + 64q + 16i
    # (first half, k=0) and 256 bytes later (second half, k=1)
    for s_ in range(4):
        for q in range(4):
            for i in range(4):
                assert _k(0, 0, 4 * s_ + i, 32 * q, 1, 16, 128, 1) == 512 * s_ + 64 * q + 16 * i
                assert _k(0, 0, 4 * s_ + i, 32 * q + 16, 1, 16, 128, 1) == 512 * s_ + 256 + 64 * q + 16 * i


def test_v_and_latent_offsets_by_hand():
    # V element (page 2, head 1, slot 3, d 4), Hkv=2, S=4, Dv=5: ((2*2+1)*5+4)*4+3 = 119 (S=4 only here:
    # V blocks need no 16-token sub-pages)
    assert (2 * 2 + 1) * 4 * 5 + int(layout.v_block_offsets(4, 5)[3, 4]) == 119
    assert int(layout.v_block_offsets(4, 5)[1, 0]) == 1
    # latent (page 3, slot 5, d 7) of a 576-wide, 16-slot pool: (3*16 + 5)*576 + 7 = 30535
    assert layout.element_offset("latent", 3, 0, 5, 7, 1, 16, 576, 1) == 30535
    assert layout.element_offset("latent", 2, 0, 63, 575, 1, 64, 576, 1) == 3 * 64 * 576 - 1


@pytest.mark.parametrize("kind,S,D,elt", [("k", 16, 128, 1), ("k", 16, 128, 2), ("k", 64, 128, 1),
                                          ("k", 32, 576, 1), ("k", 16, 576, 2), ("k", 16, 64, 1),
                                          ("v", 16, 128, 1), ("v", 64, 128, 2), ("latent", 64, 576, 1)])
def test_block_offsets_are_a_bijection(kind, S, D, elt):
    off = layout.block_offsets(kind, S, D, elt)
    assert np.array_equal(np.sort(off.ravel()), np.arange(S * D))


@pytest.mark.parametrize("kind,elt", [("k", 1), ("k", 2), ("v", 1), ("v", 2), ("latent", 1)])
def test_to_and_from_device_round_trip(kind, elt):
    rng = np.random.Generator(np.random.PCG64(7))
    P, H, S, D = 3, 2, 32, 64
    dt = np.uint8 if elt == 1 else np.uint16
    pool = rng.integers(0, 2 ** (8 * elt), (P, H, S, D)).astype(dt)
    flat = layout.to_device(pool, kind, elt)
    assert flat.shape == (P * H * S * D,)
    assert np.array_equal(layout.from_device(flat, kind, pool.shape, elt), pool)
    # one element by hand: (page 2, head 1, slot 17, d 40) sits at its element offset
    assert flat[layout.element_offset(kind, 2, 1, 17, 40, H, S, D, elt)] == pool[2, 1, 17, 40]


def test_int4_layout_hand_worked():
    N, K = 32, 256                                   # K/128 = 2 groups, 2 output tiles
    q = np.zeros((N, K), dtype=np.int8)
    q[17, 130] = 5   # t=1, nn=1, g=1 -> tile 3; kk=2 -> j=0, qq=0, e=2 -> lane 1, nibble slot 1
    q[0, 37] = -3    # t=0, g=0; kk=37 -> j=1, qq=0, e=5 -> lane 0, slot 6 (dword 1, byte 3, low nibble)
    p = layout.pack_w4(q)
    assert p.size == N * K // 2
    want = np.full(p.size, 0x88, dtype=np.uint8)     # every nibble holds code + 8; zero codes are 8
    want[(3 * 64 + 1) * 16] = (5 + 8) << 4 | 8
    want[4 + 3] = 8 << 4 | (-3 + 8)
    assert np.array_equal(p, want)
    assert np.array_equal(layout.unpack_w4(p, N, K), q)


def test_fp8_weight_layout_and_scales_hand_worked():
    N, K = 32, 256
    c = np.zeros((N, K), dtype=np.uint8)
    c[17, 130] = 0x3A
    c[5, 255] = 0xC1  # t=0, nn=5, g=1 -> tile 1; kk=127 -> j=3, qq=3, e=7 -> lane 53, byte 31
    p = layout.pack_w8(c)
    want = np.zeros(N * K, dtype=np.uint8)
    want[(3 * 64 + 1) * 32 + 2] = 0x3A
    want[(1 * 64 + 53) * 32 + 31] = 0xC1
    assert np.array_equal(p, want)
    assert np.array_equal(layout.unpack_w8(p, N, K), c)
    s = np.arange(N * 2, dtype=np.uint16).reshape(N, 2)
    ps = layout.pack_scales(s)
    assert ps.shape == (2, 2, 16) and ps[1, 0, 3] == s[19, 0] and ps[0, 1, 15] == s[15, 1]
    assert np.array_equal(layout.unpack_scales(ps, N, K), s)


def test_weight_packing_round_trips_random_codes():
    rng = np.random.Generator(np.random.PCG64(8))
    N, K = 48, 384
    q = rng.integers(-8, 8, (N, K)).astype(np.int8)
    c = rng.integers(0, 256, (N, K)).astype(np.uint8)
    assert np.array_equal(layout.unpack_w4(layout.pack_w4(q), N, K), q)
    assert np.array_equal(layout.unpack_w8(layout.pack_w8(c), N, K), c)
    assert np.array_equal(np.sort(layout._w8_index(N, K).ravel()), np.arange(N * K))
