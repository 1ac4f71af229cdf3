"""The library's host-side page allocator (kv_page_alloc_*, no GPU needed) against the oracle's, on
seeded random operation sequences: identical pages, tags, errors and free counts."""
import ctypes as C

import numpy as np
import pytest

from oracle.paged import PageAllocator as OracleAllocator


@pytest.fixture(scope="module")
def kv():
    import fp8_paged_kv_append_amd as kv
    kv.lib()
    return kv


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_same_pages_tags_and_errors_as_the_oracle(kv, seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.integers(1, 64))
    init = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
    init[0] = 0xFFFFFFFF
    lib_a = kv.PageAllocator(P, initial_tags=init)
    ora_a = OracleAllocator(P, initial_tags=init)
    held = []
    for _ in range(600):
        op = rng.random()
        if op < 0.4 and held:
            owner = held.pop(int(rng.integers(len(held))))
            if owner and rng.random() < 0.1:            # a bad free: add a duplicate or a stray id
                bad = owner + [owner[0]] if rng.random() < 0.5 else owner + [P + 3]
                assert ora_a.free(bad) == OracleAllocator.INVALID
                with pytest.raises(kv.KvFp8Error) as e:
                    lib_a.free(bad)
                assert e.value.status == -7
            assert ora_a.free(owner) is None
            lib_a.free(owner)
        else:
            n = int(rng.integers(0, 12))
            r = ora_a.alloc(n)
            if r == OracleAllocator.NOSPACE:
                with pytest.raises(kv.KvFp8Error) as e:
                    lib_a.alloc(n)
                assert e.value.status == -8
            else:
                pages, tags = lib_a.alloc(n)
                assert np.array_equal(pages, r[0]) and np.array_equal(tags, r[1])
                held.append(pages.tolist())
        assert lib_a.free_count == ora_a.free_count
    assert np.array_equal(lib_a.tags(), ora_a.tags)


def test_abi_validation(kv):
    lib = kv.lib()
    assert lib.kv_page_alloc_state_bytes(0) == 0
    n = lib.kv_page_alloc_state_bytes(10)
    buf = np.zeros(n // 4 + 1, dtype=np.uint32)
    assert lib.kv_page_alloc_free_count(buf.ctypes.data) == -1                  # not initialised
    assert lib.kv_page_alloc_init(None, n, 10, None) == -1
    assert lib.kv_page_alloc_init(buf.ctypes.data, n - 1, 10, None) == -4       # too small
    assert lib.kv_page_alloc_init(buf.ctypes.data, n, 0, None) == -2
    assert lib.kv_page_alloc_init(buf.ctypes.data + 2, n, 10, None) == -5       # misaligned
    assert lib.kv_page_alloc_init(buf.ctypes.data, n, 10, None) == 0
    pages = np.zeros(4, dtype=np.int32)
    assert lib.kv_page_alloc(buf.ctypes.data, -1, pages.ctypes.data, None) == -2
    assert lib.kv_page_alloc(buf.ctypes.data, 11, pages.ctypes.data, None) == -8
    assert lib.kv_page_alloc(buf.ctypes.data, 4, pages.ctypes.data, None) == 0   # tags out may be NULL
    assert pages.tolist() == [0, 1, 2, 3]
    assert lib.kv_page_free(buf.ctypes.data, None, 1) == -1
    assert lib.kv_page_free(buf.ctypes.data, pages.ctypes.data, 4) == 0
    assert lib.kv_page_alloc_free_count(buf.ctypes.data) == 10
