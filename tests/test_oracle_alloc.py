"""Pins of the oracle's page allocator (agentlenshq summary, section "KV Cache 完整性检查"; xujun.org
note, section "一个不能出错的共享缓存": a page's tag changes when the page is reallocated)."""
import numpy as np

from oracle.paged import PageAllocator


def test_fresh_allocator_hands_out_pages_in_order_with_bumped_tags():
    a = PageAllocator(6)
    pages, tags = a.alloc(4)
    assert pages.tolist() == [0, 1, 2, 3] and tags.tolist() == [1, 1, 1, 1]
    assert a.free_count == 2 and a.tags.tolist() == [1, 1, 1, 1, 0, 0]


def test_reallocation_changes_the_tag_and_reuses_last_freed_first():
    a = PageAllocator(4)
    p1, t1 = a.alloc(3)
    assert a.free([2, 0]) is None                  # freeing leaves the tags alone
    assert a.tags.tolist() == [1, 1, 1, 0]
    p2, t2 = a.alloc(2)                            # stack: last freed (0) first
    assert p2.tolist() == [0, 2] and t2.tolist() == [2, 2]
    # an old holder of page 0 expects tag 1; the page now carries 2
    assert int(t1[0]) != int(a.tags[0])


def test_nospace_and_invalid_frees_change_nothing():
    a = PageAllocator(3)
    a.alloc(2)
    before = (a.tags.copy(), list(a.free_list), list(a.in_use))
    assert a.alloc(2) == PageAllocator.NOSPACE
    assert a.free([1, 1]) == PageAllocator.INVALID       # listed twice
    assert a.free([2]) == PageAllocator.INVALID          # not in use
    assert a.free([5]) == PageAllocator.INVALID          # out of range
    assert a.free([0, -1]) == PageAllocator.INVALID
    assert (a.tags.tolist(), a.free_list, a.in_use) == (before[0].tolist(), before[1], before[2])


def test_tag_wraps_mod_2_32():
    a = PageAllocator(1, initial_tags=[0xFFFFFFFF])
    _, t = a.alloc(1)
    assert int(t[0]) == 0


def test_random_sequences_keep_the_invariants():
    """Against a model with no stack: a page is never held twice, every page is free or held, and each
    tag equals its initial value plus the number of times the page was handed out (mod 2**32)."""
    rng = np.random.default_rng(5)
    P = 40
    init = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
    a = PageAllocator(P, initial_tags=init)
    held = []                      # pages currently held, per owner
    handed = np.zeros(P, dtype=np.int64)
    for _ in range(2000):
        if held and rng.random() < 0.45:
            owner = held.pop(int(rng.integers(len(held))))
            assert a.free(owner) is None
        else:
            n = int(rng.integers(0, 9))
            r = a.alloc(n)
            if r == PageAllocator.NOSPACE:
                assert n > a.free_count
                continue
            pages, tags = r
            flat = [p for o in held for p in o]
            assert not set(pages.tolist()) & set(flat) and len(set(pages.tolist())) == n
            handed[pages] += 1
            assert np.array_equal(tags, ((init[pages].astype(np.int64) + handed[pages]) % 2 ** 32).astype(np.uint32))
            held.append(pages.tolist())
        flat = [p for o in held for p in o]
        assert a.free_count + len(flat) == P and sorted(flat + a.free_list) == list(range(P))
