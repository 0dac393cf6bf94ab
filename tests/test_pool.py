"""The block pool and the fork's host logic (no GPU: forks at block
boundaries copy nothing).  HPD-Parsing wiki, inference scheduling: a branch
shares its parent's KV through a fork pointer, zero copy, and the shared
blocks are released by reference count."""
import numpy as np
import pytest

from decode_focal_layer_amd import kvsel
from oracle import oracle as O


def test_alloc_retain_release_and_free_list():
    p = kvsel.BlockPool(8)
    assert p.free_count() == 8
    a = p.alloc(3)
    assert len(set(a.tolist())) == 3 and all(p.refcount(b) == 1 for b in a)
    assert p.free_count() == 5
    p.retain(a[:2])
    assert [p.refcount(b) for b in a] == [2, 2, 1]
    p.release(a)                       # 2 -> 1, 2 -> 1, 1 -> 0 (freed)
    assert [p.refcount(b) for b in a] == [1, 1, 0] and p.free_count() == 6
    p.release(a[:2])
    assert p.free_count() == 8 and all(p.refcount(b) == 0 for b in range(8))
    assert p.refcount(8) == -1 and p.refcount(-1) == -1


def test_rejections_change_nothing():
    p = kvsel.BlockPool(4)
    a = p.alloc(2)
    with pytest.raises(kvsel.KvselError) as e:
        p.alloc(3)                     # only 2 free
    assert e.value.status == -2        # KVSEL_ENOSPC
    with pytest.raises(kvsel.KvselError) as e:
        p.release([a[0], a[0]])        # one reference, released twice
    assert e.value.status == -1        # KVSEL_EINVAL
    with pytest.raises(kvsel.KvselError):
        p.retain([3 if 3 not in a else 2])   # a free block
    with pytest.raises(kvsel.KvselError):
        p.release([9])
    assert p.free_count() == 2 and p.refcount(a[0]) == 1 and p.refcount(a[1]) == 1
    with pytest.raises(ValueError):
        kvsel.BlockPool(0)


@pytest.mark.parametrize("L", [0, 16, 48, 80])
def test_fork_at_block_boundary_shares_every_block(L):
    p = kvsel.BlockPool(16)
    parent = np.full(6, -1, dtype=np.int32)
    blocks = p.alloc(5)
    parent[:5] = blocks
    child = p.fork(parent, L)
    np.testing.assert_array_equal(child, O.fork_child_table(parent, L, new_block=-7))
    n = L // 16
    assert [p.refcount(b) for b in blocks] == [2] * n + [1] * (5 - n)
    assert p.free_count() == 11
    # the parent finishes first: the child still holds the shared blocks
    p.release(blocks)
    assert [p.refcount(b) for b in blocks] == [1] * n + [0] * (5 - n)
    p.release(child[:n])
    assert p.free_count() == 16


def test_fork_of_a_partial_block_needs_the_pools_and_a_free_block():
    p = kvsel.BlockPool(4)
    parent = np.full(2, -1, dtype=np.int32)
    parent[:2] = p.alloc(2)
    with pytest.raises(kvsel.KvselError):
        p.fork(parent, 20)             # rows 16..19 sit in a partly filled block: no pools given
    assert p.refcount(parent[0]) == 1 and p.free_count() == 2
    with pytest.raises(kvsel.KvselError):
        p.fork(parent, 33)             # beyond the parent's table
    with pytest.raises(kvsel.KvselError):
        p.fork(np.array([3, -1], dtype=np.int32), 16)   # a block the pool has not handed out
