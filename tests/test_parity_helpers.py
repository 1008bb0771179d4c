"""The list comparison of the parity tests (vectorised for whole 1080p views) on
hand-made lists: exact lists pass, a swapped or foreign entry fails, a culling
difference passes only inside the 1e-3 band around the threshold (and is counted)."""
import numpy as np

import parity as P


def _fixture():
    # three tiles: pre-cull lists with cull quantities q (kept iff q >= 1)
    pre = [np.array([4, 1, 7], np.int32), np.array([], np.int32), np.array([2, 9, 3, 5], np.int32)]
    q = [np.array([2.0, 0.5, 1.0]), np.array([]), np.array([1.0005, 3.0, 0.2, 7.0])]
    off = np.concatenate([[0], np.cumsum([len(a) for a in pre])]).astype(np.int64)
    ora = {"lists_pre": (off, np.concatenate(pre), np.concatenate(q))}
    return pre, q, ora


def _gpu(lists, tiles_total=3, shuffle_tiles=False):
    """A GPU-like (ranges, ids) pair holding ``lists`` per tile, tile-major."""
    order = list(range(tiles_total))[::-1] if shuffle_tiles else list(range(tiles_total))
    ids, ranges, pos = [], np.zeros((tiles_total, 2), np.int32), 0
    for t in order:
        ranges[t] = (pos, pos + len(lists[t]))
        ids.extend(lists[t])
        pos += len(lists[t])
    return {"ranges": ranges, "ids": np.array(ids, np.int32)}


def test_exact_lists_pass():
    pre, q, ora = _fixture()
    tiles = np.arange(3)
    kept = [a[b >= 1.0] for a, b in zip(pre, q)]
    for shuffle in (False, True):
        r = P.compare_lists(None, _gpu(kept, shuffle_tiles=shuffle), ora, tiles, cull=True)
        assert r["list_mismatch"] == 0 and r["cull_exempt"] == 0
        r = P.compare_lists(None, _gpu(pre, shuffle_tiles=shuffle), ora, tiles, cull=False)
        assert r["list_mismatch"] == 0


def test_wrong_lists_fail():
    pre, q, ora = _fixture()
    tiles = np.arange(3)
    kept = [a[b >= 1.0] for a, b in zip(pre, q)]
    swapped = [kept[0][::-1], kept[1], kept[2]]
    assert P.compare_lists(None, _gpu(swapped), ora, tiles, cull=True)["list_mismatch"] == 1
    foreign = [kept[0], np.array([8], np.int32), kept[2]]
    assert P.compare_lists(None, _gpu(foreign), ora, tiles, cull=True)["list_mismatch"] == 1
    far_culled = [kept[0][:1], kept[1], kept[2]]  # id 7 (q = 1.0) dropped: q is on the band edge
    r = P.compare_lists(None, _gpu(far_culled), ora, tiles, cull=True)
    assert r["list_mismatch"] == 0 and r["cull_exempt"] == 1
    dropped_far = [kept[0], kept[1], np.array([2, 5], np.int32)]  # id 9 (q = 3) dropped: wrong
    assert P.compare_lists(None, _gpu(dropped_far), ora, tiles, cull=True)["list_mismatch"] == 1
    kept_far = [np.array([4, 1, 7], np.int32), kept[1], kept[2]]  # id 1 (q = 0.5) kept: wrong
    assert P.compare_lists(None, _gpu(kept_far), ora, tiles, cull=True)["list_mismatch"] == 1
    pre_swapped = [pre[0], pre[1], pre[2][[1, 0, 2, 3]]]
    assert P.compare_lists(None, _gpu(pre_swapped), ora, tiles, cull=False)["list_mismatch"] == 1


def test_tile_subset():
    pre, q, ora = _fixture()
    # the oracle's lists of a sample (tiles 0 and 2 of 3); the GPU holds all three
    sub = {"lists_pre": (np.array([0, 3, 7]), np.concatenate([pre[0], pre[2]]), np.concatenate([q[0], q[2]]))}
    kept = [a[b >= 1.0] for a, b in zip(pre, q)]
    g = _gpu([kept[0], np.array([11, 12], np.int32), kept[2]])
    assert P.compare_lists(None, g, sub, np.array([0, 2]), cull=True)["list_mismatch"] == 0
    g = _gpu([kept[0], np.array([11, 12], np.int32), kept[2][:-1]])
    assert P.compare_lists(None, g, sub, np.array([0, 2]), cull=True)["list_mismatch"] == 1
