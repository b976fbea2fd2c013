"""Pins for the oracle expert sort / block alignment: a second, differently
written construction (Python's stable ``sorted`` on (expert, flat id) keys)
on small random routings, and the structural invariants of the layout."""

import numpy as np
import pytest

from oracle.align import moe_align, max_blocks


def _by_sorting(ids2d, E, block_m):
    flat = [int(v) for v in np.asarray(ids2d).reshape(-1)]
    R = len(flat)
    order = sorted(range(R), key=lambda r: (flat[r], r))
    blocks = []  # (expert, [rows])
    for r in order:
        e = flat[r]
        if blocks and blocks[-1][0] == e and len(blocks[-1][1]) < block_m:
            blocks[-1][1].append(r)
        else:
            blocks.append((e, [r]))
    return blocks


@pytest.mark.parametrize("seed", range(40))
def test_matches_sorted_construction(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(0, 40))
    topk = int(rng.integers(1, 5))
    E = int(rng.integers(max(topk, 1), 12))
    block_m = int(rng.choice([1, 2, 3, 4, 8, 16]))
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]) if M else np.zeros((0, topk), int)
    sorted_ids, expert_ids, offsets, nb = moe_align(ids, E, block_m)
    ref = _by_sorting(ids, E, block_m)
    R = M * topk
    assert nb == len(ref)
    assert sorted_ids.size == max_blocks(M, topk, E, block_m) * block_m
    row = 0
    for mb, (e, rows) in enumerate(ref):
        assert expert_ids[mb] == e
        assert offsets[mb] == row
        got = sorted_ids[mb * block_m:(mb + 1) * block_m]
        assert list(got[:len(rows)]) == rows
        assert np.all(got[len(rows):] == R)
        row += len(rows)
    assert np.all(expert_ids[nb:] == -1)
    assert np.all(offsets[nb:] == R)
    assert np.all(sorted_ids[nb * block_m:] == R)


def test_invariants_on_skewed_routing():
    rng = np.random.default_rng(99)
    M, topk, E, block_m = 500, 8, 64, 16
    p = np.arange(1, E + 1) ** -1.1
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=topk, replace=False, p=p) for _ in range(M)])
    sorted_ids, expert_ids, offsets, nb = moe_align(ids, E, block_m)
    R = M * topk
    m_size = np.diff(offsets)[:nb]
    assert m_size.sum() == R and np.all(m_size >= 1) and np.all(m_size <= block_m)
    real = np.concatenate([sorted_ids[mb * block_m: mb * block_m + m_size[mb]] for mb in range(nb)])
    assert np.array_equal(np.sort(real), np.arange(R))  # every row exactly once
    assert np.all(np.diff(expert_ids[:nb]) >= 0)  # blocks are expert-sorted
    flat = ids.reshape(-1)
    for mb in range(nb):
        rows = sorted_ids[mb * block_m: mb * block_m + m_size[mb]]
        assert np.all(flat[rows] == expert_ids[mb])
    # only the last block of an expert may be partial
    for mb in range(nb - 1):
        if expert_ids[mb] == expert_ids[mb + 1]:
            assert m_size[mb] == block_m


def test_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        moe_align(np.array([[0, 5]]), 5, 4)
