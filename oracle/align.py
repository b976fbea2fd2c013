"""Oracle expert sort / block alignment (test infrastructure only).

"vLLM PR 50949 review", ``moe_fp8.cpp`` listing: the fused expert kernel walks
expert blocks ``mb``; ``expert_ids[mb]`` names the expert, ``offsets[mb]`` is
the first row of the block in the compact intermediate buffer, the block holds
``offsets[mb+1] - offsets[mb]`` real rows (zero for an empty block, which is
skipped), and ``sorted_ids[mb * BLOCK_M + m]`` is a flat routed-row id whose
token is ``id / topk``.  The producer of these arrays is not on the pages; the
canonical layout both sides of the parity tests use is:

* routed rows are flat ids ``r = t * topk + k`` for ``R = M * topk`` rows;
* rows are grouped by expert in ascending expert id, and inside one expert
  they keep ascending ``r`` (a stable sort);
* each expert's rows are cut into blocks of ``block_m`` rows (the last block of
  an expert may be partial); experts with no rows get no block;
* ``offsets[mb]`` is the running row count before block ``mb``;
* slots past a block's real rows hold the pad value ``R``;
* blocks past ``num_blocks`` have ``expert_ids = -1`` and ``offsets = R``
  (so they are empty).

The arrays are sized for the worst case ``max_blocks(M, topk, E, block_m) =
ceil(R / block_m) + min(E, R)`` so no host synchronisation is needed to size
them.
"""

import numpy as np


def max_blocks(M: int, topk: int, E: int, block_m: int) -> int:
    R = M * topk
    return -(-R // block_m) + min(E, R)


def moe_align(topk_ids: np.ndarray, E: int, block_m: int):
    """int [M, topk] expert ids -> (sorted_ids, expert_ids, offsets, num_blocks)."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    M = np.asarray(topk_ids).shape[0]
    topk = np.asarray(topk_ids).shape[1] if np.asarray(topk_ids).ndim == 2 else 1
    R = ids.size
    if np.any(ids < 0) or np.any(ids >= E):
        raise ValueError("expert id out of range")
    nb_max = max_blocks(M, topk, E, block_m)
    sorted_ids = np.full(nb_max * block_m, R, dtype=np.int32)
    expert_ids = np.full(nb_max, -1, dtype=np.int32)
    offsets = np.full(nb_max + 1, R, dtype=np.int32)
    mb = 0
    row = 0
    for e in range(E):
        rows_e = np.nonzero(ids == e)[0]  # ascending flat ids
        for b0 in range(0, rows_e.size, block_m):
            chunk = rows_e[b0:b0 + block_m]
            expert_ids[mb] = e
            offsets[mb] = row
            sorted_ids[mb * block_m: mb * block_m + chunk.size] = chunk
            row += chunk.size
            mb += 1
    offsets[mb:] = R
    return sorted_ids, expert_ids, offsets, mb
