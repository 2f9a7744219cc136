"""Token-to-expert permutation lists (oracle; test-only).

Not described on the pages; it is the bookkeeping any grouped expert
computation needs once routing is known.  Definition used:

  pair p = t*k + j is the j-th choice of token t, expert e = ids[t, j];
  counts[e]      number of pairs routed to e;
  offsets        exclusive prefix sum of counts, offsets[0] = 0,
                 offsets[E] = T*k;
  sorted_pairs   for each expert, the pairs routed to it in ascending p,
                 expert segments laid out in expert order;
  pair_to_row    inverse: sorted_pairs[pair_to_row[p]] == p.

Built by walking the pairs in order and appending each to its expert's list.

With drop_invalid=True (the library's rule for bad input, a reading: the
pages never route outside the experts) a pair whose id is outside [0, E) is
left out: it is not counted, has no row (pair_to_row = -1) and offsets[E]
counts only the kept pairs; sorted_pairs holds offsets[E] entries followed
by -1.
"""

import numpy as np


def permute(ids, E, drop_invalid=False):
    """ids int[T, k] -> dict(counts, offsets, sorted_pairs, pair_to_row), all int32."""
    ids = np.asarray(ids)
    if ids.ndim != 2:
        raise ValueError("ids must be [T, k]")
    T, k = ids.shape
    R = T * k
    lists = [[] for _ in range(E)]
    flat = ids.reshape(-1).tolist()
    for p in range(R):
        e = flat[p]
        if not 0 <= e < E:
            if drop_invalid:
                continue
            raise ValueError("expert id out of range")
        lists[e].append(p)
    counts = np.array([len(lst) for lst in lists], dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    running = 0
    for e in range(E):
        offsets[e] = running
        running += len(lists[e])
    offsets[E] = running
    sorted_pairs = np.full(R, -1, dtype=np.int32)
    pair_to_row = np.full(R, -1, dtype=np.int32)
    row = 0
    for e in range(E):
        for p in lists[e]:
            sorted_pairs[row] = p
            pair_to_row[p] = row
            row += 1
    return {"counts": counts, "offsets": offsets,
            "sorted_pairs": sorted_pairs, "pair_to_row": pair_to_row}
