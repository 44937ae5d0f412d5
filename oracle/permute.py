"""Expert histogram and expert-sorted token permutation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages do not describe this step; it follows from the layer itself: the
routed experts are almost all of the weight bytes (page
"NeuroSenko/Step-5-Preview-Int4-g128", "Recipe": 96.7 % of the model), so the
assignments of one expert are gathered together and its weights stream once.

Definition (slot s = t*K + k is the k-th choice of token t):
* counts[e]          number of slots routed to expert e;
* expert_offsets     exclusive prefix sum of counts, length E+1;
* padded_offsets     exclusive prefix sum of counts rounded up to tile_m;
* sorted_slots       for each expert in ascending order, its slots in
                     ascending slot order (a stable sort by expert), each
                     segment padded with -1 up to its padded length; only
                     entries [0, padded_offsets[E]) are defined;
* slot_to_row[s]     the position of slot s in sorted_slots;
* tile_expert[i]     the expert owning rows [i*tile_m, (i+1)*tile_m);
* num_tiles          padded_offsets[E] / tile_m;
* active_experts     the experts with counts > 0, ascending; num_active.
"""
import numpy as np


def permute(ids, E, tile_m):
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.ravel()
    n = flat.size
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)[:E]
    expert_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    padded = -(-counts // tile_m) * tile_m
    padded_offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    total = int(padded_offsets[-1])
    sorted_slots = np.full(total, -1, dtype=np.int32)
    slot_to_row = np.empty(n, dtype=np.int32)
    for e in range(E):
        seg = order[expert_offsets[e]:expert_offsets[e + 1]]
        rows = padded_offsets[e] + np.arange(seg.size)
        sorted_slots[rows] = seg
        slot_to_row[seg] = rows
    num_tiles = total // tile_m
    tile_expert = np.empty(num_tiles, dtype=np.int32)
    for e in range(E):
        tile_expert[padded_offsets[e] // tile_m: padded_offsets[e + 1] // tile_m] = e
    active = np.nonzero(counts)[0].astype(np.int32)
    return dict(counts=counts.astype(np.int32), expert_offsets=expert_offsets,
                padded_offsets=padded_offsets, sorted_slots=sorted_slots,
                slot_to_row=slot_to_row, tile_expert=tile_expert,
                num_tiles=num_tiles, active_experts=active,
                num_active=int(active.size))


def max_rows(T, K, E, tile_m):
    """Upper bound on padded_offsets[E] for any routing of T tokens."""
    n = T * K
    return n + min(E, n) * (tile_m - 1)


def max_tiles(T, K, E, tile_m):
    return max_rows(T, K, E, tile_m) // tile_m
