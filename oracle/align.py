"""Alignment oracle: the plain definition of the deterministic token sort.

Test infrastructure only (see the package docstring).

What is computed, restated from the pages:

* nbxtensor ``moe_align.py``, module docstring: the tables are sized on the
  shape-derived worst case ``min(n*BS, n + E*(BS-1))`` rounded up to a whole
  number of BS blocks; the real padded total exists only as a device scalar;
  the within-expert order is the one a stable host sort of the slots by expert
  gives (each slot's rank is the number of earlier slots routed to the same
  expert), with no atomics.
* ``moe_align.py``, stage-1 kernel docstring: per-expert counts, counts padded
  up to a multiple of BS, the exclusive prefix of the padded counts, and the
  total.
* ``moe_align.py``, stage-2 kernel docstring: every table position not holding
  a slot keeps the sentinel ``n``; each BS block is labelled with the expert
  whose padded segment contains the block's first position, or -1 past the
  total.
* ``moe_align.py``, stage-3 kernel docstring and body comment: a slot whose id
  lies outside ``[0, E)`` is skipped (the host scatter's bounds check); a slot
  ``i`` lands at ``offset[id] + rank(i)``; the table stores the flat slot index
  ``i = token*top_k + k``.
* metrale ``fp8_moe_grouped.rs``, doc of ``moe_fp8_grouped_sort`` and of
  ``Fp8GroupedSortOut``: the sort also returns ``token_to_perm`` (slot ->
  sorted position) and the active experts in ascending order with their count;
  doc of ``fp8_grouped_active_cap``: the active list is sized
  ``min(n, E)``, independent of the routing.

Readings where the pages leave a choice (listed in the design notes): tables
are int32-valued; ``expert_offsets`` has ``E+1`` entries with the total last;
``token_to_perm`` is -1 for a skipped slot; ``active_experts`` is filled with -1
past the count.
"""

from __future__ import annotations

import numpy as np


def max_total(n: int, E: int, BS: int) -> int:
    """Worst-case table length: ``min(n*BS, n + E*(BS-1))`` rounded up to BS."""
    bound = min(n * BS, n + E * (BS - 1))
    return -(-bound // BS) * BS


def active_cap(n: int, E: int) -> int:
    """At most ``min(n, E)`` distinct experts can receive a slot."""
    return min(n, E)


def align(topk_ids, E: int, BS: int) -> dict:
    """Build every alignment table from the router's ``topk_ids`` ([M, top_k] or flat).

    Returns a dict of int64 numpy arrays: ``expert_counts[E]``,
    ``expert_offsets[E+1]``, ``total`` (scalar), ``sorted_token_ids[max_total]``,
    ``block_expert_ids[max_total/BS]``, ``token_to_perm[n]``,
    ``active_experts[cap]``, ``active_count`` (scalar).
    """
    ids = np.asarray(topk_ids).astype(np.int64).reshape(-1)  # flat slot i = t*top_k + k
    n = int(ids.size)
    valid = (ids >= 0) & (ids < E)

    # per-expert counts of in-range slots
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(valid & (ids == e)))

    # pad each count up to a multiple of BS; exclusive prefix; total
    padded = (counts + BS - 1) // BS * BS
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + padded[e]
    total = int(offsets[E])

    # sentinel-filled worst-case table, then each expert's slots in ascending
    # flat index (the stable host sort order)
    mt = max_total(n, E, BS)
    sorted_ids = np.full(mt, n, dtype=np.int64)
    token_to_perm = np.full(n, -1, dtype=np.int64)
    for e in range(E):
        slots = np.flatnonzero(valid & (ids == e))
        for r, i in enumerate(slots):
            pos = offsets[e] + r
            sorted_ids[pos] = i
            token_to_perm[i] = pos

    # expert owning each BS block; -1 for blocks at or past the total
    block_expert = np.full(mt // BS, -1, dtype=np.int64)
    for b in range(mt // BS):
        start = b * BS
        for e in range(E):
            if offsets[e] <= start < offsets[e + 1]:
                block_expert[b] = e
                break

    # ascending active experts, padded with -1 up to the cap
    cap = active_cap(n, E)
    active = [e for e in range(E) if counts[e] > 0]
    active_experts = np.full(cap, -1, dtype=np.int64)
    active_experts[: len(active)] = active

    return {
        "expert_counts": counts,
        "expert_offsets": offsets,
        "total": total,
        "sorted_token_ids": sorted_ids,
        "block_expert_ids": block_expert,
        "token_to_perm": token_to_perm,
        "active_experts": active_experts,
        "active_count": len(active),
        "max_total": mt,
        "cap": cap,
        "n": n,
    }
