"""Adapter-aware batch former -- TEST INFRASTRUCTURE ONLY (the oracle).

Picks the requests of the next step from a waiting queue so that the batch
shares adapters.  Written from "m07 -- Multi-Adapter (LoRA) Serving":
* "6. Deep Dive A", "The adapter-aware scheduler": group the queue by adapter,
  take the biggest groups first and whole where possible, and stop admitting
  new adapters once the batch holds ``max_distinct`` of them and at least
  ``min_batch`` requests;
* same section, "The fairness cost, which must be stated": requests that have
  waited past a deadline are admitted first, whatever the grouping;
* "The Revision", R1: a few batch slots are reserved for the oldest requests
  whose adapter no other waiting request uses (the long tail), and the grouped
  fill gets the remaining adapter budget.
"12. Adapter Serving and Multi-Tenant Customization", "Batching across
adapters" groups base-only requests as a group of their own.

Readings where the pages leave a step open (each listed in the design notes):
* The queue is in arrival order, oldest first; "oldest" means earliest in it.
* Groups of equal size are taken in the order of their oldest request (a
  stable sort over groups met in queue order); inside a group, oldest first.
* Base-only requests (adapter < 0) form one group; admitting it adds no
  adapter to the count, and no base-only request takes a reserved tail slot.
* The minimum batch size is checked against the whole batch (urgent, tail and
  grouped requests), so the cap bounds the batch's distinct adapters
  whenever ``min_batch <= max_distinct``.
* The grouped fill's capacity is what the urgent and tail requests leave of
  ``max_batch``; its adapter budget is ``max_distinct`` less the tail's
  adapters.  The reserved slots are part of that budget ("4 of 32"), so the
  tail takes at most ``min(reserved_tail, max_distinct)``.  Urgent requests
  are outside the budget (the override's point).
* Group sizes are counted over the requests the step still considers: the
  tail test over the queue without the urgent requests, the fill's order over
  what remains after the tail.

Nothing here is shared with the library's native former.
"""
from __future__ import annotations


def _rank_groups(adapters, taken):
    """The requests not yet taken, grouped by adapter (every base-only request
    in the one group keyed -1), as records [size, oldest position, key,
    members oldest first], ranked biggest first and, among equal sizes, by
    their oldest member."""
    members = {}
    for i, a in enumerate(adapters):
        if not taken[i]:
            members.setdefault(a if a >= 0 else -1, []).append(i)
    records = [[len(m), m[0], key, m] for key, m in members.items()]
    records.sort(key=lambda r: (-r[0], r[1]))
    return records


def form_batch(adapters, max_batch, max_distinct, min_batch=0, reserved_tail=0,
               waited_ms=None, max_wait_ms=None):
    """Queue positions of the chosen requests, in batch order: urgent ones,
    then the reserved tail, then the grouped fill.

    adapters: adapter id of each waiting request, oldest first (< 0: base only).
    waited_ms / max_wait_ms: optional ages and deadline for the override.
    """
    n = len(adapters)
    batch = []
    taken = [False] * n

    def take(i):
        batch.append(i)
        taken[i] = True

    # 1. Age override: every request past the deadline, oldest first.
    if waited_ms is not None and max_wait_ms is not None:
        for i in range(n):
            if len(batch) >= max_batch:
                break
            if waited_ms[i] > max_wait_ms:
                take(i)

    # 2. Reserved tail: the oldest requests whose adapter has no other request
    #    among those still waiting.
    count = {}
    for i in range(n):
        if not taken[i] and adapters[i] >= 0:
            count[adapters[i]] = count.get(adapters[i], 0) + 1
    tail = 0
    for i in range(n):
        if tail >= min(reserved_tail, max_distinct) or len(batch) >= max_batch:
            break
        if not taken[i] and adapters[i] >= 0 and count[adapters[i]] == 1:
            take(i)
            tail += 1

    # 3. Grouped fill.  Every group is ranked once; then each group in rank
    #    order is admitted whole (cut only by the batch's capacity) while
    #    there is room and either the fill still has adapter budget or the
    #    batch is below its minimum size.  The base-only group spends no
    #    budget.
    adapter_budget = max_distinct - tail
    adapters_admitted = 0
    for size, oldest, key, members in _rank_groups(adapters, taken):
        room = max_batch - len(batch)
        if room <= 0:
            break
        budget_spent = adapters_admitted >= adapter_budget
        big_enough = len(batch) >= min_batch
        if budget_spent and big_enough:
            break
        for i in members[:min(size, room)]:
            take(i)
        adapters_admitted += 1 if key >= 0 else 0
    return batch


def distinct_adapters(adapters, batch):
    """Number of distinct adapters (>= 0) among the chosen requests."""
    return len({adapters[i] for i in batch if adapters[i] >= 0})
