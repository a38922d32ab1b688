"""CPU oracle of the two steps around the verify attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg may import
this module. The HIP library never calls it and shares no code with it.

1. build_tree_mask: draft trees (parent pointers) -> the raw custom_mask and mask_indptr that
   the verify attention reads. Layout from "The Custom sm_120 Verify Kernel", section "The
   Debugging Gauntlet" (bug 2: a request's mask rows are prefix + q_len bytes, draft columns
   after the prefix columns); the visibility rule (every prefix column, and a draft column when
   it is the row's own node or one of its ancestors) is the usual tree-attention rule the pages
   rely on for draft-tree verification ("From Capture Safety to MoE Ceiling", section "The
   Architecture of Capture Safety": raw custom_mask with mask_indptr offsets). The pages time
   this step on the host; they print no mask.
2. compact_kv: the relocation step the pages designed and deferred ("From Capture Safety to
   MoE Ceiling", section "Tier 0 Defrag: The Art of Knowing When to Stop"; "The Art of Knowing
   When to Stop: Deferring Tier 1 Defrag", section "The Decision: Why Tier 1 Defrag Gets
   Deferred"): copy each request's prefix rows into a contiguous run of slots and rewrite
   its indices.

Readings where the pages are silent (listed with the other readings of the pages):
 - parents[b*q_len + i] is the index of draft token i's parent inside request b, -1 for a root.
   A valid parent precedes its child (parents[i] in [-1, i)); several roots are allowed.
   An entry outside [-1, i) is reported and read as -1.
 - A request's prefix length is max(0, kv_indptr[b+1] - kv_indptr[b]); mask_indptr is the
   exclusive running sum of q_len * (P_b + q_len), starting at 0.
 - Compaction moves the whole 576-wide row; destination slots are dst_start[b] + j for the
   j-th prefix token of request b. A request whose destination run leaves [0, N) is reported
   and left as it is (rows not moved, indices unchanged); a source slot outside [0, N) is
   reported, that row is not moved and keeps its index.

Pins (tests/test_tree_kv_oracle.py): the hand-listed 9-node tree of tests/golden, chain trees
against numpy's lower triangle, star trees, the reflexive-transitive closure of the parent
relation computed by boolean matrix products (a second route to the same set), row sums equal
to prefix + depth + 1, and for compaction the gather identity pool'[new] == pool[old] with
every other row untouched.
"""
from __future__ import annotations

import numpy as np

TREE_BAD_PARENT = 1
TREE_CAPACITY = 2
COMPACT_BAD_DST = 1
COMPACT_BAD_SRC = 2
INT32_MAX = 2**31 - 1


def prefix_lengths(kv_indptr, B):
    ip = np.asarray(kv_indptr, np.int64)
    return [max(0, int(ip[b + 1] - ip[b])) for b in range(B)]


def build_tree_mask(parents, kv_indptr, B: int, q_len: int, capacity: int | None = None):
    """Returns (custom_mask uint8 [capacity or total], mask_indptr int32 [B+1], status int).

    Requests whose mask does not fit the capacity (or past 2^31 - 1 bytes) are not written and
    their mask_indptr entries are clamped to the limit, as the device builder does; bytes not
    written are 0 here (the device leaves them as they were).
    """
    par = np.asarray(parents, np.int64).reshape(B, q_len)
    P = prefix_lengths(kv_indptr, B)
    status = 0
    sizes = [q_len * (P[b] + q_len) for b in range(B)]
    total = sum(sizes)
    limit = INT32_MAX if capacity is None else min(int(capacity), INT32_MAX)
    if total > limit:
        status |= TREE_CAPACITY
    mask = np.zeros(total if capacity is None else int(capacity), np.uint8)
    indptr = np.zeros(B + 1, np.int64)
    for b in range(B):
        indptr[b + 1] = indptr[b] + sizes[b]
    clamped = np.minimum(indptr, limit).astype(np.int32)
    for b in range(B):
        # the parent of node i, with an entry that does not precede i read as a root
        p = []
        for i in range(q_len):
            v = int(par[b, i])
            if not (-1 <= v < i):
                status |= TREE_BAD_PARENT
                v = -1
            p.append(v)
        if indptr[b + 1] > limit:
            continue
        L = P[b] + q_len
        base = int(indptr[b])
        for i in range(q_len):
            row = mask[base + i * L: base + (i + 1) * L]
            row[:P[b]] = 1
            j = i
            while j >= 0:          # the node itself, then each ancestor up to its root
                row[P[b] + j] = 1
                j = p[j]
    return mask, clamped, status


def compact_kv(pool, kv_indptr, kv_indices, dst_start, B: int):
    """Returns (new pool, new kv_indices, status). pool is [N, 576] (any dtype); not modified."""
    pool = np.asarray(pool)
    N = pool.shape[0]
    ip = np.asarray(kv_indptr, np.int64)
    old = np.asarray(kv_indices, np.int64)
    new_pool = pool.copy()
    new_idx = old.astype(np.int32).copy()
    status = 0
    P = prefix_lengths(kv_indptr, B)
    for b in range(B):
        d0 = int(dst_start[b])
        if P[b] > 0 and (d0 < 0 or d0 + P[b] > N):
            status |= COMPACT_BAD_DST
            continue
        for j in range(P[b]):
            t = int(ip[b]) + j
            src = int(old[t])
            if not (0 <= src < N):
                status |= COMPACT_BAD_SRC
                continue
            new_pool[d0 + j] = pool[src]
            new_idx[t] = d0 + j
    return new_pool, new_idx, status
