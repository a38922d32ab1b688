"""Seeded input generators (see the package docstring for what this holds and what it must not)."""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

LATENT = 512          # latent (= value) width of one KV row
ROPE = 64             # rope width of one KV row
ROW = LATENT + ROPE   # 576 bf16 per KV row
BF16_NAN = 0x7FC0     # quiet-NaN bit pattern used to poison unreferenced pool rows
BASE_SEED = 20261202


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_tree(rng: np.random.Generator, q_len: int) -> np.ndarray:
    """Draft tree of q_len nodes: node 0 is the root, parent(i) is uniform in [0, i)."""
    parents = np.full(q_len, -1, dtype=np.int32)
    for i in range(1, q_len):
        parents[i] = rng.integers(0, i)
    return parents


def chain_tree(q_len: int) -> np.ndarray:
    """A chain (parent(i) = i - 1): its mask is causal over the draft tokens."""
    return np.arange(-1, q_len - 1, dtype=np.int32)


def tree_mask(parents: np.ndarray, prefix: int) -> np.ndarray:
    """Visibility of one request: q_len rows of prefix + q_len bytes.

    Every prefix column is visible; draft column j is visible to draft row i iff
    j is i or an ancestor of i. Row stride is prefix + q_len.
    """
    q_len = len(parents)
    m = np.zeros((q_len, prefix + q_len), dtype=np.uint8)
    m[:, :prefix] = 1
    for i in range(q_len):
        j = i
        while j >= 0:
            m[i, prefix + j] = 1
            j = int(parents[j])
    return m


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    prefixes: tuple
    q_len: int
    H: int
    N: int
    layout: str            # "scattered" or "contiguous"
    nsplits: tuple
    seed: int
    description: str = ""
    scale: float = 1.0 / math.sqrt(192.0)

    @property
    def lengths(self):
        return [p + self.q_len for p in self.prefixes]


CONFIGS = {
    "tiny_256_h8": Workload("tiny_256_h8", 1, (256,), 9, 8, 4096, "scattered", (4,), BASE_SEED + 0,
                            "B=1, prefix 256, q_len 9, H=8, pool 4096, nsplit 4"),
    "4k_h64": Workload("4k_h64", 1, (4096,), 9, 64, 1 << 20, "scattered", (16,), BASE_SEED + 1,
                       "B=1, prefix 4096, q_len 9, H=64, pool 1M, nsplit 16"),
    "16k_h64": Workload("16k_h64", 1, (16384,), 9, 64, 1 << 20, "scattered", (16, 32, 64), BASE_SEED + 2,
                        "B=1, prefix 16384, q_len 9, H=64, pool 1M, contiguous and scattered, nsplit 16/32/64"),
    "65k_h8": Workload("65k_h8", 1, (65536,), 9, 8, 2 << 20, "scattered", (16, 64), BASE_SEED + 3,
                       "B=1, prefix 65536, q_len 9, H=8, pool 2M, nsplit 16/64"),
    "ragged4_185k_h64": Workload("ragged4_185k_h64", 4, (4096, 32768, 120000, 185000), 16, 64, 2 << 20,
                                 "scattered", (64,), BASE_SEED + 4,
                                 "B=4 ragged prefixes 4k/32k/120k/185k, q_len 16, H=64, pool 2M, nsplit 64"),
}


@dataclass
class Inputs:
    """Host arrays of one verify call (bf16 as uint16 bit patterns)."""
    B: int
    q_len: int
    H: int
    N: int
    scale: float
    q_nope: np.ndarray        # uint16 [B, q_len, H, 512]
    q_rope: np.ndarray        # uint16 [B, q_len, H, 64]
    kv_indptr: np.ndarray     # int32 [B+1]
    kv_indices: np.ndarray    # int32 [sum P_b]
    out_cache_loc: np.ndarray  # int32 [B*q_len]
    custom_mask: np.ndarray   # uint8 [sum q_len*L_b]
    mask_indptr: np.ndarray   # int32 [B+1]
    ref_slots: np.ndarray     # int32: distinct slots referenced (prefix then draft, request order)
    ref_rows: np.ndarray      # uint16 [len(ref_slots), 576]: pool contents of those slots
    parents: list = field(default_factory=list)

    @property
    def prefixes(self):
        return [int(self.kv_indptr[b + 1] - self.kv_indptr[b]) for b in range(self.B)]


def _draw_bf16(rng, shape):
    return bf16_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def make_inputs(wl: Workload, layout: str | None = None, seed: int | None = None) -> Inputs:
    """Draw one call's inputs. Draw order: trees, slot indices, q_nope, q_rope, pool rows."""
    layout = layout or wl.layout
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, q_len, H = wl.B, wl.q_len, wl.H
    prefixes = list(wl.prefixes)
    lengths = [p + q_len for p in prefixes]
    parents = [random_tree(rng, q_len) for _ in range(B)]
    total = sum(lengths)
    if layout == "scattered":
        slots = rng.choice(wl.N, size=total, replace=False).astype(np.int32)
    elif layout == "contiguous":
        if total > wl.N:
            raise ValueError("pool too small")
        # one ascending run per request, runs placed without overlap (a sorted free list)
        slots = np.empty(total, dtype=np.int32)
        gap_room = wl.N - total
        cuts = np.sort(rng.integers(0, gap_room + 1, size=B))
        pos, start = 0, 0
        for b in range(B):
            base = start + int(cuts[b])
            slots[pos:pos + lengths[b]] = np.arange(base, base + lengths[b], dtype=np.int32)
            start += lengths[b]
            pos += lengths[b]
    else:
        raise ValueError(layout)
    kv_indptr = np.zeros(B + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(prefixes)
    kv_indices = np.empty(sum(prefixes), dtype=np.int32)
    out_cache_loc = np.empty(B * q_len, dtype=np.int32)
    pos = 0
    for b in range(B):
        kv_indices[kv_indptr[b]:kv_indptr[b + 1]] = slots[pos:pos + prefixes[b]]
        out_cache_loc[b * q_len:(b + 1) * q_len] = slots[pos + prefixes[b]:pos + lengths[b]]
        pos += lengths[b]
    masks = [tree_mask(parents[b], prefixes[b]) for b in range(B)]
    mask_indptr = np.zeros(B + 1, dtype=np.int32)
    mask_indptr[1:] = np.cumsum([m.size for m in masks])
    custom_mask = np.concatenate([m.reshape(-1) for m in masks]) if B else np.zeros(0, np.uint8)
    q_nope = _draw_bf16(rng, (B, q_len, H, LATENT))
    q_rope = _draw_bf16(rng, (B, q_len, H, ROPE))
    ref_rows = _draw_bf16(rng, (total, ROW))
    return Inputs(B, q_len, H, wl.N, wl.scale, q_nope, q_rope, kv_indptr, kv_indices, out_cache_loc,
                  custom_mask, mask_indptr, slots, ref_rows, parents)


def make_custom(rng: np.random.Generator, prefixes, q_len: int, H: int, N: int | None = None,
                layout: str = "scattered", trees=None, scale: float = 1.0 / math.sqrt(192.0)) -> Inputs:
    """Inputs of any shape (edge cases); trees: None (random), "chain", or a list of parent arrays."""
    prefixes = list(prefixes)
    total = sum(p + q_len for p in prefixes)
    N = N if N is not None else max(2 * total, 64)
    wl = Workload("custom", len(prefixes), tuple(prefixes), q_len, H, N, layout, (1,), 0, scale=scale)
    seed = int(rng.integers(0, 2**31 - 1))
    inp = make_inputs(wl, seed=seed)
    if trees is not None:
        if trees == "chain":
            trees = [chain_tree(q_len) for _ in prefixes]
        masks = [tree_mask(np.asarray(trees[b], np.int32), prefixes[b]) for b in range(len(prefixes))]
        inp.custom_mask = np.concatenate([m.reshape(-1) for m in masks])
        inp.parents = [np.asarray(t, np.int32) for t in trees]
    return inp


def full_pool(inp: Inputs) -> np.ndarray:
    """The whole pool [N, 576] on the host: referenced rows in place, every other row NaN."""
    pool = np.full((inp.N, ROW), BF16_NAN, dtype=np.uint16)
    pool[inp.ref_slots] = inp.ref_rows
    return pool


def compact_inputs(inp: Inputs):
    """Relabel the referenced slots to 0..n-1 (same values, small pool) for host-side checkers.

    Returns (pool [n, 576], kv_indices, out_cache_loc) with slots renumbered by their position
    in ref_slots. Any correct implementation gives identical results on the relabelled inputs.
    """
    order = np.argsort(inp.ref_slots, kind="stable")
    sorted_slots = inp.ref_slots[order]

    def relabel(idx):
        pos = np.searchsorted(sorted_slots, idx)
        return order[pos].astype(np.int32)

    return inp.ref_rows, relabel(inp.kv_indices), relabel(inp.out_cache_loc)
