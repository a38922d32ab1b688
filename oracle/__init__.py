"""CPU fp64 oracle of the MLA tree-verify attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg
may import this package. The HIP library never calls it and shares no code with
it. The arithmetic lives in mla_verify_oracle.c (plain C, double precision,
OpenMP over rows); this file only builds that library and marshals numpy arrays.

Pins (tests/test_oracle.py): brute force in pure Python on tiny inputs, closed
forms (q = 0, one visible column, score shift), library special cases (all
visible = plain softmax attention, chain tree = causal attention, q_len = 1 =
decode), masked-column and slot-relabel invariance, split invariance and
weights summing to one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_verify_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
LATENT = 512

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (x86-64-v3, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        common = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, dbl]
        lib.mla_oracle_attn.argtypes = common + [vp, vp, i32]
        lib.mla_oracle_attn_split.argtypes = common + [i32, vp, vp, i32]
        lib.mla_oracle_attn_rows.argtypes = common + [i64, vp, vp, vp, vp, vp, i32]
        lib.mla_oracle_row_weights.argtypes = common + [i32, i32, i32, vp]
        for f in (lib.mla_oracle_attn, lib.mla_oracle_attn_split, lib.mla_oracle_attn_rows,
                  lib.mla_oracle_row_weights):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else ctypes.c_void_p(0)


class _Args:
    """Contiguous copies of one call's arrays (kept alive for the ctypes call)."""

    def __init__(self, q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                 mask_indptr, scale):
        self.q_nope = np.ascontiguousarray(q_nope, dtype=np.uint16)
        self.q_rope = np.ascontiguousarray(q_rope, dtype=np.uint16)
        self.kv_pool = np.ascontiguousarray(kv_pool, dtype=np.uint16)
        self.kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
        self.kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
        self.out_cache_loc = np.ascontiguousarray(out_cache_loc, dtype=np.int32)
        self.custom_mask = np.ascontiguousarray(custom_mask, dtype=np.uint8)
        self.mask_indptr = np.ascontiguousarray(mask_indptr, dtype=np.int32)
        self.B, self.q_len, self.H = self.q_nope.shape[:3]
        assert self.q_nope.shape[3] == LATENT and self.q_rope.shape == (self.B, self.q_len, self.H, 64)
        assert self.kv_pool.ndim == 2 and self.kv_pool.shape[1] == 576
        self.scale = float(scale)

    def head(self):
        return [_ptr(self.q_nope), _ptr(self.q_rope), _ptr(self.kv_pool), self.kv_pool.shape[0],
                _ptr(self.kv_indptr), _ptr(self.kv_indices), _ptr(self.out_cache_loc),
                _ptr(self.custom_mask), _ptr(self.mask_indptr), self.B, self.q_len, self.H, self.scale]


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")


def attn(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
         scale, nthreads: int = 0):
    """Plain definition. Returns (out float64 [B,q_len,H,512], lse float64 [B,q_len,H])."""
    a = _Args(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              scale)
    out = np.empty((a.B, a.q_len, a.H, LATENT), np.float64)
    lse = np.empty((a.B, a.q_len, a.H), np.float64)
    _check(_load().mla_oracle_attn(*a.head(), _ptr(out), _ptr(lse), nthreads))
    return out, lse


def attn_split(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
               scale, nsplit: int, nthreads: int = 0):
    """Same result through nsplit per-split partials and the log-sum-exp combine."""
    a = _Args(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              scale)
    out = np.empty((a.B, a.q_len, a.H, LATENT), np.float64)
    lse = np.empty((a.B, a.q_len, a.H), np.float64)
    _check(_load().mla_oracle_attn_split(*a.head(), int(nsplit), _ptr(out), _ptr(lse), nthreads))
    return out, lse


def attn_rows(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              scale, rows, nthreads: int = 0):
    """Only the rows listed in rows (int array [n, 3] of (b, i, h)). Returns (out [n,512], lse [n])."""
    a = _Args(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              scale)
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
    rb, ri, rh = (np.ascontiguousarray(rows[:, k]) for k in range(3))
    out = np.empty((len(rows), LATENT), np.float64)
    lse = np.empty(len(rows), np.float64)
    _check(_load().mla_oracle_attn_rows(*a.head(), len(rows), _ptr(rb), _ptr(ri), _ptr(rh), _ptr(out),
                                        _ptr(lse), nthreads))
    return out, lse


def row_weights(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                scale, b: int, i: int, h: int):
    """Softmax weights of row (b, i, h) over its prefix + q_len columns (0 where masked)."""
    a = _Args(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              scale)
    L = int(a.kv_indptr[b + 1] - a.kv_indptr[b]) + a.q_len
    w = np.empty(L, np.float64)
    _check(_load().mla_oracle_row_weights(*a.head(), int(b), int(i), int(h), _ptr(w)))
    return w


def inputs_args(inp, pool=None, kv_indices=None, out_cache_loc=None):
    """Positional arguments of the functions above from a workloads.Inputs (optionally relabelled)."""
    return (inp.q_nope, inp.q_rope, pool, inp.kv_indptr,
            inp.kv_indices if kv_indices is None else kv_indices,
            inp.out_cache_loc if out_cache_loc is None else out_cache_loc,
            inp.custom_mask, inp.mask_indptr, inp.scale)
