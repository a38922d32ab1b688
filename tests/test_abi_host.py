"""C-ABI checks that need no GPU: symbols, workspace sizing, argument validation before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import speculative_decoding_mla_split_amd as pkg

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(INCLUDE, "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mla_verify_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = pkg.library()
    names = _declared_functions()
    assert set(names) == {"mla_verify_attn", "mla_verify_attn_partial", "mla_verify_attn_combine",
                          "mla_verify_attn_workspace_size", "mla_verify_status_string",
                          "mla_verify_tree_mask", "mla_verify_kv_compact",
                          "mla_verify_attn_balanced", "mla_verify_attn_balanced_partial",
                          "mla_verify_attn_balanced_combine", "mla_verify_attn_balanced_workspace_size",
                          "mla_verify_attn_balanced_noalloc",
                          "mla_verify_attn_check", "mla_verify_attn_validate",
                          "mla_verify_attn_check_workspace_size", "mla_verify_attn_validate_workspace_size"}
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_size():
    # {m, l, 2^e, 0} float4 + 512 fp16 + an 8-byte top record per (b, split, token, head), each region padded
    # to 256 bytes
    rows = 2 * 16 * 9 * 8
    expect = -(-rows * 16 // 256) * 256 + -(-rows * 1024 // 256) * 256 + -(-rows * 8 // 256) * 256
    assert pkg.workspace_size(2, 9, 8, 16) == expect
    assert pkg.workspace_size(0, 9, 8, 16) == 0
    assert pkg.workspace_size(1, 0, 8, 16) == 0
    assert pkg.workspace_size(1, 9, 0, 16) == 0
    assert pkg.workspace_size(1, 9, 8, 0) == 0
    assert pkg.workspace_size(1, 9, 8, 1025) == 0
    assert pkg.workspace_size(1, 9, 8, 1024) > 0


def test_status_strings():
    for code in range(-6, 1):
        assert pkg.status_string(code)
    assert pkg.status_string(7) == "unknown status"


FAKE = 0x10000  # a non-null address that is never dereferenced: every call below fails validation


def _call(**kw):
    args = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE,
                out_cache_loc=FAKE, custom_mask=FAKE, mask_indptr=FAKE, B=1, q_len=9, H=8, scale=0.07,
                nsplit=4, workspace=0x100000, workspace_bytes=pkg.workspace_size(1, 9, 8, 4), out=FAKE, lse=FAKE,
                stream=None)
    args.update(kw)
    return pkg.attn_raw(**args)


@pytest.mark.parametrize("field", ["q_nope", "q_rope", "kv_pool", "kv_indptr", "out_cache_loc", "custom_mask",
                                   "mask_indptr", "out", "lse"])
def test_null_pointer_rejected(field):
    assert _call(**{field: None}) == -1


@pytest.mark.parametrize("kw", [dict(B=0), dict(q_len=0), dict(H=0), dict(N=0), dict(N=2**31),
                                dict(scale=float("inf")), dict(scale=float("nan")), dict(scale=0.0),
                                dict(scale=-0.5), dict(B=1 << 20, H=1 << 11)])
def test_bad_shape_rejected(kw):
    assert _call(**kw) == -2


@pytest.mark.parametrize("ns", [0, -1, 1025])
def test_bad_nsplit_rejected(ns):
    assert _call(nsplit=ns) == -3


def test_workspace_rejected():
    assert _call(workspace=None) == -4
    assert _call(workspace=0x100010) == -4                      # not 256-byte aligned
    assert _call(workspace_bytes=pkg.workspace_size(1, 9, 8, 4) - 1) == -4


def test_phase_entry_points_validate():
    ws_bytes = pkg.workspace_size(1, 9, 8, 4)
    base = (FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 9, 8, 0.07, 4, 0x100000, ws_bytes, None)
    assert pkg.partial_raw(*base[:2], None, *base[3:]) == -1
    assert pkg.partial_raw(*base[:13], 0, *base[14:]) == -3
    assert pkg.partial_raw(*base[:15], ws_bytes - 1, None) == -4
    assert pkg.combine_raw(0x100000, ws_bytes, FAKE, 100, 1, 9, 8, 4, None, FAKE, None) == -1
    assert pkg.combine_raw(0x100000, ws_bytes, None, 100, 1, 9, 8, 4, FAKE, FAKE, None) == -1  # pool needed
    assert pkg.combine_raw(0x100000, ws_bytes, FAKE, 0, 1, 9, 8, 4, FAKE, FAKE, None) == -2
    assert pkg.combine_raw(0x100000, ws_bytes, FAKE, 100, 1, 9, 8, 5, FAKE, FAKE, None) == -4
    assert pkg.combine_raw(0x100000, ws_bytes, FAKE, 100, 0, 9, 8, 4, FAKE, FAKE, None) == -2


def test_tree_mask_validates_before_any_hip_call():
    ok = dict(parents=FAKE, kv_indptr=FAKE, B=2, q_len=9, custom_mask=FAKE, mask_capacity=1000, mask_indptr=FAKE,
              status=FAKE, stream=None)
    for f in ("parents", "kv_indptr", "custom_mask", "mask_indptr", "status"):
        assert pkg.tree_mask_raw(**{**ok, f: None}) == -1, f
    for kw in (dict(B=0), dict(B=65536), dict(q_len=0), dict(q_len=4097), dict(mask_capacity=-1)):
        assert pkg.tree_mask_raw(**{**ok, **kw}) == -2, kw


def test_kv_compact_validates_before_any_hip_call():
    ok = dict(kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE, dst_start=FAKE, B=2, new_kv_indices=FAKE,
              status=FAKE, stream=None)
    for f in ("kv_pool", "kv_indptr", "kv_indices", "dst_start", "new_kv_indices", "status"):
        assert pkg.kv_compact_raw(**{**ok, f: None}) == -1, f
    for kw in (dict(B=0), dict(B=4097), dict(N=0), dict(N=2**31), dict(kv_pool=FAKE + 8)):
        assert pkg.kv_compact_raw(**{**ok, **kw}) == -2, kw


def test_balanced_workspace_size_and_validation():
    rows = 40 * 16 * 64
    plan = -(-(40 * 16 + 5 * 4) // 256) * 256
    expect = plan + -(-rows * 16 // 256) * 256 + -(-rows * 1024 // 256) * 256 + -(-rows * 8 // 256) * 256
    assert pkg.balanced_workspace_size(4, 16, 64, 40) == expect
    assert pkg.balanced_workspace_size(4, 16, 64, 3) == 0          # fewer units than requests
    assert pkg.balanced_workspace_size(4, 16, 64, 4097) == 0
    assert pkg.balanced_workspace_size(4097, 1, 1, 4097) == 0
    ws = pkg.balanced_workspace_size(2, 9, 8, 8)
    base = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE,
                out_cache_loc=FAKE, custom_mask=FAKE, mask_indptr=FAKE, B=2, q_len=9, H=8, scale=0.07, units=8,
                workspace=0x100000, workspace_bytes=ws, out=FAKE, lse=FAKE, stream=None)
    assert pkg.balanced_raw(**{**base, "out": None}) == -1
    assert pkg.balanced_raw(**{**base, "units": 1}) == -3
    assert pkg.balanced_raw(**{**base, "units": 4097}) == -3
    assert pkg.balanced_raw(**{**base, "B": 4097}) == -2
    assert pkg.balanced_raw(**{**base, "workspace_bytes": ws - 1}) == -4
    assert pkg.balanced_raw(**{**base, "workspace": 0x100010}) == -4
    assert pkg.balanced_combine_raw(0x100000, ws, FAKE, 100, 2, 9, 8, 8, None, FAKE, None) == -1
    assert pkg.balanced_combine_raw(0x100000, ws, None, 100, 2, 9, 8, 8, FAKE, FAKE, None) == -1
    assert pkg.balanced_combine_raw(0x100000, ws, FAKE, 2**31, 2, 9, 8, 8, FAKE, FAKE, None) == -2
    assert pkg.balanced_combine_raw(0x100000, ws - 1, FAKE, 100, 2, 9, 8, 8, FAKE, FAKE, None) == -4


def test_check_workspace_sizes():
    # 72 rows at stride 1 -> 72 checked rows x 64 pieces x ((m, sum) + 512 accumulators)
    pieces = 72 * 64
    expect = -(-pieces * 8 // 256) * 256 + -(-pieces * 2048 // 256) * 256
    assert pkg.check_workspace_size(1, 9, 8, 1) == expect
    assert pkg.check_workspace_size(1, 9, 8, 8) < expect
    assert pkg.check_workspace_size(1, 9, 8, 0) == 0
    assert pkg.validate_workspace_size(1, 9, 8, 4, 1) == max(expect, pkg.workspace_size(1, 9, 8, 4))
    assert pkg.validate_workspace_size(1, 9, 8, 0, 1) == 0


def test_check_and_validate_validate_before_any_hip_call():
    cws = pkg.check_workspace_size(1, 9, 8, 1)
    base = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE,
                out_cache_loc=FAKE, custom_mask=FAKE, mask_indptr=FAKE, B=1, q_len=9, H=8, scale=0.07, out=FAKE,
                lse=FAKE, sample_stride=1, workspace=0x100000, workspace_bytes=cws, report=FAKE, stream=None)
    for f in ("q_nope", "kv_pool", "out", "lse", "report", "mask_indptr"):
        assert pkg.check_raw(**{**base, f: None}) == -1, f
    for kw in (dict(sample_stride=0), dict(B=0), dict(N=0), dict(scale=float("nan"))):
        assert pkg.check_raw(**{**base, **kw}) == -2, kw
    assert pkg.check_raw(**{**base, "workspace_bytes": cws - 1}) == -4
    assert pkg.check_raw(**{**base, "workspace": 0x100010}) == -4
    ws = pkg.validate_workspace_size(1, 9, 8, 4, 1)
    v = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE, out_cache_loc=FAKE,
             custom_mask=FAKE, mask_indptr=FAKE, B=1, q_len=9, H=8, scale=0.07, nsplit=4, workspace=0x100000,
             workspace_bytes=ws, out=FAKE, lse=FAKE, sample_stride=1, report=FAKE, stream=None)
    assert pkg.validate_raw(**{**v, "report": None}) == -1
    assert pkg.validate_raw(**{**v, "sample_stride": 0}) == -2
    assert pkg.validate_raw(**{**v, "nsplit": 0}) == -3
    assert pkg.validate_raw(**{**v, "workspace_bytes": ws - 1}) == -4


def test_noalloc_validation_before_any_hip_call():
    """The no-alloc entry point rejects bad arguments, and sizes whose balanced workspace exceeds
    its static scratch, before touching the device (so these calls run without a GPU)."""
    base = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, N=100, kv_indptr=FAKE, kv_indices=FAKE, out_cache_loc=FAKE,
                custom_mask=FAKE, mask_indptr=FAKE, B=4, q_len=16, H=64, scale=0.07, units=32, out=FAKE, lse=FAKE,
                stream=None)
    assert pkg.balanced_noalloc_raw(**{**base, "out": None}) == -1
    assert pkg.balanced_noalloc_raw(**{**base, "lse": None}) == -1
    assert pkg.balanced_noalloc_raw(**{**base, "q_len": 0}) == -2
    assert pkg.balanced_noalloc_raw(**{**base, "scale": float("nan")}) == -2
    assert pkg.balanced_noalloc_raw(**{**base, "units": 3}) == -3
    assert pkg.balanced_noalloc_raw(**{**base, "units": 4097}) == -3
    # the ragged four-request batch of 64 heads and 16 tokens fits at 32 units, not at 128
    assert pkg.balanced_workspace_size(4, 16, 64, 32) <= pkg.NOALLOC_SCRATCH_BYTES
    assert pkg.balanced_workspace_size(4, 16, 64, 128) > pkg.NOALLOC_SCRATCH_BYTES
    assert pkg.balanced_noalloc_raw(**{**base, "units": 128}) == -6
    assert "static scratch" in pkg.status_string(-6)
