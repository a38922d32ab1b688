"""MI355X tree-verify attention over an MLA paged KV cache (split-KV flash-decode).

A thin ctypes binding of libmla_verify.so (C ABI declared in include/mla_verify.h). It only
checks and marshals arguments: every step of the computation runs in the library's HIP kernels.
There is no fallback path; calling without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_verify.so")
LATENT, ROPE, ROW = 512, 64, 576
MAX_NSPLIT = 1024
WORKSPACE_ALIGN = 256
NOALLOC_SCRATCH_BYTES = 128 << 20  # static scratch per device of the no-alloc entry point

STATUS = {0: "MLA_VERIFY_OK", -1: "MLA_VERIFY_ERR_NULL", -2: "MLA_VERIFY_ERR_SHAPE",
          -3: "MLA_VERIFY_ERR_NSPLIT", -4: "MLA_VERIFY_ERR_WORKSPACE", -5: "MLA_VERIFY_ERR_LAUNCH",
          -6: "MLA_VERIFY_ERR_SCRATCH"}

_lib = None


class MlaVerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libmla_verify.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m speculative_decoding_mla_split_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.mla_verify_attn_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.mla_verify_attn_workspace_size.restype = sz
        lib.mla_verify_status_string.argtypes = [i32]
        lib.mla_verify_status_string.restype = ctypes.c_char_p
        lib.mla_verify_attn.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp, sz, vp,
                                        vp, vp]
        lib.mla_verify_attn.restype = i32
        lib.mla_verify_attn_partial.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp,
                                                sz, vp]
        lib.mla_verify_attn_partial.restype = i32
        lib.mla_verify_attn_combine.argtypes = [vp, sz, vp, i64, i32, i32, i32, i32, vp, vp, vp]
        lib.mla_verify_attn_combine.restype = i32
        lib.mla_verify_attn_balanced_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.mla_verify_attn_balanced_workspace_size.restype = sz
        lib.mla_verify_attn_balanced.argtypes = lib.mla_verify_attn.argtypes
        lib.mla_verify_attn_balanced.restype = i32
        lib.mla_verify_attn_balanced_partial.argtypes = lib.mla_verify_attn_partial.argtypes
        lib.mla_verify_attn_balanced_partial.restype = i32
        lib.mla_verify_attn_balanced_combine.argtypes = lib.mla_verify_attn_combine.argtypes
        lib.mla_verify_attn_balanced_combine.restype = i32
        lib.mla_verify_attn_balanced_noalloc.argtypes = lib.mla_verify_attn.argtypes[:14] + [vp, vp, vp]
        lib.mla_verify_attn_balanced_noalloc.restype = i32
        lib.mla_verify_attn_check.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, i32, vp,
                                              sz, vp, vp]
        lib.mla_verify_attn_check_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.mla_verify_attn_check_workspace_size.restype = sz
        lib.mla_verify_attn_validate_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        lib.mla_verify_attn_validate_workspace_size.restype = sz
        lib.mla_verify_attn_check.restype = i32
        lib.mla_verify_attn_validate.argtypes = lib.mla_verify_attn.argtypes[:18] + [i32, vp, vp]
        lib.mla_verify_attn_validate.restype = i32
        lib.mla_verify_tree_mask.argtypes = [vp, vp, i32, i32, vp, i64, vp, vp, vp]
        lib.mla_verify_tree_mask.restype = i32
        lib.mla_verify_kv_compact.argtypes = [vp, i64, vp, vp, vp, i32, vp, vp, vp]
        lib.mla_verify_kv_compact.restype = i32
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().mla_verify_status_string(int(status)).decode()


def workspace_size(B: int, q_len: int, H: int, nsplit: int) -> int:
    """Bytes of workspace verify_attn needs (0 if an argument is out of range)."""
    return int(library().mla_verify_attn_workspace_size(int(B), int(q_len), int(H), int(nsplit)))


def attn_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
             B, q_len, H, scale, nsplit, workspace, workspace_bytes, out, lse, stream) -> int:
    """Direct call of mla_verify_attn with integer device addresses; returns the status."""
    return int(library().mla_verify_attn(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices, out_cache_loc,
                                         custom_mask, mask_indptr, int(B), int(q_len), int(H), float(scale),
                                         int(nsplit), workspace, int(workspace_bytes), out, lse, stream))


def partial_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                B, q_len, H, scale, nsplit, workspace, workspace_bytes, stream) -> int:
    """Direct call of mla_verify_attn_partial with integer device addresses; returns the status."""
    return int(library().mla_verify_attn_partial(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices,
                                                 out_cache_loc, custom_mask, mask_indptr, int(B), int(q_len), int(H),
                                                 float(scale), int(nsplit), workspace, int(workspace_bytes), stream))


def combine_raw(workspace, workspace_bytes, kv_pool, N, B, q_len, H, nsplit, out, lse, stream) -> int:
    """Direct call of mla_verify_attn_combine with integer device addresses; returns the status."""
    return int(library().mla_verify_attn_combine(workspace, int(workspace_bytes), kv_pool, int(N), int(B), int(q_len),
                                                 int(H), int(nsplit), out, lse, stream))


def balanced_workspace_size(B: int, q_len: int, H: int, units: int) -> int:
    """Bytes of workspace verify_attn_balanced needs (0 if an argument is out of range)."""
    return int(library().mla_verify_attn_balanced_workspace_size(int(B), int(q_len), int(H), int(units)))


def balanced_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                 B, q_len, H, scale, units, workspace, workspace_bytes, out, lse, stream) -> int:
    """Direct call of mla_verify_attn_balanced with integer device addresses; returns the status."""
    return int(library().mla_verify_attn_balanced(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices,
                                                  out_cache_loc, custom_mask, mask_indptr, int(B), int(q_len),
                                                  int(H), float(scale), int(units), workspace,
                                                  int(workspace_bytes), out, lse, stream))


def balanced_partial_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                         B, q_len, H, scale, units, workspace, workspace_bytes, stream) -> int:
    """Direct call of mla_verify_attn_balanced_partial; returns the status."""
    return int(library().mla_verify_attn_balanced_partial(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices,
                                                          out_cache_loc, custom_mask, mask_indptr, int(B),
                                                          int(q_len), int(H), float(scale), int(units), workspace,
                                                          int(workspace_bytes), stream))


def balanced_combine_raw(workspace, workspace_bytes, kv_pool, N, B, q_len, H, units, out, lse, stream) -> int:
    """Direct call of mla_verify_attn_balanced_combine; returns the status."""
    return int(library().mla_verify_attn_balanced_combine(workspace, int(workspace_bytes), kv_pool, int(N), int(B),
                                                          int(q_len), int(H), int(units), out, lse, stream))


def balanced_noalloc_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                         B, q_len, H, scale, units, out, lse, stream) -> int:
    """Direct call of mla_verify_attn_balanced_noalloc (the library's static scratch in place of a
    workspace); returns the status."""
    return int(library().mla_verify_attn_balanced_noalloc(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices,
                                                          out_cache_loc, custom_mask, mask_indptr, int(B),
                                                          int(q_len), int(H), float(scale), int(units), out, lse,
                                                          stream))


REPORT_MAX_OUT, REPORT_MAX_LSE, REPORT_ROWS, REPORT_BAD, REPORT_WORDS = 0, 1, 2, 3, 4


def check_workspace_size(B: int, q_len: int, H: int, sample_stride: int) -> int:
    """Bytes of workspace check_attn needs (0 if an argument is out of range)."""
    return int(library().mla_verify_attn_check_workspace_size(int(B), int(q_len), int(H), int(sample_stride)))


def validate_workspace_size(B: int, q_len: int, H: int, nsplit: int, sample_stride: int) -> int:
    """Bytes of workspace mla_verify_attn_validate needs (0 if an argument is out of range)."""
    return int(library().mla_verify_attn_validate_workspace_size(int(B), int(q_len), int(H), int(nsplit),
                                                                 int(sample_stride)))


def check_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
              B, q_len, H, scale, out, lse, sample_stride, workspace, workspace_bytes, report, stream) -> int:
    """Direct call of mla_verify_attn_check with integer device addresses; returns the status."""
    return int(library().mla_verify_attn_check(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices, out_cache_loc,
                                               custom_mask, mask_indptr, int(B), int(q_len), int(H), float(scale),
                                               out, lse, int(sample_stride), workspace, int(workspace_bytes), report,
                                               stream))


def validate_raw(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                 B, q_len, H, scale, nsplit, workspace, workspace_bytes, out, lse, sample_stride, report,
                 stream) -> int:
    """Direct call of mla_verify_attn_validate with integer device addresses; returns the status."""
    return int(library().mla_verify_attn_validate(q_nope, q_rope, kv_pool, int(N), kv_indptr, kv_indices,
                                                  out_cache_loc, custom_mask, mask_indptr, int(B), int(q_len),
                                                  int(H), float(scale), int(nsplit), workspace, int(workspace_bytes),
                                                  out, lse, int(sample_stride), report, stream))


def tree_mask_raw(parents, kv_indptr, B, q_len, custom_mask, mask_capacity, mask_indptr, status, stream) -> int:
    """Direct call of mla_verify_tree_mask with integer device addresses; returns the status."""
    return int(library().mla_verify_tree_mask(parents, kv_indptr, int(B), int(q_len), custom_mask,
                                              int(mask_capacity), mask_indptr, status, stream))


def kv_compact_raw(kv_pool, N, kv_indptr, kv_indices, dst_start, B, new_kv_indices, status, stream) -> int:
    """Direct call of mla_verify_kv_compact with integer device addresses; returns the status."""
    return int(library().mla_verify_kv_compact(kv_pool, int(N), kv_indptr, kv_indices, dst_start, int(B),
                                               new_kv_indices, status, stream))


TREE_BAD_PARENT, TREE_CAPACITY = 1, 2
COMPACT_BAD_DST, COMPACT_BAD_SRC = 1, 2


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def verify_attn(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                scale: float, nsplit: int, workspace, out, lse, stream=None, balanced: bool = False) -> None:
    """Tree-verify attention on torch device tensors (no copies, no host synchronisation).

    q_nope bf16 [B,q_len,H,512], q_rope bf16 [B,q_len,H,64], kv_pool bf16 [N,576],
    kv_indptr int32 [B+1], kv_indices int32, out_cache_loc int32 [B*q_len], custom_mask uint8/bool,
    mask_indptr int32 [>=B], workspace uint8 [>= workspace_size(...)], out bf16 [B,q_len,H,512],
    lse float32 [B,q_len,H]. stream: a torch.cuda.Stream (default: the current stream).
    balanced=True runs mla_verify_attn_balanced with nsplit as the batch's split budget (`units`,
    workspace from balanced_workspace_size).
    """
    import torch

    B, q_len, H, d = q_nope.shape
    _need(d == LATENT and tuple(q_rope.shape) == (B, q_len, H, ROPE), "q_nope/q_rope shapes")
    _need(kv_pool.dim() == 2 and kv_pool.shape[1] == ROW, "kv_pool must be [N, 576]")
    _need(tuple(out.shape) == (B, q_len, H, LATENT) and tuple(lse.shape) == (B, q_len, H), "out/lse shapes")
    for name, t, dt in (("q_nope", q_nope, torch.bfloat16), ("q_rope", q_rope, torch.bfloat16),
                        ("kv_pool", kv_pool, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("lse", lse, torch.float32), ("kv_indptr", kv_indptr, torch.int32),
                        ("kv_indices", kv_indices, torch.int32), ("out_cache_loc", out_cache_loc, torch.int32),
                        ("mask_indptr", mask_indptr, torch.int32), ("workspace", workspace, torch.uint8)):
        _need(t.dtype == dt, f"{name} must be {dt}")
        _need(t.is_cuda, f"{name} must be a device tensor")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(custom_mask.dtype in (torch.uint8, torch.bool) and custom_mask.is_cuda and custom_mask.is_contiguous(),
          "custom_mask must be a contiguous uint8/bool device tensor")
    _need(kv_indptr.numel() >= B + 1 and mask_indptr.numel() >= B and out_cache_loc.numel() >= B * q_len,
          "index array lengths")
    if stream is None:
        stream = torch.cuda.current_stream(q_nope.device)
    call = balanced_raw if balanced else attn_raw
    rc = call(q_nope.data_ptr(), q_rope.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                  kv_indptr.data_ptr(), kv_indices.data_ptr() if kv_indices.numel() else None,
                  out_cache_loc.data_ptr(), custom_mask.data_ptr(), mask_indptr.data_ptr(), B, q_len, H, scale,
                  nsplit, workspace.data_ptr(), workspace.numel(), out.data_ptr(), lse.data_ptr(),
                  stream.cuda_stream)
    if rc != 0:
        raise MlaVerifyError(rc, status_string(rc))


def _dev_i32(name, t):
    import torch
    _need(t.dtype == torch.int32 and t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous int32 device tensor")


def build_tree_mask(parents, kv_indptr, custom_mask, mask_indptr, status, stream=None) -> None:
    """Device-built custom_mask + mask_indptr from draft trees (no copies, no host synchronisation).

    parents int32 [B, q_len] (parent index inside the request, -1 for a root), kv_indptr int32 [B+1],
    custom_mask uint8 (capacity = its numel), mask_indptr int32 [B+1], status int32 [1]
    (TREE_BAD_PARENT / TREE_CAPACITY bits, read it whenever convenient).
    """
    import torch

    _need(parents.dim() == 2, "parents must be [B, q_len]")
    B, q_len = parents.shape
    for name, t in (("parents", parents), ("kv_indptr", kv_indptr), ("mask_indptr", mask_indptr),
                    ("status", status)):
        _dev_i32(name, t)
    _need(custom_mask.dtype in (torch.uint8, torch.bool) and custom_mask.is_cuda and custom_mask.is_contiguous(),
          "custom_mask must be a contiguous uint8/bool device tensor")
    _need(kv_indptr.numel() >= B + 1 and mask_indptr.numel() >= B + 1 and status.numel() >= 1, "array lengths")
    if stream is None:
        stream = torch.cuda.current_stream(parents.device)
    rc = tree_mask_raw(parents.data_ptr(), kv_indptr.data_ptr(), B, q_len, custom_mask.data_ptr(),
                       custom_mask.numel(), mask_indptr.data_ptr(), status.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise MlaVerifyError(rc, status_string(rc))


def compact_kv(kv_pool, kv_indptr, kv_indices, dst_start, new_kv_indices, status, stream=None) -> None:
    """Move each request's prefix rows to dst_start[b] + j in place and write the new indices.

    kv_pool bf16 [N, 576] (modified), kv_indptr int32 [B+1], kv_indices int32, dst_start int32 [B],
    new_kv_indices int32 (same length as kv_indices, not overlapping it), status int32 [1]
    (COMPACT_BAD_DST / COMPACT_BAD_SRC bits).
    """
    import torch

    _need(kv_pool.dim() == 2 and kv_pool.shape[1] == ROW and kv_pool.dtype == torch.bfloat16 and kv_pool.is_cuda
          and kv_pool.is_contiguous(), "kv_pool must be a contiguous bf16 [N, 576] device tensor")
    B = dst_start.numel()
    for name, t in (("kv_indptr", kv_indptr), ("kv_indices", kv_indices), ("dst_start", dst_start),
                    ("new_kv_indices", new_kv_indices), ("status", status)):
        _dev_i32(name, t)
    _need(kv_indptr.numel() >= B + 1 and new_kv_indices.numel() >= kv_indices.numel(), "array lengths")
    if stream is None:
        stream = torch.cuda.current_stream(kv_pool.device)
    rc = kv_compact_raw(kv_pool.data_ptr(), kv_pool.shape[0], kv_indptr.data_ptr(), kv_indices.data_ptr(),
                        dst_start.data_ptr(), B, new_kv_indices.data_ptr(), status.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise MlaVerifyError(rc, status_string(rc))


def check_attn(q_nope, q_rope, kv_pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
               scale: float, out, lse, report, workspace, sample_stride: int = 1, stream=None) -> None:
    """Device-side cross-check of out/lse against the per-row reference (validate mode).

    Same tensors as verify_attn; report is a float32 device tensor of REPORT_WORDS values that
    receives (max |out - ref|, max |lse - ref|, rows checked, bad rows); workspace is a uint8 device
    tensor of check_workspace_size(...) bytes. Nothing is synchronised.
    """
    import torch

    B, q_len, H, _ = q_nope.shape
    _need(report.dtype == torch.float32 and report.is_cuda and report.numel() >= REPORT_WORDS, "report")
    _need(workspace.dtype == torch.uint8 and workspace.is_cuda, "workspace")
    if stream is None:
        stream = torch.cuda.current_stream(q_nope.device)
    rc = check_raw(q_nope.data_ptr(), q_rope.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0], kv_indptr.data_ptr(),
                   kv_indices.data_ptr() if kv_indices.numel() else None, out_cache_loc.data_ptr(),
                   custom_mask.data_ptr(), mask_indptr.data_ptr(), B, q_len, H, scale, out.data_ptr(), lse.data_ptr(),
                   sample_stride, workspace.data_ptr(), workspace.numel(), report.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise MlaVerifyError(rc, status_string(rc))
