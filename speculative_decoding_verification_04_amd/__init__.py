"""MI355X-native verify-and-commit step of batch speculative decoding.

Thin Python binding over libspecverify.so (include/spec_verify.h).  The
functions carry the C entry points' names and only marshal arguments:
torch tensors on the GPU become device pointers, the current HIP stream is
passed along, and a nonzero return code raises SpecError.  Every step runs in
the library's HIP kernels; there is no other implementation.
"""
from __future__ import annotations

import ctypes

from . import _lib

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_OK, SPEC_EINVAL, SPEC_EWORKSPACE, SPEC_ECAPACITY, SPEC_EHIP = 0, -1, -2, -3, -4
SPEC_ST_DRAFT_OOR, SPEC_ST_Q_ZERO, SPEC_ST_RESID_ZERO = 1, 2, 4
SPEC_ST_NONFINITE, SPEC_ST_BAD_STATE, SPEC_ST_CAPACITY = 8, 16, 32
SPEC_MAX_K, SPEC_GROUP_MAX_N, SPEC_PROC_MAX_V, SPEC_TREE_MAX_N = 127, 4096, 524288, 256

__all__ = [
    "SpecError", "spec_strerror", "spec_verify_greedy_workspace_bytes", "spec_verify_greedy",
    "spec_verify_sample_workspace_bytes", "spec_verify_sample", "spec_process_workspace_bytes",
    "spec_process_logits", "spec_verify_sample_logits_workspace_bytes", "spec_verify_sample_logits",
    "spec_commit_realign_kv", "spec_resync_draft_kv", "spec_commit_paged",
    "spec_verify_tree_workspace_bytes", "spec_verify_tree", "spec_compact_tree_kv",
    "spec_group_same_length", "workspace", "library",
]


class SpecError(RuntimeError):
    def __init__(self, code: int, name: str):
        super().__init__(f"{name} failed: {spec_strerror(code)} ({code})")
        self.code = code


def library() -> ctypes.CDLL:
    return _lib.load()


def spec_strerror(code: int) -> str:
    return library().spec_strerror(int(code)).decode()


def _check(code: int, name: str) -> None:
    if code != SPEC_OK:
        raise SpecError(code, name)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace(nbytes: int, device=None):
    """A device workspace of at least nbytes (its contents need no initialisation)."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


def spec_verify_greedy_workspace_bytes(B: int, k: int, V: int, dtype_code: int) -> int:
    return int(library().spec_verify_greedy_workspace_bytes(B, k, V, dtype_code))


def spec_verify_sample_workspace_bytes(B: int, k: int, V: int) -> int:
    return int(library().spec_verify_sample_workspace_bytes(B, k, V))


def spec_verify_greedy(logits, draft, accept_len, emit_count, out_tokens, ws, *,
                       eos_id: int = -1, remaining=None, emit_offsets=None, status=None,
                       stream=None) -> None:
    """logits [B, k+1, V] (bf16/f32), draft [B, k] int32; outputs int32 tensors."""
    B, kp1, V = logits.shape
    code = library().spec_verify_greedy(
        _ptr(logits), _dtype_code(logits), B, kp1 - 1, V, _ptr(draft), int(eos_id), _ptr(remaining),
        _ptr(accept_len), _ptr(emit_count), _ptr(out_tokens), _ptr(emit_offsets), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_greedy")


def spec_verify_sample(p, q, draft, uniforms, accept_len, emit_count, out_tokens, ws, *,
                       eos_id: int = -1, remaining=None, emit_offsets=None, final_mass=None,
                       status=None, stream=None) -> None:
    """p [B, k+1, V] f32, q [B, k, V] f32, draft [B, k] int32, uniforms [B, k+1] f32."""
    B, kp1, V = p.shape
    code = library().spec_verify_sample(
        _ptr(p), _ptr(q), _ptr(draft), _ptr(uniforms), B, kp1 - 1, V, int(eos_id), _ptr(remaining),
        _ptr(accept_len), _ptr(emit_count), _ptr(out_tokens), _ptr(emit_offsets), _ptr(final_mass),
        _ptr(status), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_sample")


def spec_process_workspace_bytes(R: int, V: int) -> int:
    return int(library().spec_process_workspace_bytes(R, V))


def spec_verify_sample_logits_workspace_bytes(B: int, k: int, V: int) -> int:
    return int(library().spec_verify_sample_logits_workspace_bytes(B, k, V))


def spec_process_logits(logits, temperature: float, ws, *, top_k: int = 0, top_p: float = 1.0,
                        probs=None, row_max=None, row_threshold=None, row_mass=None,
                        stream=None) -> None:
    """logits [..., V] (bf16/f32); optional outputs probs [..., V] f32, row_max / row_threshold
    [R] f32, row_mass [R] f64 (R = number of rows)."""
    V = logits.shape[-1]
    R = logits.numel() // V
    code = library().spec_process_logits(
        _ptr(logits), _dtype_code(logits), R, V, float(temperature), int(top_k), float(top_p),
        _ptr(probs), _ptr(row_max), _ptr(row_threshold), _ptr(row_mass), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_process_logits")


def spec_verify_sample_logits(target_logits, draft_logits, draft, uniforms, accept_len, emit_count,
                              out_tokens, ws, *, temperature: float, top_k: int = 0,
                              top_p: float = 1.0, eos_id: int = -1, remaining=None,
                              emit_offsets=None, final_mass=None, status=None, stream=None) -> None:
    """target_logits [B, k+1, V], draft_logits [B, k, V] (same dtype, bf16/f32)."""
    B, kp1, V = target_logits.shape
    if draft_logits.dtype != target_logits.dtype:
        raise ValueError("target and draft logits must share a dtype")
    code = library().spec_verify_sample_logits(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, kp1 - 1, V,
        float(temperature), int(top_k), float(top_p), _ptr(draft), _ptr(uniforms), int(eos_id),
        _ptr(remaining), _ptr(accept_len), _ptr(emit_count), _ptr(out_tokens), _ptr(emit_offsets),
        _ptr(final_mass), _ptr(status), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_sample_logits")


def spec_commit_realign_kv(kv, k: int, end_col, kv_len_in, emit_count, end_col_out, kv_len_out,
                           pos_ids, mask, *, bytes_moved=None, status=None, stream=None) -> None:
    """kv [L, 2, B, H, C, D] (bf16/f32) is realigned in place."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_commit_realign_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(k), _ptr(end_col), _ptr(kv_len_in),
        _ptr(emit_count), _ptr(end_col_out), _ptr(kv_len_out), _ptr(pos_ids), _ptr(mask),
        _ptr(bytes_moved), _ptr(status), _stream(stream))
    _check(code, "spec_commit_realign_kv")


def spec_resync_draft_kv(kv, k: int, end_col, kv_len_in, emit_count, end_col_out, kv_len_out, *,
                         pos_ids=None, mask=None, bytes_moved=None, status=None, stream=None) -> None:
    """Draft cache kv [L, 2, B, H, C, D] (bf16/f32) keeps min(e_b, k) of its k forward slots."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_resync_draft_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(k), _ptr(end_col), _ptr(kv_len_in),
        _ptr(emit_count), _ptr(end_col_out), _ptr(kv_len_out), _ptr(pos_ids), _ptr(mask),
        _ptr(bytes_moved), _ptr(status), _stream(stream))
    _check(code, "spec_resync_draft_kv")


def spec_commit_paged(k: int, page_size: int, kv_len_in, emit_count, block_table, kv_len_out,
                      pages_kept, freed_pages, freed_offsets, *, status=None, stream=None) -> None:
    """block_table [B, max_pages] int32; freed_pages holds B * ceil((k+1)/page_size) ids."""
    B, max_pages = block_table.shape
    code = library().spec_commit_paged(
        B, int(k), int(page_size), max_pages, _ptr(kv_len_in), _ptr(emit_count), _ptr(block_table),
        _ptr(kv_len_out), _ptr(pages_kept), _ptr(freed_pages), _ptr(freed_offsets), _ptr(status),
        _stream(stream))
    _check(code, "spec_commit_paged")


def spec_verify_tree_workspace_bytes(B: int, N: int, V: int, dtype_code: int) -> int:
    return int(library().spec_verify_tree_workspace_bytes(B, N, V, dtype_code))


def spec_verify_tree(logits, draft, first_child, next_sibling, accept_len, emit_count, out_tokens, path,
                     ws, *, eos_id: int = -1, remaining=None, emit_offsets=None, status=None,
                     stream=None) -> None:
    """logits [B, N, V] (bf16/f32); draft, first_child, next_sibling [B, N] int32."""
    B, N, V = logits.shape
    code = library().spec_verify_tree(
        _ptr(logits), _dtype_code(logits), B, N, V, _ptr(draft), _ptr(first_child), _ptr(next_sibling),
        int(eos_id), _ptr(remaining), _ptr(accept_len), _ptr(emit_count), _ptr(out_tokens), _ptr(path),
        _ptr(emit_offsets), _ptr(status), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_tree")


def spec_compact_tree_kv(kv, N: int, end_col, path, emit_count, *, status=None, stream=None) -> None:
    """kv [L, 2, B, H, C, D] (bf16/f32): kept tree slots moved to columns E .. E+e-1 in place."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_compact_tree_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(N), _ptr(end_col), _ptr(path), _ptr(emit_count),
        _ptr(status), _stream(stream))
    _check(code, "spec_compact_tree_kv")


def spec_group_same_length(lengths, B: int, min_group: int, perm, batch_start, batch_len,
                           num_batches, num_grouped, *, stream=None) -> None:
    """lengths [N] int32; outputs perm [N], batch_start [N+1], batch_len [N], two scalars."""
    N = lengths.numel()
    code = library().spec_group_same_length(
        _ptr(lengths), N, int(B), int(min_group), _ptr(perm), _ptr(batch_start), _ptr(batch_len),
        _ptr(num_batches), _ptr(num_grouped), _stream(stream))
    _check(code, "spec_group_same_length")
