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
SPEC_ST_NONFINITE, SPEC_ST_BAD_STATE, SPEC_ST_CAPACITY, SPEC_ST_INCOMPLETE = 8, 16, 32, 64
SPEC_MAX_K, SPEC_GROUP_MAX_N, SPEC_PROC_MAX_V, SPEC_TREE_MAX_N = 127, 4096, 524288, 256
SPEC_GREEDY_SCRATCH_BYTES = 8 << 20

__all__ = [
    "SpecError", "spec_strerror", "spec_verify_greedy_workspace_bytes", "spec_verify_greedy",
    "spec_verify_greedy_noalloc", "SPEC_GREEDY_SCRATCH_BYTES",
    "spec_verify_sample_workspace_bytes", "spec_verify_sample", "spec_process_workspace_bytes",
    "spec_process_logits", "spec_verify_sample_logits_workspace_bytes", "spec_verify_sample_logits",
    "spec_commit_realign_kv", "spec_resync_draft_kv", "spec_repad_kv", "spec_unpad_kv", "spec_commit_paged",
    "spec_verify_tree_workspace_bytes", "spec_verify_tree", "spec_compact_tree_kv", "spec_verify_tree_sample_workspace_bytes",
    "spec_verify_tree_sample",
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


def spec_set_wait_bound(polls: int) -> int:
    """Bound the single-launch greedy and tree commit's wait (polls; <= 0: the
    default); returns the previous setting.  For tests of the incomplete path."""
    return int(library().spec_set_wait_bound(int(polls)))


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


def _arg(t, dtype: str, numel: int, name: str, optional: bool = False):
    """Device pointer of an argument tensor after host checks of its dtype
    (e.g. "int32"), size (at least numel elements), layout and device; the
    C library takes plain pointers and cannot check these itself."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if str(t.dtype) != "torch." + dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")
    return _ptr(t)


def _same(t, ref, name: str):
    """Pointer of a tensor that must have ref's dtype and shape."""
    if t.dtype != ref.dtype or tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} must match {tuple(ref.shape)} {ref.dtype}, got {tuple(t.shape)} {t.dtype}")
    return _ptr(t)


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
    """A zero-filled device workspace of at least nbytes.  Greedy, tree and
    stochastic verification need a zero-filled workspace that no other kind
    of call writes into (they keep it zero-filled between calls); the other
    calls ignore the contents."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


def spec_verify_greedy_workspace_bytes(B: int, k: int, V: int, dtype_code: int) -> int:
    return int(library().spec_verify_greedy_workspace_bytes(B, k, V, dtype_code))


def spec_verify_sample_workspace_bytes(B: int, k: int, V: int) -> int:
    return int(library().spec_verify_sample_workspace_bytes(B, k, V))


def spec_verify_greedy(logits, draft, accept_len, emit_count, out_tokens, ws, *,
                       eos_id: int = -1, remaining=None, emit_offsets=None, status=None,
                       stream=None) -> None:
    """logits [B, k+1, V] (bf16/f32), draft [B, k] int32; outputs int32 tensors."""
    B, kp1, V = logits.shape
    k = kp1 - 1
    code = library().spec_verify_greedy(
        _ptr(logits), _dtype_code(logits), B, k, V, _arg(draft, "int32", B * k, "draft"), int(eos_id),
        _arg(remaining, "int32", B, "remaining", True), _arg(accept_len, "int32", B, "accept_len"),
        _arg(emit_count, "int32", B, "emit_count"), _arg(out_tokens, "int32", B * kp1, "out_tokens"),
        _arg(emit_offsets, "int32", B + 1, "emit_offsets", True), _arg(status, "int32", B, "status", True),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_greedy")


def spec_verify_greedy_noalloc(logits, draft, accept_len, emit_count, out_tokens, *,
                               eos_id: int = -1, remaining=None, emit_offsets=None, status=None,
                               stream=None) -> None:
    """spec_verify_greedy without a workspace: the library's static per-GPU
    array holds the chunk results (calls overlapping on one GPU race)."""
    B, kp1, V = logits.shape
    k = kp1 - 1
    code = library().spec_verify_greedy_noalloc(
        _ptr(logits), _dtype_code(logits), B, k, V, _arg(draft, "int32", B * k, "draft"), int(eos_id),
        _arg(remaining, "int32", B, "remaining", True), _arg(accept_len, "int32", B, "accept_len"),
        _arg(emit_count, "int32", B, "emit_count"), _arg(out_tokens, "int32", B * kp1, "out_tokens"),
        _arg(emit_offsets, "int32", B + 1, "emit_offsets", True), _arg(status, "int32", B, "status", True),
        _stream(stream))
    _check(code, "spec_verify_greedy_noalloc")


def spec_verify_sample(p, q, draft, uniforms, accept_len, emit_count, out_tokens, ws, *,
                       eos_id: int = -1, remaining=None, emit_offsets=None, final_mass=None,
                       status=None, stream=None) -> None:
    """p [B, k+1, V] f32, q [B, k, V] f32, draft [B, k] int32, uniforms [B, k+1] f32."""
    B, kp1, V = p.shape
    k = kp1 - 1
    code = library().spec_verify_sample(
        _arg(p, "float32", B * kp1 * V, "p"), _arg(q, "float32", B * k * V, "q"),
        _arg(draft, "int32", B * k, "draft"), _arg(uniforms, "float32", B * kp1, "uniforms"), B, k, V,
        int(eos_id), _arg(remaining, "int32", B, "remaining", True), _arg(accept_len, "int32", B, "accept_len"),
        _arg(emit_count, "int32", B, "emit_count"), _arg(out_tokens, "int32", B * kp1, "out_tokens"),
        _arg(emit_offsets, "int32", B + 1, "emit_offsets", True),
        _arg(final_mass, "float64", B, "final_mass", True), _arg(status, "int32", B, "status", True),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
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
        _arg(probs, "float32", R * V, "probs", True), _arg(row_max, "float32", R, "row_max", True),
        _arg(row_threshold, "float32", R, "row_threshold", True), _arg(row_mass, "float64", R, "row_mass", True),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_process_logits")


def spec_verify_sample_logits(target_logits, draft_logits, draft, uniforms, accept_len, emit_count,
                              out_tokens, ws, *, temperature: float, top_k: int = 0,
                              top_p: float = 1.0, eos_id: int = -1, remaining=None,
                              emit_offsets=None, final_mass=None, status=None, stream=None) -> None:
    """target_logits [B, k+1, V], draft_logits [B, k, V] (same dtype, bf16/f32)."""
    B, kp1, V = target_logits.shape
    k = kp1 - 1
    if draft_logits.dtype != target_logits.dtype:
        raise ValueError("target and draft logits must share a dtype")
    if tuple(draft_logits.shape) != (B, k, V):
        raise ValueError(f"draft_logits must be {(B, k, V)}, got {tuple(draft_logits.shape)}")
    code = library().spec_verify_sample_logits(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, k, V,
        float(temperature), int(top_k), float(top_p), _arg(draft, "int32", B * k, "draft"),
        _arg(uniforms, "float32", B * kp1, "uniforms"), int(eos_id), _arg(remaining, "int32", B, "remaining", True),
        _arg(accept_len, "int32", B, "accept_len"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(out_tokens, "int32", B * kp1, "out_tokens"), _arg(emit_offsets, "int32", B + 1, "emit_offsets", True),
        _arg(final_mass, "float64", B, "final_mass", True), _arg(status, "int32", B, "status", True),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_sample_logits")


def spec_commit_realign_kv(kv, k: int, end_col, kv_len_in, emit_count, end_col_out, kv_len_out,
                           pos_ids, mask, *, bytes_moved=None, status=None, stream=None) -> None:
    """kv [L, 2, B, H, C, D] (bf16/f32) is realigned in place."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_commit_realign_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(k), _arg(end_col, "int32", 1, "end_col"),
        _arg(kv_len_in, "int32", B, "kv_len_in"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(end_col_out, "int32", 1, "end_col_out"), _arg(kv_len_out, "int32", B, "kv_len_out"),
        _arg(pos_ids, "int32", B * C, "pos_ids"), _arg(mask, "int32", B * C, "mask"),
        _arg(bytes_moved, "int64", 1, "bytes_moved", True), _arg(status, "int32", B, "status", True),
        _stream(stream))
    _check(code, "spec_commit_realign_kv")


def spec_resync_draft_kv(kv, k: int, end_col, kv_len_in, emit_count, end_col_out, kv_len_out, *,
                         pos_ids=None, mask=None, bytes_moved=None, status=None, stream=None) -> None:
    """Draft cache kv [L, 2, B, H, C, D] (bf16/f32) keeps min(e_b, k) of its k forward slots."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_resync_draft_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(k), _arg(end_col, "int32", 1, "end_col"),
        _arg(kv_len_in, "int32", B, "kv_len_in"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(end_col_out, "int32", 1, "end_col_out"), _arg(kv_len_out, "int32", B, "kv_len_out"),
        _arg(pos_ids, "int32", B * C, "pos_ids", True), _arg(mask, "int32", B * C, "mask", True),
        _arg(bytes_moved, "int64", 1, "bytes_moved", True), _arg(status, "int32", B, "status", True),
        _stream(stream))
    _check(code, "spec_resync_draft_kv")


def _ragged_shapes(pool, rect):
    L, two, N, H, Cs, D = pool.shape
    L2, two2, B, H2, C, D2 = rect.shape
    if two != 2 or two2 != 2 or (L, H, D) != (L2, H2, D2) or pool.dtype != rect.dtype:
        raise ValueError(f"pool {tuple(pool.shape)} and rectangle {tuple(rect.shape)} do not match")
    return L, N, H, Cs, D, B, C


def spec_repad_kv(pool, rect, index, kv_len, end_col, *, status=None, stream=None) -> None:
    """pool [L, 2, N, H, Cs, D] (ragged rows at columns 0..n-1), rect
    [L, 2, B, H, C, D]; index, kv_len [B] int32; end_col device int32 [1]."""
    L, N, H, Cs, D, B, C = _ragged_shapes(pool, rect)
    code = library().spec_repad_kv(
        _ptr(pool), _ptr(rect), _dtype_code(pool), L, N, H, Cs, D, B, C, _arg(index, "int32", B, "index"),
        _arg(kv_len, "int32", B, "kv_len"), _arg(end_col, "int32", 1, "end_col"),
        _arg(status, "int32", B, "status", True), _stream(stream))
    _check(code, "spec_repad_kv")


def spec_unpad_kv(rect, pool, index, kv_len, emit_count, end_col, kv_len_out, *, status=None,
                  stream=None) -> None:
    """Copies each member's rows [E - n, E + e) of rect back to pool columns [0, n + e)."""
    L, N, H, Cs, D, B, C = _ragged_shapes(pool, rect)
    code = library().spec_unpad_kv(
        _ptr(rect), _ptr(pool), _dtype_code(pool), L, N, H, Cs, D, B, C, _arg(index, "int32", B, "index"),
        _arg(kv_len, "int32", B, "kv_len"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(end_col, "int32", 1, "end_col"), _arg(kv_len_out, "int32", B, "kv_len_out"),
        _arg(status, "int32", B, "status", True), _stream(stream))
    _check(code, "spec_unpad_kv")


def spec_commit_paged(k: int, page_size: int, kv_len_in, emit_count, block_table, kv_len_out,
                      pages_kept, freed_pages, freed_offsets, *, status=None, stream=None) -> None:
    """block_table [B, max_pages] int32; freed_pages holds B * ceil((k+1)/page_size) ids."""
    B, max_pages = block_table.shape
    per = (int(k) + int(page_size)) // max(int(page_size), 1)
    code = library().spec_commit_paged(
        B, int(k), int(page_size), max_pages, _arg(kv_len_in, "int32", B, "kv_len_in"),
        _arg(emit_count, "int32", B, "emit_count"), _arg(block_table, "int32", B * max_pages, "block_table"),
        _arg(kv_len_out, "int32", B, "kv_len_out"), _arg(pages_kept, "int32", B, "pages_kept"),
        _arg(freed_pages, "int32", B * per, "freed_pages"), _arg(freed_offsets, "int32", B + 1, "freed_offsets"),
        _arg(status, "int32", B, "status", True), _stream(stream))
    _check(code, "spec_commit_paged")


def spec_verify_tree_workspace_bytes(B: int, N: int, V: int, dtype_code: int) -> int:
    return int(library().spec_verify_tree_workspace_bytes(B, N, V, dtype_code))


def spec_verify_tree(logits, draft, first_child, next_sibling, accept_len, emit_count, out_tokens, path,
                     ws, *, eos_id: int = -1, remaining=None, emit_offsets=None, status=None,
                     stream=None) -> None:
    """logits [B, N, V] (bf16/f32); draft, first_child, next_sibling [B, N] int32."""
    B, N, V = logits.shape
    code = library().spec_verify_tree(
        _ptr(logits), _dtype_code(logits), B, N, V, _arg(draft, "int32", B * N, "draft"),
        _arg(first_child, "int32", B * N, "first_child"), _arg(next_sibling, "int32", B * N, "next_sibling"),
        int(eos_id), _arg(remaining, "int32", B, "remaining", True), _arg(accept_len, "int32", B, "accept_len"),
        _arg(emit_count, "int32", B, "emit_count"), _arg(out_tokens, "int32", B * N, "out_tokens"),
        _arg(path, "int32", B * N, "path"), _arg(emit_offsets, "int32", B + 1, "emit_offsets", True),
        _arg(status, "int32", B, "status", True), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_tree")


def spec_verify_tree_sample_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(library().spec_verify_tree_sample_workspace_bytes(B, N, V))


def spec_verify_tree_sample(p, q, draft, first_child, next_sibling, uniforms, accept_len, emit_count,
                            out_tokens, path, ws=None, *, eos_id: int = -1, remaining=None, emit_offsets=None,
                            final_mass=None, status=None, stream=None) -> None:
    """p, q [B, N, V] f32; draft, first_child, next_sibling [B, N] int32; uniforms [B, N] f32;
    ws: None (one workgroup per sequence) or a zero-filled workspace of
    spec_verify_tree_sample_workspace_bytes(B, N, V) bytes."""
    B, N, V = p.shape
    code = library().spec_verify_tree_sample(
        _arg(p, "float32", B * N * V, "p"), _arg(q, "float32", B * N * V, "q"),
        _arg(draft, "int32", B * N, "draft"), _arg(first_child, "int32", B * N, "first_child"),
        _arg(next_sibling, "int32", B * N, "next_sibling"), _arg(uniforms, "float32", B * N, "uniforms"),
        B, N, V, int(eos_id), _arg(remaining, "int32", B, "remaining", True),
        _arg(accept_len, "int32", B, "accept_len"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(out_tokens, "int32", B * N, "out_tokens"), _arg(path, "int32", B * N, "path"),
        _arg(emit_offsets, "int32", B + 1, "emit_offsets", True),
        _arg(final_mass, "float64", B, "final_mass", True), _arg(status, "int32", B, "status", True),
        None if ws is None else _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(code, "spec_verify_tree_sample")


def spec_compact_tree_kv(kv, N: int, end_col, path, emit_count, *, status=None, stream=None) -> None:
    """kv [L, 2, B, H, C, D] (bf16/f32): kept tree slots moved to columns E .. E+e-1 in place."""
    L, two, B, H, C, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [L, 2, B, H, C, D]")
    code = library().spec_compact_tree_kv(
        _ptr(kv), _dtype_code(kv), L, B, H, C, D, int(N), _arg(end_col, "int32", 1, "end_col"),
        _arg(path, "int32", B * int(N), "path"), _arg(emit_count, "int32", B, "emit_count"),
        _arg(status, "int32", B, "status", True), _stream(stream))
    _check(code, "spec_compact_tree_kv")


def spec_group_same_length(lengths, B: int, min_group: int, perm, batch_start, batch_len,
                           num_batches, num_grouped, *, stream=None) -> None:
    """lengths [N] int32; outputs perm [N], batch_start [N+1], batch_len [N], two scalars."""
    N = lengths.numel()
    code = library().spec_group_same_length(
        _arg(lengths, "int32", N, "lengths") if N else None, N, int(B), int(min_group),
        _arg(perm, "int32", N, "perm"), _arg(batch_start, "int32", N + 1, "batch_start"),
        _arg(batch_len, "int32", N, "batch_len"), _arg(num_batches, "int32", 1, "num_batches"),
        _arg(num_grouped, "int32", 1, "num_grouped"), _stream(stream))
    _check(code, "spec_group_same_length")
