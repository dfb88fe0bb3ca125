"""Synthetic KV-cache contents.

A cached key/value row of a real model is a function of the sequence, the
position and the token at that position (plus everything before it).  The
synthetic stand-in is a pure function of (sequence b, position, token,
plane, element d), where plane = (layer * 2 + kv) * H + head.  It is a 32-bit
integer hash (the "lowbias32" mixer published by C. Wellons) mapped to a
finite, nonzero bf16 or f32 bit pattern.  Because the token enters the hash,
a cell holding the KV of a rejected draft differs from the KV of the token
that was finally committed at that position.

Cells outside a sequence's range (left padding, unused capacity) hold the
same hash taken at position KV_PAD_POS + column and token 0.

The numpy and torch versions compute identical bits (checked by a CPU test);
the torch one fills large caches in device memory.

Cache layout everywhere: kv[L][2][B][H][C][D], element bits contiguous in D.
"""
from __future__ import annotations

import numpy as np

M32 = 0xFFFFFFFF
KV_PAD_POS = 0x3FFF0000
_K_TOK, _K_B, _K_PLANE, _K_SEED, _K_D = 0x01000193, 0x9E3779B1, 0x85EBCA77, 0x2545F491, 0x27D4EB2F


# ---------------------------------------------------------------- numpy ----
def _mix32_np(x: np.ndarray) -> np.ndarray:
    x = np.array(x, dtype=np.uint32, ndmin=1, copy=True)
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    return x


def _u32(a) -> np.ndarray:
    return (np.asarray(a, dtype=np.int64) & M32).astype(np.uint32)


def _row_key_np(b, pos, tok, plane) -> np.ndarray:
    with np.errstate(over="ignore"):
        return _row_key_np_(b, pos, tok, plane)


def _row_key_np_(b, pos, tok, plane) -> np.ndarray:
    t = (_u32(tok) * np.uint32(_K_TOK) + _u32(b) * np.uint32(_K_B)
         + _u32(plane) * np.uint32(_K_PLANE) + np.uint32(_K_SEED))
    return _mix32_np(_mix32_np(t) ^ _u32(pos))


def _finish_np(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        bits = ((v >> np.uint32(16)) & np.uint32(0x807F)) | \
               ((((v >> np.uint32(7)) & np.uint32(0x1F)) + np.uint32(0x70)) << np.uint32(7))
        return bits.astype(np.uint16)
    bits = (v & np.uint32(0x807FFFFF)) | \
           ((((v >> np.uint32(23)) & np.uint32(0x1F)) + np.uint32(0x70)) << np.uint32(23))
    return bits.astype(np.uint32)


def kv_bits_np(b, pos, tok, plane, d, dtype: str) -> np.ndarray:
    """Bits of kv element (b, pos, tok, plane, d); all arguments broadcast."""
    key = _row_key_np(b, pos, tok, plane)
    v = key ^ (_u32(d) * np.uint32(_K_D))
    return _finish_np(v, dtype)


def _np_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.uint32


def fill_kv_np(L, H, D, B, C, E, n, tokens, dtype: str, seq=None) -> np.ndarray:
    """Rectangle with sequence b's cached rows 0..n_b-1 at columns [E-n_b, E).

    tokens[b, pos] is the confirmed token at position pos.  E may be one end
    column or one per sequence (E = n gives ragged rows at columns 0..n_b-1).
    seq[b] (default b) is the sequence identity the contents are keyed by.
    Returns element bits (uint16 for bf16, uint32 for f32) of shape
    [L, 2, B, H, C, D].
    """
    n = np.asarray(n, dtype=np.int64)
    Eb = np.broadcast_to(np.asarray(E, dtype=np.int64), n.shape)
    col = np.arange(C, dtype=np.int64)[None, :]
    pos = col - (Eb[:, None] - n[:, None])             # [B, C]
    valid = (pos >= 0) & (pos < n[:, None])
    tok = np.where(valid, np.take_along_axis(tokens, np.clip(pos, 0, tokens.shape[1] - 1), 1), 0)
    pos = np.where(valid, pos, KV_PAD_POS + col)
    out = np.empty((L, 2, B, H, C, D), dtype=_np_dtype(dtype))
    d = np.arange(D, dtype=np.int64)
    bidx = (np.arange(B, dtype=np.int64) if seq is None else np.asarray(seq, np.int64))[:, None, None]
    for l in range(L):
        for kv in range(2):
            plane = ((l * 2 + kv) * H + np.arange(H, dtype=np.int64))[None, :, None]
            key = _row_key_np(bidx, pos[:, None, :], tok[:, None, :], plane)      # [B, H, C]
            out[l, kv] = _finish_np(key[..., None] ^ (_u32(d) * np.uint32(_K_D)), dtype)
    return out


def write_forward_slots_np(kv: np.ndarray, E: int, n, slot_tokens, dtype: str) -> None:
    """Write the verify forward's k+1 rows at columns E..E+k.

    slot_tokens[b, j] is the token whose KV lands in slot j: the last confirmed
    token for j = 0, draft j-1 for j >= 1.  Slot j holds position n_b + j.
    """
    L, _, B, H, C, D = kv.shape
    n = np.asarray(n, dtype=np.int64)
    kp1 = slot_tokens.shape[1]
    pos = n[:, None] + np.arange(kp1, dtype=np.int64)[None, :]            # [B, k+1]
    d = np.arange(D, dtype=np.int64)
    bidx = np.arange(B, dtype=np.int64)[:, None, None]
    for l in range(L):
        for kvi in range(2):
            plane = ((l * 2 + kvi) * H + np.arange(H, dtype=np.int64))[None, :, None]
            key = _row_key_np(bidx, pos[:, None, :], np.asarray(slot_tokens)[:, None, :], plane)
            kv[l, kvi, :, :, E:E + kp1, :] = _finish_np(key[..., None] ^ (_u32(d) * np.uint32(_K_D)), dtype)


# ---------------------------------------------------------------- torch ----
def _mul32_t(x, c: int):
    """(x * c) mod 2**32 for int64 tensors x in [0, 2**32), without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + ((x * hi) & 0xFFFF) * 65536) & M32


def _mix32_t(x):
    x = x ^ (x >> 16)
    x = _mul32_t(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32_t(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _row_key_t(b, pos, tok, plane):
    t = (_mul32_t(tok & M32, _K_TOK) + _mul32_t(b & M32, _K_B)
         + _mul32_t(plane & M32, _K_PLANE) + _K_SEED) & M32
    return _mix32_t(_mix32_t(t) ^ (pos & M32))


def _finish_t(v, dtype: str):
    import torch
    if dtype == "bf16":
        bits = ((v >> 16) & 0x807F) | ((((v >> 7) & 0x1F) + 0x70) << 7)
        return (bits - ((bits >> 15) & 1) * 65536).to(torch.int16)
    bits = (v & 0x807FFFFF) | ((((v >> 23) & 0x1F) + 0x70) << 23)
    return (bits - ((bits >> 31) & 1) * (1 << 32)).to(torch.int32)


def kv_bits_torch(b, pos, tok, plane, d, dtype: str):
    """Same bits as kv_bits_np, as a signed int16/int32 tensor."""
    key = _row_key_t(b, pos, tok, plane)
    return _finish_t(key ^ _mul32_t(d & M32, _K_D), dtype)


def _int_view(kv):
    import torch
    return kv.view(torch.int16) if kv.element_size() == 2 else kv.view(torch.int32)


def fill_kv_torch(kv, E, n, tokens, dtype: str, seq=None) -> None:
    """Device version of fill_kv_np, writing into kv [L, 2, B, H, C, D] in place.

    tokens: int64 tensor [B, T] on kv's device; E and seq as in fill_kv_np.
    """
    import torch
    L, _, B, H, C, D = kv.shape
    dev = kv.device
    n_np = np.asarray(n, dtype=np.int64)
    n_t = torch.as_tensor(n_np, device=dev)
    E_t = torch.as_tensor(np.broadcast_to(np.asarray(E, dtype=np.int64), n_np.shape).copy(), device=dev)
    col = torch.arange(C, device=dev, dtype=torch.int64)[None, :]
    pos = col - (E_t[:, None] - n_t[:, None])
    valid = (pos >= 0) & (pos < n_t[:, None])
    tok = torch.where(valid, torch.gather(tokens, 1, pos.clamp(0, tokens.shape[1] - 1)),
                      torch.zeros_like(pos))
    pos = torch.where(valid, pos, KV_PAD_POS + col)
    d = torch.arange(D, device=dev, dtype=torch.int64)
    dterm = _mul32_t(d, _K_D)
    bidx = (torch.arange(B, device=dev, dtype=torch.int64) if seq is None
            else torch.as_tensor(np.asarray(seq, np.int64), device=dev))[:, None, None]
    iv = _int_view(kv)
    for l in range(L):
        for kvi in range(2):
            plane = ((l * 2 + kvi) * H + torch.arange(H, device=dev, dtype=torch.int64))[None, :, None]
            key = _row_key_t(bidx, pos[:, None, :], tok[:, None, :], plane)       # [B, H, C]
            iv[l, kvi].copy_(_finish_t(key[..., None] ^ dterm, dtype))
            del key


def write_forward_slots_torch(kv, E: int, n, slot_tokens, dtype: str) -> None:
    """Device version of write_forward_slots_np (slot_tokens: int64 tensor [B, k+1])."""
    import torch
    L, _, B, H, C, D = kv.shape
    dev = kv.device
    n_t = torch.as_tensor(np.asarray(n, dtype=np.int64), device=dev)
    kp1 = slot_tokens.shape[1]
    pos = n_t[:, None] + torch.arange(kp1, device=dev, dtype=torch.int64)[None, :]
    d = torch.arange(D, device=dev, dtype=torch.int64)
    dterm = _mul32_t(d, _K_D)
    bidx = torch.arange(B, device=dev, dtype=torch.int64)[:, None, None]
    iv = _int_view(kv)
    for l in range(L):
        for kvi in range(2):
            plane = ((l * 2 + kvi) * H + torch.arange(H, device=dev, dtype=torch.int64))[None, :, None]
            key = _row_key_t(bidx, pos[:, None, :], slot_tokens[:, None, :], plane)
            iv[l, kvi, :, :, E:E + kp1, :].copy_(_finish_t(key[..., None] ^ dterm, dtype))


# ------------------------------------------------------- chosen rows ----
def write_rows_np(kv: np.ndarray, rows, seq, col0, pos0, tokens, dtype: str) -> None:
    """For each i: the KV of sequence seq[i] at positions pos0[i] + t for the
    tokens tokens[i, t] (t < T), written into row rows[i] of kv [L, 2, R, H,
    C, D] at columns col0[i] + t.  Used for verify-forward slots of chosen
    sequences of a pool or a rectangle."""
    L, _, R, H, C, D = kv.shape
    tokens = np.asarray(tokens, np.int64)
    T = tokens.shape[1]
    d = np.arange(D, dtype=np.int64)
    plane = np.arange(L * 2 * H, dtype=np.int64).reshape(L, 2, H)[:, :, :, None, None]
    for i in range(len(rows)):
        pos = (int(pos0[i]) + np.arange(T, dtype=np.int64))[None, None, None, :, None]
        key = _row_key_np(int(seq[i]), pos, tokens[i][None, None, None, :, None], plane)
        c0 = int(col0[i])
        kv[:, :, int(rows[i]), :, c0:c0 + T, :] = _finish_np(key ^ (_u32(d) * np.uint32(_K_D)), dtype)


def write_rows_torch(kv, rows, seq, col0, pos0, tokens, dtype: str) -> None:
    """Device version of write_rows_np (tokens: int64 array [R', T])."""
    import torch
    L, _, R, H, C, D = kv.shape
    dev = kv.device
    tokens = np.asarray(tokens, np.int64)
    T = tokens.shape[1]
    dterm = _mul32_t(torch.arange(D, device=dev, dtype=torch.int64), _K_D)
    plane = torch.arange(L * 2 * H, device=dev, dtype=torch.int64).reshape(L, 2, H)[:, :, :, None, None]
    iv = _int_view(kv)
    tok_t = torch.as_tensor(tokens, device=dev)
    for i in range(len(rows)):
        pos = (int(pos0[i]) + torch.arange(T, device=dev, dtype=torch.int64))[None, None, None, :, None]
        key = _row_key_t(torch.full((1,), int(seq[i]), device=dev, dtype=torch.int64), pos,
                         tok_t[i][None, None, None, :, None], plane)
        c0 = int(col0[i])
        iv[:, :, int(rows[i]), :, c0:c0 + T, :].copy_(_finish_t(key ^ dterm, dtype))
