"""GPU parity of the processed-distribution calls (temperature, top-k, top-p)
against the oracle.

Tolerances, from the arithmetic stated in include/spec_verify.h.  A GPU
weight is the accurate float32 expf of (z - max z) / T with the argument's
rounding error folded back in (relative error <= 2^-23 + 2^-24); the kept
weight is an exact sum of weights truncated to 2^-40 (error <= V * 2^-40,
and the kept weight is at least 1); 1 / mass and p' = w * (1 / mass) are each
rounded once.  So a kept probability p' agrees with the oracle's float64 value
to a relative

    E_P(V) = 2 (2^-23 + 2^-24) + 2 * 2^-24 + V * 2^-40   (4.8e-7 + 9.1e-13 V),

checked against RTOL = 1e-5; the row maximum is exact; a kept set is exact
except that a top-p boundary may move where the oracle, run with top_p -/+
1e-5, brackets the GPU's threshold.  Verification: a = min(1, p'(x) / q'(x))
differs by at most ACCEPT(V) = 2 E_P(V) + 2^-24 (1.0e-6 + 1.8e-12 V: the
the benchmark spec's 1e-6, widened by the kept-weight truncation), so a decision may
differ only where |u - a| < ACCEPT(V); the residual mass S = sum max(p' - q', 0)
and every prefix sum of the drawn row differ by at most 2 E_P(V) absolute, so
S must agree to 1e-5 * S + 2 E_P(V) and a drawn token may differ only where
u * S lies within that distance of a prefix boundary.  Decisions near the
boundary occur with probability about ACCEPT(V) per decision (none expected
in these cases, so none is allowed); a draw differs with probability about
4 E_P(V) / p'(token) per draw, so at most one per case is allowed.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_04_amd as sv

import oracle
import workloads as W
from oracle.process import process_row
from tests._gpu import DEV, _WS, host, logits_to_device, note, process, requires_gpu, verify_sample_logits

pytestmark = [pytest.mark.gpu, requires_gpu]

RTOL = 1e-5
PTOL = 1e-5


def e_p(V: int) -> float:
    """Relative bound on a GPU p' against the oracle's (module docstring)."""
    return 2 * (2.0 ** -23 + 2.0 ** -24) + 2 * 2.0 ** -24 + V * 2.0 ** -40


def accept_allowance(V: int) -> float:
    return 2 * e_p(V) + 2.0 ** -24


def _rows(rng, R, V, dtype, sd=3.0, ties=False):
    z = (rng.standard_normal((R, V)) * sd).astype(np.float32)
    if ties:
        z = np.round(z * 2) / 2
    if dtype == "bf16":
        bits = W.bf16_bits_from_f32(z)
        return bits, oracle.widen_bf16(bits)
    return z, z


def _check_rows(zw, got, T, K, P):
    """zw: the oracle's view of the logits [R, V]; got: host outputs of process()."""
    R, V = zw.shape
    for r in range(R):
        p, info = process_row(zw[r], T, K, P)
        assert got["row_max"][r] == np.float32(info["zmax"]), r
        thr_g = float(got["row_threshold"][r])
        if thr_g != info["threshold"]:
            assert P < 1.0, (r, thr_g, info["threshold"])
            hi = process_row(zw[r], T, K, max(P - PTOL, 1e-6))[1]["threshold"]
            lo = process_row(zw[r], T, K, min(P + PTOL, 1.0))[1]["threshold"]
            assert lo <= thr_g <= hi, (r, thr_g, info["threshold"], lo, hi)
            continue
        g = got["probs"][r]
        kept = info["kept"]
        assert np.all(g[~kept] == 0.0), r
        o = p.astype(np.float64)
        assert np.all(np.abs(g[kept] - o[kept]) <= RTOL * o[kept] + 1e-37), r
        if info["mass"] > 0:
            assert abs(got["row_mass"][r] - info["mass"]) <= RTOL * info["mass"], r
        else:
            assert got["row_mass"][r] == 0.0


CASES = [(1.0, 0, 1.0), (0.7, 0, 1.0), (0.7, 50, 1.0), (0.7, 0, 0.9), (0.7, 50, 0.9), (1.3, 1, 1.0),
         (0.5, 0, 0.5), (2.0, 1000, 0.95), (0.05, 0, 0.99), (1.0, 3, 0.3)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 1000, 4097, 32001])
def test_process_rows_parity(dtype, V):
    rng = np.random.default_rng(V + (7 if dtype == "bf16" else 0))
    dev_in, zw = _rows(rng, 4, V, dtype)
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in CASES:
        note(f"process {dtype} V={V} T={T} K={K} P={P}")
        got = host(process(zd, T, K, P))
        _check_rows(zw, got, T, K, P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_process_ties_and_special_rows(dtype):
    rng = np.random.default_rng(11)
    dev_in, zw = _rows(rng, 6, 3001, dtype, sd=2.0, ties=True)     # many exact ties
    if dtype == "f32":
        dev_in[2] = -np.inf                                         # a row without mass
        dev_in[3, ::3] = -np.inf                                    # masked entries
        zw = dev_in
    else:
        dev_in[2] = 0xFF80                                          # bf16 -inf
        dev_in[3, ::3] = 0xFF80
        zw = oracle.widen_bf16(dev_in)
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in CASES + [(1.0, 3001, 1.0), (1.0, 5000, 0.5), (0.9, 2, 0.999)]:
        note(f"process ties {dtype} T={T} K={K} P={P}")
        got = host(process(zd, T, K, P))
        _check_rows(zw, got, T, K, P)
    got = host(process(zd, 1.0, 7, 0.5))
    assert np.all(got["probs"][2] == 0.0) and got["row_mass"][2] == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_process_topk_crowded_rows(dtype):
    """Rows whose top bucket holds far more than K entries (all equal, a narrow
    spread, half -inf): the per-slice candidate lists overflow and the row is
    read whole; K near and above the list path's limit."""
    rng = np.random.default_rng(13)
    V = 60000
    z = np.zeros((4, V), np.float32)
    z[1] = rng.standard_normal(V).astype(np.float32) * 0.01
    z[2, ::2] = -np.inf
    z[2, 1::2] = 1.5
    z[3] = rng.standard_normal(V).astype(np.float32) * 3.0
    if dtype == "bf16":
        dev_in = W.bf16_bits_from_f32(z)
        zw = oracle.widen_bf16(dev_in)
    else:
        dev_in, zw = z, z
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in [(1.0, 50, 1.0), (0.7, 50, 0.9), (1.0, 1024, 0.95), (1.0, 1025, 1.0), (0.8, 4000, 0.9),
                    (1.0, 0, 0.9), (0.7, 0, 1.0), (2.0, 0, 0.3)]:
        note(f"process crowded {dtype} T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_process_topk_concentrated_rows(dtype):
    """Rows whose largest logits sit in one slice (the first, the short last
    one, or two of them): the slices' lower bounds of the K-th largest are far
    apart, and the candidates the statistics keep must still hold every logit
    at or above the row's K-th largest."""
    rng = np.random.default_rng(15)
    V = 100003
    sl = 16384 if dtype == "bf16" else 8192
    S = (V + sl - 1) // sl
    z = (rng.standard_normal((5, V)) * 1.0).astype(np.float32)
    hot = [(0, 0), (1, S - 1), (2, 1), (2, S // 2), (3, S // 2)]
    for r, s in hot:
        lo = s * sl
        n = min(400, V - lo)
        z[r, lo:lo + n] = (8.0 + rng.standard_normal(n)).astype(np.float32)
    z[4, :] = np.float32(-3.0)
    z[4, rng.choice(V, 300, replace=False)] = (6.0 + rng.standard_normal(300)).astype(np.float32)
    if dtype == "bf16":
        dev_in = W.bf16_bits_from_f32(z)
        zw = oracle.widen_bf16(dev_in)
    else:
        dev_in, zw = z, z
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in [(1.0, 1, 1.0), (0.7, 7, 1.0), (0.7, 50, 0.9), (1.0, 200, 1.0), (0.9, 256, 0.95),
                    (0.9, 257, 0.95), (1.0, 64, 0.5)]:           # 256: largest slice-path K; 257: whole rows
        note(f"process concentrated {dtype} T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)


@pytest.mark.parametrize("dtype,V", [("bf16", 393216), ("bf16", 393217), ("f32", 196608), ("f32", 196609)])
def test_process_topk_slice_count_boundary(dtype, V):
    """Rows of 24 slices (one wave gathers the lists) and of 25 (the workgroup
    path), with K such that some lists hold about 64 entries."""
    rng = np.random.default_rng(16)
    dev_in, zw = _rows(rng, 3, V, dtype, sd=2.0)
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in [(0.7, 50, 0.9), (1.0, 60, 1.0), (1.0, 200, 0.95)]:
        note(f"process slice-count boundary {dtype} V={V} T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)


def test_process_misaligned_rows():
    rng = np.random.default_rng(12)
    V = 1001                                                        # odd: bf16 rows start misaligned
    bits, zw = _rows(rng, 5, V, "bf16")
    buf = torch.empty(bits.size + 1, dtype=torch.int16, device=DEV)
    buf[1:].copy_(torch.from_numpy(bits.view(np.int16).reshape(-1)).to(DEV))
    zd = buf[1:].view(torch.bfloat16).view(5, V)
    for T, K, P in [(0.8, 20, 0.8), (0.8, 0, 0.8), (1.0, 0, 1.0)]:
        note(f"process misaligned bf16 T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K,P", [(0.7, 50, 0.9), (0.7, 0, 0.9)])
def test_process_workload_rows_full_size(dtype, T, K, P):
    """Stochastic workload shapes: V = 151936, temperature 0.7."""
    g = W.sample_logits(2)
    z = g["zt"].reshape(-1, g["V"])[[0, 9, 17, 30]]
    if dtype == "bf16":
        bits = W.bf16_bits_from_f32(z)
        dev_in, zw = bits, oracle.widen_bf16(bits)
    else:
        dev_in, zw = z, z
    note(f"process workload rows {dtype} T={T} K={K} P={P}")
    got = host(process(logits_to_device(dev_in, dtype), T, K, P))
    _check_rows(zw, got, T, K, P)


def _check_verify(p, q, d, u, got, ref):
    """Verification outputs on processed rows p, q (the oracle's).  Returns
    counts: exact (identical outputs), accept_tol (a decision differing inside
    ACCEPT(V)), draw_tol (a draw differing inside the window), draws."""
    B, kp1, V = p.shape
    k = kp1 - 1
    A = accept_allowance(V)
    D = 2 * e_p(V)
    c = dict(exact=0, accept_tol=0, draw_tol=0, draws=0)
    for b in range(B):
        mr, mg = int(ref["accept_len"][b]), int(got["accept_len"][b])
        if mr != mg:
            j = min(mr, mg)
            x = int(d[b, j])
            a = min(1.0, float(p[b, j, x]) / float(q[b, j, x])) if q[b, j, x] > 0 else float(p[b, j, x] > 0)
            assert abs(float(u[b, j]) - a) < A, (b, j, u[b, j], a)
            c["accept_tol"] += 1
            continue
        assert got["emit_count"][b] == ref["emit_count"][b], b
        assert got["status"][b] == ref["status"][b], b
        e = int(ref["emit_count"][b])
        assert np.array_equal(got["out_tokens"][b, :mr], ref["out_tokens"][b, :mr])
        assert (got["out_tokens"][b, e:] == -1).all()
        Sr, Sg = float(ref["final_mass"][b]), float(got["final_mass"][b])
        if e == mr:
            assert Sg == 0.0 and Sr == 0.0
            c["exact"] += 1
            continue
        c["draws"] += 1
        w = 1e-5 * abs(Sr) + D
        assert abs(Sg - Sr) <= w, (b, Sg, Sr)
        vg, vr = int(got["out_tokens"][b, e - 1]), int(ref["out_tokens"][b, e - 1])
        if vg == vr:
            c["exact"] += 1
            continue
        row = np.maximum(p[b, mr] - q[b, mr], 0) if mr < k else p[b, k]
        if mr < k and ref["status"][b] & oracle.ST_RESID_ZERO:
            row = p[b, mr]
        C = np.cumsum(row.astype(np.float64))
        Tt = float(u[b, k]) * Sr
        lo = C[vg - 1] if vg > 0 else 0.0
        assert row[vg] > 0 and lo - w <= Tt <= C[vg] + w, (b, vg, vr)
        c["draw_tol"] += 1
    return c


def _assert_counts(c, B):
    assert c["accept_tol"] == 0, c
    assert c["draw_tol"] <= 1, c
    assert c["exact"] + c["draw_tol"] == B, c


def _verify_case(zt, zd_, T, K, P, seed, dtype):
    """Drafts are drawn from the oracle's q' (drafting is outside the step)."""
    B, kp1, V = zt.shape
    k = kp1 - 1
    if dtype == "bf16":
        bt, bd = W.bf16_bits_from_f32(zt), W.bf16_bits_from_f32(zd_)
        zt_w, zd_w = oracle.widen_bf16(bt), oracle.widen_bf16(bd)
        dev_t, dev_d = logits_to_device(bt, "bf16"), logits_to_device(bd, "bf16")
    else:
        zt_w, zd_w = zt, zd_
        dev_t, dev_d = logits_to_device(zt, "f32"), logits_to_device(zd_, "f32")
    p, _ = oracle.process_rows(zt_w, T, K, P)
    q, _ = oracle.process_rows(zd_w, T, K, P)
    rng = np.random.default_rng(seed)
    d = W.draw_inverse_cdf(q, rng.random((B, k)))
    u = rng.random((B, kp1), dtype=np.float32)
    got = host(verify_sample_logits(dev_t, dev_d, d, u, T, K, P))
    ref = oracle.sample_verify(p, q, d, u)
    return _check_verify(p, q, d, u, got, ref), got, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [5, 1000, 4097])
def test_verify_from_logits_parity(dtype, V):
    rng = np.random.default_rng(100 + V)
    B, k = 24, 3
    zt = (rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32)
    zd_ = (zt[:, :k] + rng.standard_normal((B, k, V)) * 0.7).astype(np.float32)
    for T, K, P in [(1.0, 0, 1.0), (0.7, 20, 0.9), (1.5, 0, 0.8), (0.6, 3, 1.0)]:
        note(f"verify logits {dtype} V={V} T={T} K={K} P={P}")
        counts, got, ref = _verify_case(zt, zd_, T, K, P, V, dtype)
        _assert_counts(counts, B)
        assert got["emit_offsets"][-1] == got["emit_count"].sum()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [50, 0])
def test_verify_from_logits_workload_full_size(dtype, K):
    """Stochastic workload: B=8, k=4, V=151936, T=0.7, top-p 0.9, with top-k
    50 and without (rows then keep several hundred entries: the draw orders
    them slice by slice)."""
    g = W.sample_logits(2)
    note(f"verify logits workload {dtype} K={K}")
    counts, got, ref = _verify_case(g["zt"], g["zd"], g["temperature"], K, 0.9, 2, dtype)
    _assert_counts(counts, 8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_from_logits_crowded_and_tied_rows(dtype):
    """Top-k rows whose kept entries are not a short list: every logit equal
    (the slice lists overflow), 2000 logits tied at the top (the lists hold
    them, but more than one per lane of the drawing workgroup), half -inf and
    half equal, a narrow spread; beside ordinary rows and a target row of
    -inf only (no mass: the draw gives token 0 with SPEC_ST_RESID_ZERO).
    The draws then come from the whole rows instead of the lists."""
    rng = np.random.default_rng(61)
    B, k, V = 6, 2, 60000
    zt = (rng.standard_normal((B, k + 1, V)) * 1.0).astype(np.float32)
    zt[0] = 0.0
    top = rng.choice(V, 2000, replace=False)
    zt[1] *= 0.5
    zt[1][:, top] = 5.0
    zt[2][:, ::2] = -np.inf
    zt[2][:, 1::2] = 1.5
    zt[3] *= 3.0
    zt[4] *= 0.01
    zt[5, 0] = -np.inf
    zd_ = (zt[:, :k] + rng.standard_normal((B, k, V)) * 0.3).astype(np.float32)
    zd_[2] = np.where(np.isinf(zt[2, :k]), -np.inf, 1.5).astype(np.float32)
    zd_[2][:, rng.choice(np.arange(1, V, 2), 100, replace=False)] = 2.0
    # K = 256 without top-p keeps 256 entries of an ordinary row (more with
    # bf16 ties): the largest kept sets drawn from the lists
    for T, K, P in [(1.0, 50, 1.0), (0.7, 50, 0.9), (1.0, 256, 0.95), (1.0, 256, 1.0), (1.0, 0, 0.9), (0.7, 0, 0.5)]:
        note(f"verify logits crowded {dtype} T={T} K={K} P={P}")
        counts, got, ref = _verify_case(zt, zd_, T, K, P, 62, dtype)
        _assert_counts(counts, B)
        assert got["emit_offsets"][-1] == got["emit_count"].sum()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_from_logits_largest_vocabulary(dtype):
    """V = SPEC_PROC_MAX_V with top-k: the most slices per row (64 for f32,
    more than the drawing workgroup has waves) and the smallest lists."""
    rng = np.random.default_rng(524)
    B, k, V = 2, 1, sv.SPEC_PROC_MAX_V
    zt = (rng.standard_normal((B, k + 1, V)) * 2.0).astype(np.float32)
    zd_ = (zt[:, :k] + rng.standard_normal((B, k, V)) * 0.7).astype(np.float32)
    for T, K, P in [(0.7, 50, 0.9), (1.0, 200, 1.0), (0.7, 0, 0.9)]:
        note(f"verify logits largest V {dtype} T={T} K={K} P={P}")
        counts, got, ref = _verify_case(zt, zd_, T, K, P, 63, dtype)
        _assert_counts(counts, B)


def test_verify_from_logits_output_law():
    """The emitted token follows p' (drafts weighted by q', stratified grids)."""
    zt1 = np.log(np.array([0.5, 0.3, 0.15, 0.05])).astype(np.float32)
    zd1 = np.log(np.array([0.1, 0.2, 0.3, 0.4])).astype(np.float32)
    T, K, P = 0.8, 3, 0.95
    p1, _ = process_row(zt1, T, K, P)
    q1, _ = process_row(zd1, T, K, P)
    N = 200
    grid = np.array([(i + 0.5) / N for i in range(N)], np.float32)
    xs = [x for x in range(4) if q1[x] > 0]
    X, A, D = np.meshgrid(np.array(xs), grid, grid, indexing="ij")
    d = X.reshape(-1, 1).astype(np.int32)
    u = np.stack([A.reshape(-1), D.reshape(-1)], axis=1).astype(np.float32)
    wts = q1[d[:, 0]].astype(np.float64) / (N * N)
    B = d.shape[0]
    zt = np.broadcast_to(zt1, (B, 2, 4)).copy()
    zd_ = np.broadcast_to(zd1, (B, 1, 4)).copy()
    note(f"verify logits output law B={B}")
    got = host(verify_sample_logits(logits_to_device(zt, "f32"), logits_to_device(zd_, "f32"), d, u, T, K, P))
    law = np.bincount(got["out_tokens"][:, 0], weights=wts, minlength=4)
    assert np.allclose(law, p1, atol=2e-3)


def test_verify_from_logits_repeatable():
    g = W.sample_logits(2, round_=3, B=4)
    zt = logits_to_device(g["zt"], "f32")
    zd_ = logits_to_device(g["zd"], "f32")
    rng = np.random.default_rng(3)
    d = rng.integers(0, g["V"], size=(4, g["k"])).astype(np.int32)
    note("verify logits repeatable")
    first = host(verify_sample_logits(zt, zd_, d, g["uniforms"], 0.7, 40, 0.9, ws_key="vl"))
    # the leading part (row statistics, candidate lists) is rewritten by
    # every call, whatever it holds; the trailing completion flags are left
    # zero-filled by every call
    B, k, V = 4, g["k"], g["V"]
    flags = sv.spec_verify_sample_workspace_bytes(B, k, V)
    lead = sv.spec_verify_sample_logits_workspace_bytes(B, k, V) - flags
    w = _WS[("sample_logits", "vl")]
    for it in range(6):
        w[:lead].fill_(0x5A)
        again = host(verify_sample_logits(zt, zd_, d, g["uniforms"], 0.7, 40, 0.9, ws_key="vl"))
        for key in first:
            assert np.array_equal(first[key], again[key]), key
        assert int(torch.count_nonzero(w[lead:lead + flags]).item()) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_process_largest_vocabulary(dtype):
    """V = SPEC_PROC_MAX_V: the most slices per row (64 for f32), the smallest
    per-slice list capacity, and the union path for top-p alone."""
    rng = np.random.default_rng(14)
    V = sv.SPEC_PROC_MAX_V
    dev_in, zw = _rows(rng, 3, V, dtype, sd=3.0)
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in [(0.7, 50, 0.9), (1.0, 128, 1.0), (0.7, 0, 0.9), (1.0, 0, 1.0), (0.7, 300, 0.95)]:
        note(f"process largest V {dtype} T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_from_logits_largest_k(dtype):
    """k = SPEC_MAX_K (127) through the processed path: draft logits close to
    the target's keep most drafts accepted, so the chains run long."""
    k = sv.SPEC_MAX_K
    rng = np.random.default_rng(1270)
    B, V = 3, 300
    zt = (rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32)
    zd_ = zt[:, :k].copy()
    zd_[1] += (rng.standard_normal((k, V)) * 0.05).astype(np.float32)
    zd_[2] += (rng.standard_normal((k, V)) * 0.5).astype(np.float32)
    note(f"verify logits k={k} {dtype}")
    counts, got, ref = _verify_case(zt, zd_, 0.8, 10, 0.9, 7, dtype)
    assert ref["accept_len"][0] == k                  # identical p' and q': every draft accepted
    _assert_counts(counts, B)
    assert got["emit_offsets"][-1] == got["emit_count"].sum()


@pytest.mark.parametrize("dtype,V", [("bf16", 256000), ("f32", 256000), ("bf16", 524288)])
def test_process_whole_row_histograms_of_long_rows(dtype, V):
    """Rows long enough that one lane column of the whole-row histogram
    receives thousands of logits (about V/64), most of them in a few buckets
    of the top digit: large top-k (the row path) and top-p with most of the
    weight spread over the row (the slices' union carries too little of it).
    N(0, 1) logits at T = 1 put about 4% of a row in one bucket."""
    rng = np.random.default_rng(V % 1000 + (1 if dtype == "bf16" else 0))
    dev_in, zw = _rows(rng, 3, V, dtype, sd=1.0)
    zd = logits_to_device(dev_in, dtype)
    for T, K, P in [(1.0, 10000, 1.0), (1.0, 0, 0.5), (1.0, 10000, 0.5), (1.0, 0, 0.9), (0.8, 40000, 0.97)]:
        note(f"process long rows {dtype} V={V} T={T} K={K} P={P}")
        _check_rows(zw, host(process(zd, T, K, P)), T, K, P)
