"""Helpers shared by the GPU parity tests (input plumbing and comparison rules).

Nothing here computes any step of the method: the HIP library is called
through its binding, the oracle through its own module, and this file only
moves arrays between them and applies the parity rules:

* block selections: rows whose oracle margin between the (k-1)-th and k-th
  best non-local block exceeds 1e-3 (relative) must match exactly; the other
  rows must be admissible -- same size, local block present, and every block in
  the symmetric difference within 1e-3 (relative) of the selection boundary;
* outputs (bf16): max |diff| <= 2e-2 and mean |diff| <= 2e-3; fp8 inputs:
  max |diff| <= 6e-2.
"""
from __future__ import annotations

import sys

import numpy as np

import block_sparse_attention_idx_amd as msa
import oracle
import synth

MARGIN = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dims_of(w: synth.Workload):
    return msa.make_dims(w.batch, w.N, w.H_q, w.H_kv, w.d_h, w.d_idx, w.B_k, w.k, H_idx=w.H_idx)


def opts_of(w: synth.Workload, **kw):
    if w.dtype == "fp8":
        s = synth.fp8_scale()
        return msa.make_opts("fp8", q_scale=s, k_scale=s, v_scale=s, q_chunk=w.q_chunk, **kw)
    return msa.make_opts("bf16", q_chunk=w.q_chunk, **kw)


def device_inputs(w: synth.Workload, dev):
    return {x: synth.device_tensor(w, x, dev) for x in ("q", "k", "v", "q_idx", "k_idx")}


def oracle_index_rows(w: synth.Workload, rows: np.ndarray, bat: int = 0):
    """Oracle selection for query rows of batch element `bat`."""
    flat = bat * w.N + rows
    q_idx = synth.host_rows(w, "q_idx", flat)
    k_idx = synth.host_rows(w, "k_idx", bat * w.N + np.arange(w.N))
    return oracle.index_topk(w.N, w.B_k, w.k, rows, q_idx, k_idx)


def admissible(gsel, osel, Mrow, k) -> bool:
    g = set(int(x) for x in gsel if x >= 0)
    o = set(int(x) for x in osel if x >= 0)
    if len(g) != len(o) or max(o) not in g:
        return False
    # blocks forced by a +inf score besides the local one leave k - 1 - forced
    # free choices among the finite scores
    free = k - 1 - (int(np.sum(Mrow == np.inf)) - 1)
    cand = np.sort(Mrow[np.isfinite(Mrow)])[::-1]
    if len(cand) <= free or free < 1:
        return g == o
    ck1, ck = float(cand[free - 1]), float(cand[free])
    tol = MARGIN * max(abs(ck1), abs(ck), 1e-6)
    return (all(Mrow[b] >= ck1 - tol for b in g - o) and
            all(Mrow[b] <= ck + tol for b in o - g))


def check_selection(gpu, orc, marg, M, k, what=""):
    """gpu, orc: [H_sel, n, k]; marg: [H_sel, n]; M: [n, H_sel, B].  Returns stats."""
    sure = marg > MARGIN
    exact_ok = np.array_equal(gpu[sure], orc[sure])
    if not exact_ok:
        bad = np.argwhere(sure & ~(gpu == orc).all(axis=2))
        r, i = bad[0]
        raise AssertionError(f"{what}: selection differs on a clear-margin row (group {r}, row {i}): "
                             f"gpu {gpu[r, i].tolist()} oracle {orc[r, i].tolist()} "
                             f"margin {marg[r, i]:.3g} ({len(bad)} rows)")
    near = np.argwhere(~sure)
    n_diff = 0
    for r, i in near:
        if not np.array_equal(gpu[r, i], orc[r, i]):
            n_diff += 1
            assert admissible(gpu[r, i], orc[r, i], M[i, r], k), (
                f"{what}: inadmissible selection (group {r}, row {i}): gpu {gpu[r, i].tolist()} "
                f"oracle {orc[r, i].tolist()}")
    return {"rows": int(sure.size), "clear": int(sure.sum()), "near_tie": int((~sure).sum()),
            "near_tie_differing": n_diff}


def err_stats(got, ref, label=None):
    """max |diff| and mean |diff|; with a label, also log the cosine
    similarity and the relative L2 error ||got - ref|| / ||ref||."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    d = np.abs(g - r)
    mx, mn = float(d.max()), float(d.mean())
    if label is not None:
        nr, ng = float(np.linalg.norm(r)), float(np.linalg.norm(g))
        cos = float((g * r).sum() / max(nr * ng, 1e-300))
        rel = float(np.linalg.norm(g - r) / max(nr, 1e-300))
        log(f"  {label}: max |diff| {mx:.3g}  mean |diff| {mn:.3g}  cos-sim {cos:.8f}  rel L2 {rel:.3g}")
    return mx, mn


def compact_attention_rows(w: synth.Workload, rows: np.ndarray, sel: np.ndarray, bat: int = 0):
    """Oracle attention for a few query rows of a long sequence without
    regenerating all of K and V: for each row, the union U of its selected
    blocks (all groups) is regenerated, in ascending block order, as a short
    sequence; block b maps to its rank in U and the query to the same offset in
    the local block's new position.  Every selected block before the local one
    stays fully visible and the local block keeps its causal prefix, so the
    attention is unchanged.  sel: [H_sel, n, k] (the selection to attend to)."""
    O = np.zeros((len(rows), w.H_q, w.d_h))
    lse = np.zeros((len(rows), w.H_q))
    code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
    sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
    qrows = synth.host_rows(w, "q", bat * w.N + rows)
    for n, i in enumerate(rows):
        s = sel[:, n, :]
        U = np.unique(s[s >= 0])
        rank = {int(b): c for c, b in enumerate(U)}
        tok = (U[:, None] * w.B_k + np.arange(w.B_k)[None, :]).reshape(-1)
        tok = np.minimum(tok, w.N - 1)          # tokens past N are never visible
        Kc = synth.host_rows(w, "k", bat * w.N + tok)
        Vc = synth.host_rows(w, "v", bat * w.N + tok)
        L = i // w.B_k
        ip = rank[int(L)] * w.B_k + (i - L * w.B_k)
        sc_sel = np.where(s >= 0, np.vectorize(lambda b: rank.get(int(b), -1))(s), -1).astype(np.int32)
        o1, l1 = oracle.attention(len(U) * w.B_k, w.B_k, np.array([ip]), qrows[n:n + 1], Kc, Vc,
                                  sc_sel[:, None, :], dtype=code, q_scale=sc, k_scale=sc,
                                  v_scale=sc)
        O[n], lse[n] = o1[0], l1[0]
    return O, lse


def sample_rows(N: int, B_k: int, n: int, seed: int) -> np.ndarray:
    """Edge rows (first rows, block boundaries, last rows) plus seeded random rows."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, B_k - 1, B_k, B_k + 1, 2 * B_k - 1, N // 2, N - B_k - 1, N - B_k, N - 2, N - 1]
    edge = [e for e in edge if 0 <= e < N]
    rnd = rng.integers(0, N, size=max(0, n - len(edge)))
    return np.unique(np.concatenate([edge, rnd]).astype(np.int64))
