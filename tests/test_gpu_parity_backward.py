"""Parity of the backward pass (msa_backward, called through the C ABI) with
the CPU oracle.

The selection is an input of the backward (the forward's, held constant): the
GPU forward's block_idx, O and LSE feed msa_backward, and the oracle
recomputes the gradients from the definition with that same selection.

Tolerance, derived from the arithmetic: the kernels round P, dS and the KL
gradient g to bf16 (unit roundoff u = 2^-8 / 2 = 2^-9) as MFMA operands,
keep per-slot dQ partials in bf16 and round every output to bf16, and
D = rowsum(dO * O) uses the forward's bf16 O.  Each gradient element is a
sum of terms whose rounding errors are independent, so the error is a few u
of the root-sum-square of the terms, itself of the order of the result:
relative L2 error <= 2e-2 (about 10 u) per tensor, and every element within
3e-2 (about 16 u) of the tensor's largest magnitude.  KL values are fp32 sums
of fp32 terms: |diff| <= 1e-3 max(1, max |KL|).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_idx_amd as msa
import oracle
import synth
from gpu_util import device_inputs, dims_of, log, opts_of, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TINY = synth.TINY
KL_W = 0.37


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _f(t):
    return t.view(torch.bfloat16).float().cpu().numpy().astype(np.float64) if t.dtype in (
        torch.int16, torch.bfloat16) else t.cpu().numpy().astype(np.float64)


def _grad_check(name, got, ref):
    d = got - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(d).max() / max(np.abs(ref).max(), 1e-30))
    log(f"  {name}: rel L2 {rel:.3g}  max |diff| / max |ref| {mx:.3g}")
    assert rel <= 2e-2 and mx <= 3e-2, name


def _run(w, t, d_o, index=True):
    d, o = dims_of(w), opts_of(w)
    bi = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_forward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"],
                                  block_idx_out=bi, want_lse=True)
    g = msa.msa_backward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], out, lse, d_o, bi,
                         kl_weight=KL_W, index=index)
    torch.cuda.synchronize()
    return g, bi.cpu().numpy()


BWD_CASES = [
    TINY,                                                       # G 4, d_idx 64
    TINY.with_(N=1000, H_q=32, H_kv=2, d_idx=128, k=3),         # G 16, partial last block
    TINY.with_(N=1500, H_q=2, H_kv=2, k=5, q_chunk=512),        # G 1, three query chunks
    TINY.with_(N=900, H_q=16, H_kv=2, H_idx=8, k=4),            # 8 index heads over 2 K/V heads
    TINY.with_(N=1300, H_q=16, H_kv=2, k=6, d_idx=128),         # G 8
    TINY.with_(N=700, batch=2, k=3),                            # batch 2
    TINY.with_(N=1100, batch=2, k=4, q_chunk=384),              # batch 2, three query chunks (ragged)
    # G 16 and 8 at N = 4096: a group's 512-1024 passes leave every workgroup
    # several consecutive passes of one key block, so the index branch's
    # chunks join passes (a pass holds 256 / G entries, a chunk 64)
    TINY.with_(N=4096, H_q=32, H_kv=2, d_idx=128, k=4),
    TINY.with_(N=4096, H_q=16, H_kv=2, d_idx=64, k=4),
]


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: f"N{w.N}_G{w.G}_Hs{w.H_sel}_d{w.d_idx}_k{w.k}_b{w.batch}_c{w.q_chunk}")
def test_backward_parity(w):
    log(f"backward N={w.N} H_q={w.H_q} H_kv={w.H_kv} H_sel={w.H_sel} d_idx={w.d_idx} k={w.k} "
        f"batch={w.batch} q_chunk={w.q_chunk}")
    t = device_inputs(w, DEV)
    d_o = synth.device_tensor(w, "d_o", DEV)
    g, sel = _run(w, t, d_o)
    for bat in range(w.batch):
        rows = np.arange(w.N)
        flat = bat * w.N + rows
        h = {x: synth.host_rows(w, x, flat) for x in ("q", "k", "v", "q_idx", "k_idx", "d_o")}
        ref = oracle.backward(w.N, w.B_k, rows, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], sel[bat],
                              h["d_o"], kl_weight=KL_W)
        for name in ("dq", "dk", "dv", "dq_idx", "dk_idx"):
            _grad_check(f"{name}[{bat}]", _f(g[name][bat]), ref[name])
        kl = _f(g["kl"][bat])
        err = float(np.abs(kl - ref["kl"]).max())
        log(f"  kl[{bat}]: max |diff| {err:.3g} (max {ref['kl'].max():.3g})")
        assert err <= 1e-3 * max(1.0, float(ref["kl"].max()))


def test_backward_without_index_branch_matches():
    """Skipping the index branch leaves the main-branch gradients unchanged."""
    w = TINY.with_(N=1100, k=3)
    t = device_inputs(w, DEV)
    d_o = synth.device_tensor(w, "d_o", DEV)
    a, _ = _run(w, t, d_o, index=True)
    b, _ = _run(w, t, d_o, index=False)
    assert b["dq_idx"] is None and b["kl"] is None
    assert torch.equal(a["dq"], b["dq"])
    for name in ("dk", "dv"):  # fp32 atomics: the order of the additions may differ
        _grad_check(name, _f(b[name]), _f(a[name]))


@pytest.mark.parametrize("w", [synth.P16K, synth.P128K_HOT], ids=lambda w: w.name)
def test_backward_sampled_rows_and_sums(w):
    """The 16K prefill and the 128K prefill with planted hot blocks (the
    backward bench workload), 64 query heads: dQ, dq_idx and KL on sampled
    rows against the oracle; over all rows, the exact sums sum_j dK_j = 0,
    sum_j dk_idx_j = 0 (softmax rows sum to one, dS and g rows to zero) and
    sum_j dV_j = sum over rows and heads of dO."""
    log(f"backward {w.name}")
    t = device_inputs(w, DEV)
    d_o = synth.device_tensor(w, "d_o", DEV)
    g, sel = _run(w, t, d_o)
    rows = sample_rows(w.N, w.B_k, 48, seed=5)
    allk = {x: synth.host_rows(w, x, np.arange(w.N)) for x in ("k", "v", "k_idx")}
    ref = oracle.backward(w.N, w.B_k, rows, synth.host_rows(w, "q", rows), allk["k"], allk["v"],
                          synth.host_rows(w, "q_idx", rows), allk["k_idx"], sel[0][:, rows],
                          synth.host_rows(w, "d_o", rows), kl_weight=KL_W)
    ri = torch.as_tensor(rows, device=DEV)
    _grad_check("dq (sampled rows)", _f(g["dq"][0][ri]), ref["dq"])
    _grad_check("dq_idx (sampled rows)", _f(g["dq_idx"][0][ri]), ref["dq_idx"])
    kl = _f(g["kl"][0][:, ri])
    assert np.abs(kl - ref["kl"]).max() <= 1e-3 * max(1.0, float(ref["kl"].max()))
    dk = g["dk"][0].view(torch.bfloat16).double()
    dv = g["dv"][0].view(torch.bfloat16).double()
    dki = g["dk_idx"][0].view(torch.bfloat16).double()
    sum_do = d_o[0].view(torch.bfloat16).double().reshape(w.N, w.H_kv, w.G, w.d_h).sum(dim=(0, 2))
    # scale of the sums: the root-sum-square of the summed gradients
    for name, s, x in (("sum dK", dk.sum(0), dk), ("sum dk_idx", dki.sum(0), dki),
                       ("sum dV - sum dO", dv.sum(0) - sum_do, dv)):
        rss = float(x.pow(2).sum(0).sqrt().max())
        err = float(s.abs().max())
        log(f"  {name}: max {err:.3g} (root-sum-square {rss:.3g})")
        assert err <= 2e-2 * rss, name


@pytest.mark.parametrize("w", [synth.P16K, synth.P128K_HOT], ids=lambda w: w.name)
def test_backward_key_blocks_elementwise(w):
    """Whole key blocks of dK, dV and dk_idx, element by element, at full size.
    A key's gradient sums over every query that selected its block, so the
    oracle runs on exactly those queries (found in the forward's selection):
    for group 1, the last block (selected only as the local block), the one
    before it, and the least-selected block of the middle half of the
    sequence; for dk_idx (shared by all groups) the last block over all
    groups.  A misplaced atomic (another key row, another head) fails here
    even when the column sums agree."""
    log(f"backward key blocks {w.name}")
    t = device_inputs(w, DEV)
    d_o = synth.device_tensor(w, "d_o", DEV)
    g, sel = _run(w, t, d_o)
    sel0 = sel[0]                                     # [H_sel, N, k]
    B, r, G = w.B, 1, w.G_sel
    allk = {x: synth.host_all(w, x) for x in ("k", "v", "k_idx")}
    picked = lambda rr, b: np.nonzero((sel0[rr] == b).any(axis=1))[0]
    mid = np.arange(B // 4, 3 * B // 4)
    counts = np.array([len(picked(r, b)) for b in mid])
    blocks = [B - 1, B - 2, int(mid[int(np.argmin(counts))])]
    rows = np.unique(np.concatenate([picked(r, b) for b in blocks]))
    log(f"  group {r}: blocks {blocks}, {len(rows)} selecting queries")
    heads = slice(r * G, (r + 1) * G)
    ref = oracle.backward(w.N, w.B_k, rows, synth.host_rows(w, "q", rows)[:, heads],
                          allk["k"][:, r:r + 1], allk["v"][:, r:r + 1],
                          synth.host_rows(w, "q_idx", rows)[:, r:r + 1], allk["k_idx"],
                          np.ascontiguousarray(sel0[r:r + 1][:, rows]),
                          synth.host_rows(w, "d_o", rows)[:, heads], kl_weight=KL_W)
    dk, dv = _f(g["dk"][0]), _f(g["dv"][0])
    for b in blocks:
        keys = slice(b * w.B_k, min((b + 1) * w.B_k, w.N))
        _grad_check(f"dK block {b}", dk[keys, r], ref["dk"][keys, 0])
        _grad_check(f"dV block {b}", dv[keys, r], ref["dv"][keys, 0])
    last = np.unique(np.concatenate([picked(rr, B - 1) for rr in range(w.H_sel)]))
    ref2 = oracle.backward(w.N, w.B_k, last, synth.host_rows(w, "q", last), allk["k"], allk["v"],
                           synth.host_rows(w, "q_idx", last), allk["k_idx"],
                           np.ascontiguousarray(sel0[:, last]), synth.host_rows(w, "d_o", last),
                           kl_weight=KL_W)
    keys = slice((B - 1) * w.B_k, w.N)
    _grad_check(f"dk_idx block {B - 1}", _f(g["dk_idx"][0])[keys], ref2["dk_idx"][keys])
