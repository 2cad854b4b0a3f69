"""A seeded random sweep of shapes through the whole forward (msa_forward) and
the backward (msa_backward), called through the C ABI and compared with the
oracle: ragged N, k, the GQA factor G (1..16), more index heads than K/V heads,
B_k in {32, 64, 128}, d_idx in {64, 128}, query chunking, batch 2 and fp8
Q/K/V, drawn from a fixed seed so that every run checks the same cases.

Forward: the selection is checked on sampled rows (edge rows and seeded random
rows) by the margin rule of the other parity tests, and the output and LSE of
those rows against the oracle's attention over the GPU's own selection.
Backward (B_k = 128; small N, and N of 2.5K-8K where workgroups take runs of
consecutive passes): every gradient and the KL over all rows, with the
tolerances of the backward parity tests.  Decode: the last token of every
sequence, selection and output, as in the decode parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_attention_idx_amd as msa
import oracle
import synth
from gpu_util import (check_selection, device_inputs, dims_of, err_stats, log, opts_of, oracle_index_rows,
                      sample_rows)
from test_gpu_parity import _check_decode, _decode_inputs
from test_gpu_parity_backward import KL_W, _f, _grad_check, _run

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _draw(rng, backward: bool, seed: int) -> synth.Workload:
    B_k = 128 if backward else int(rng.choice([32, 64, 128]))
    H_kv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    per_kv = int(rng.choice([1, 1, 2, 4]))       # index heads per K/V head
    while G % per_kv:
        per_kv //= 2
    max_blocks = 12 if backward else 24
    N = int(rng.integers(1, max_blocks)) * B_k + int(rng.integers(0, B_k))
    fp8 = (not backward) and B_k == 128 and rng.random() < 0.3
    return synth.TINY.with_(
        name=f"sweep{seed}", seed=seed, N=max(N, 1), H_q=H_kv * G, H_kv=H_kv,
        H_idx=H_kv * per_kv if per_kv > 1 else 0, B_k=B_k, k=int(rng.integers(1, 17)),
        d_idx=int(rng.choice([64, 128])), batch=int(rng.choice([1, 1, 2])),
        q_chunk=int(rng.choice([0, 0, 3 * B_k, 8 * B_k])), dtype="fp8" if fp8 else "bf16")


_RNG = np.random.default_rng(20261202)
FWD_SWEEP = [_draw(_RNG, False, 1000 + j) for j in range(14)]
BWD_SWEEP = [_draw(_RNG, True, 2000 + j) for j in range(6)]
DEC_SWEEP = [_draw(_RNG, False, 3000 + j).with_(dtype="bf16", q_chunk=0, N=int(_RNG.integers(1, 6000)))
             for j in range(6)]


def _draw_joined(rng, seed: int) -> synth.Workload:
    """Backward shapes where a group's passes outnumber the 256 workgroups at
    least twice (N k >= 2 * 256 * 256 / G), so workgroups get runs of
    consecutive passes of one key block and the index-branch chunks join
    them."""
    G = int(rng.choice([8, 16]))
    k = int(rng.integers(3, 6))
    N = max(int(rng.integers(2500, 4600)), 2 * 256 * 256 // (G * k) + int(rng.integers(0, 128)))
    return synth.TINY.with_(name=f"sweepj{seed}", seed=seed, N=N, H_q=2 * G, H_kv=2, H_idx=0, B_k=128, k=k,
                            d_idx=int(rng.choice([64, 128])), batch=1, q_chunk=0, dtype="bf16")


_RNG_J = np.random.default_rng(20261203)
BWD_JOINED = [_draw_joined(_RNG_J, 4000 + j) for j in range(3)]


def _wid(w):
    return (f"N{w.N}_G{w.G}_Hs{w.H_sel}_bk{w.B_k}_k{w.k}_d{w.d_idx}_b{w.batch}_c{w.q_chunk}_{w.dtype}")


@pytest.mark.parametrize("w", FWD_SWEEP, ids=_wid)
def test_forward_sweep(w):
    log(f"sweep forward {_wid(w)}")
    t = device_inputs(w, DEV)
    d, o = dims_of(w), opts_of(w)
    bi = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_forward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"],
                                  block_idx_out=bi, want_lse=True)
    torch.cuda.synchronize()
    gsel = bi.cpu().numpy()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = sample_rows(w.N, w.B_k, 40, seed=w.seed)
    code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
    sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
    for b in range(w.batch):
        ob, marg, M = oracle_index_rows(w, rows, bat=b)
        st = check_selection(gsel[b][:, rows], ob, marg, M, w.k, what=f"sweep batch {b}")
        log(f"  batch {b} selection: {st}")
        keys = b * w.N + np.arange(w.N)
        O, L = oracle.attention(w.N, w.B_k, rows, synth.host_rows(w, "q", b * w.N + rows),
                                synth.host_rows(w, "k", keys), synth.host_rows(w, "v", keys),
                                np.ascontiguousarray(gsel[b][:, rows]), dtype=code, q_scale=sc,
                                k_scale=sc, v_scale=sc)
        mx, mn = err_stats(out[b][rows], O, label="O")
        assert mx <= (6e-2 if w.dtype == "fp8" else 2e-2) and mn <= 2e-3
        lmx, _ = err_stats(lse[b][rows], L)
        assert lmx <= 1e-3


@pytest.mark.parametrize("w", BWD_SWEEP + BWD_JOINED, ids=_wid)
def test_backward_sweep(w):
    log(f"sweep backward {_wid(w)}")
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
        assert float(np.abs(kl - ref["kl"]).max()) <= 1e-3 * max(1.0, float(ref["kl"].max()))


@pytest.mark.parametrize("w", DEC_SWEEP, ids=_wid)
def test_decode_sweep(w):
    log(f"sweep decode {_wid(w)}")
    t = device_inputs(w, DEV)
    q1, qi1 = _decode_inputs(w, t)
    bi = torch.empty((w.batch, w.H_sel, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_decode(dims_of(w), msa.make_opts(), q1, qi1, t["k"], t["v"], t["k_idx"],
                                 block_idx_out=bi, want_lse=True)
    torch.cuda.synchronize()
    _check_decode(w, t, out.float().cpu().numpy(), lse.cpu().numpy(), bi.cpu().numpy())
