"""The accounting model reproduces the numbers the pages print."""
import json
import os

import numpy as np
import pytest

from block_sparse_attention_idx_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _near(got, ent):
    return abs(got - ent["value"]) <= ent["rounding"] + 1e-12


def test_flops_reduction_at_1m():
    e = GOLD["flops_reduction_1M"]
    assert _near(acc.flops_reduction(**e["config"]), e)
    # with a smaller index head the printed figure is not reproduced
    c = dict(e["config"], d_idx=64)
    assert not _near(acc.flops_reduction(**c), e)


def test_attended_context_reductions():
    for key in ("attended_reduction_128K", "attended_reduction_1M"):
        e = GOLD[key]
        assert _near(acc.attended_context_reduction(**e["config"]), e)
    e = GOLD["budget_tokens"]
    assert e["config"]["k"] * e["config"]["B_k"] == e["value"]


def test_intensities():
    kv = acc.kv_outer_intensity(**GOLD["kv_outer_intensity"]["config"])
    qo = acc.q_outer_intensity(**GOLD["q_outer_intensity"]["config"])
    assert _near(kv, GOLD["kv_outer_intensity"])
    assert _near(qo, GOLD["q_outer_intensity"])
    assert _near(kv / qo, GOLD["intensity_ratio"])


def test_io_crossover_model():
    e = GOLD["io_model"]
    m = acc.io_model(**e["config"])
    for key in ("hbm_per_token", "hbm_per_block", "l2_per_token", "l2_per_block", "q_outer_l2_token"):
        assert m[key] == pytest.approx(e[key], abs=0.5), key
    for key in ("hbm_latency_token", "hbm_latency_block", "l2_latency_token", "l2_latency_block"):
        assert m[key] == pytest.approx(e[key], abs=0.5), key
    assert m["crossover"] == pytest.approx(e["crossover"], abs=0.005)


def test_exact_counts_small():
    # one sequence, B_k = 4, N = 10: rows 0..9, L = 0,0,0,0,1,1,1,1,2,2
    assert acc.index_flops(0, 10, 1, 2, 4) == 2 * 2 * 1 * 4 * (0 * 4 + 1 * 4 + 2 * 2)
    bi = np.array([[[0, -1], [0, -1], [0, 1], [1, 2]]], np.int32)   # rows 4..7
    vis = acc.visible_keys(bi, 4, 10, 4)
    assert vis.tolist() == [[4, 4, 4 + 3, 4 + 0]]  # row 6 sees 4..6 of block 1; row 7 none of block 2


def test_dense_flops_closed_form_and_chunks():
    """Dense causal FLOPs: 4 d_h H_q N (N + 1) / 2; chunks add up; the per-token
    GQA figure the pages use (N / 2 keys per query) matches to O(1 / N)."""
    N, H_q, d_h = 131072, 64, 128
    full = acc.dense_flops(0, N, H_q, d_h)
    assert full == 4.0 * d_h * H_q * N * (N + 1) / 2
    parts = sum(acc.dense_flops(b, 32768, H_q, d_h) for b in range(0, N, 32768))
    assert parts == full
    assert abs(full / (N * acc.gqa_flops_per_token(N, H_q, d_h)) - 1.0) < 2.0 / N
    assert acc.dense_flops(0, 1, 1, 1, batch=3) == 12.0


def test_decode_bytes_dominated_by_index_scan():
    """At 1M tokens the K^idx scan (256 B per earlier token) is almost all of a
    decode step's traffic; a single-block context reads no K^idx at all."""
    N = 1 << 20
    total = acc.decode_bytes(1, N, 64, 4, 128, 128, 128, 16, 4 * 16)
    scan = (N - 128) * 128 * 2
    assert scan < total < 1.02 * scan + 5e6
    small = acc.decode_bytes(2, 100, 8, 2, 128, 64, 128, 4, 2 * 2)
    assert small == (2 * 2 * 64 * 2 + 2 * 4 * 2 * 2 * 1 + 4 * 2 * 128 * 128 * 2
                     + 2 * 4 * 4 * (256 + 4) + 2 * 4 * 2 * 2 * 4 + 2 * 2 * 8 * 128 * 2)


def test_backward_flops_relations():
    """The backward's main-branch count is 2.5x the forward's 4 d_h per visible
    key (S recomputed, dP, dV, dK, dQ), the index branch's 8 d_idx per visible
    (query, group, key), and nothing when the index branch is off; a full
    budget (every causal block selected) counts every key j <= i."""
    N, B_k, k, G, d_h, d_idx = 640, 64, 16, 4, 128, 64
    i = np.arange(N)
    L = i // B_k
    sel = np.full((2, N, k), -1, np.int32)
    for r in range(2):
        for row in range(N):
            sel[r, row, :L[row] + 1] = np.arange(L[row] + 1)   # k * B_k >= N: all causal blocks
    fwd = acc.main_flops(sel, 0, N, B_k, G, d_h)
    main, idx = acc.backward_flops(sel, 0, N, B_k, G, d_h, d_idx)
    keys = float((i + 1).sum()) * 2                             # visible (query, group, key)
    assert fwd == 4.0 * d_h * G * keys
    assert main == 2.5 * fwd
    assert idx == 8.0 * d_idx * keys
    assert acc.backward_flops(sel, 0, N, B_k, G, d_h, d_idx, index=False)[1] == 0.0
