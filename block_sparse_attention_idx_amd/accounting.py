"""Work accounting for the MSA forward pass (host-side bookkeeping only).

FLOP conventions:

* Index branch, as executed: every row i scores the L(i) = floor(i / B_k)
  earlier blocks in full (the local block is forced and never scored), so
  index FLOPs = sum_i 2 * d_idx * H_kv * B_k * L(i).
* Main branch: 4 * d_h FLOPs (QK^T and PV) per (query head, visible key);
  visible keys are the tokens of the selected blocks at or before the query.
* Per-token model of "MiniMax Sparse Attention", sec. 3.3 / Figure 4: causal
  GQA costs 4 d_h H_q N / 2 per token; MSA costs 2 d_idx H_kv N / 2 for the
  index branch plus 4 d_h H_q k B_k for the main branch.

Byte conventions for the HBM-bound kernels are stated next to each function.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- per-token model

def gqa_flops_per_token(N: int, H_q: int, d_h: int) -> float:
    return 4.0 * d_h * H_q * N / 2.0


def msa_flops_per_token(N: int, H_q: int, H_kv: int, d_h: int, d_idx: int, B_k: int, k: int) -> float:
    return 2.0 * d_idx * H_kv * N / 2.0 + 4.0 * d_h * H_q * k * B_k


def flops_reduction(N, H_q, H_kv, d_h, d_idx, B_k, k) -> float:
    return gqa_flops_per_token(N, H_q, d_h) / msa_flops_per_token(N, H_q, H_kv, d_h, d_idx, B_k, k)


def attended_context_reduction(N: int, B_k: int, k: int) -> float:
    """Full context over the fixed k * B_k budget."""
    return N / float(k * B_k)


# ---------------------------------------------------------------- intensity (sec. 4.2)

def q_outer_intensity(G: int, B_k: int, d_h: int, elem: int = 2) -> float:
    """Q-outer: one query's G heads against one K/V block.  FLOPs 4 d_h B_k G;
    traffic is the K and V block, 2 B_k d_h elements of ``elem`` bytes."""
    return 4.0 * d_h * B_k * G / (2.0 * B_k * d_h * elem)


def kv_outer_intensity(B_k: int, d_h: int, elem: int = 2) -> float:
    """KV-outer: per (query head, block) 4 d_h B_k FLOPs against reading q,
    writing one partial output and reading it back (3 d_h elements)."""
    return 4.0 * d_h * B_k / (3.0 * d_h * elem)


# ---------------------------------------------------------------- I/O crossover model

def io_model(G=16, D=128, top_k=16, B_k=128, data_bytes=1, partial_bytes=2,
             hbm_tbs=7.4, l2_tbs=24.0):
    """Bandwidth model of the KV-outer vs Q-outer crossover, per (token,
    kv head): Q = O = G D data bytes, one partial output = G D partial bytes,
    a K+V block = 2 B_k D data bytes.  Returns a dict of the coefficients."""
    q = o = G * D * data_bytes
    part = top_k * G * D * partial_bytes
    kv = 2 * B_k * D * data_bytes
    hbm_n = q + o + part
    l2_n = top_k * q + 2 * part + o
    q_outer_l2 = (top_k * kv + q + o) / l2_tbs
    return {
        "hbm_per_token": hbm_n, "hbm_per_block": kv,
        "l2_per_token": l2_n, "l2_per_block": kv,
        "hbm_latency_token": hbm_n / hbm_tbs, "hbm_latency_block": kv / hbm_tbs,
        "l2_latency_token": l2_n / l2_tbs, "l2_latency_block": kv / l2_tbs,
        "q_outer_l2_token": q_outer_l2,
        "crossover": (q_outer_l2 - hbm_n / hbm_tbs) / (kv / hbm_tbs),
    }


# ---------------------------------------------------------------- exact counts

def index_flops(q_begin: int, q_count: int, H_kv: int, d_idx: int, B_k: int, batch: int = 1) -> float:
    i = np.arange(q_begin, q_begin + q_count, dtype=np.int64)
    return float(batch) * 2.0 * d_idx * H_kv * B_k * float((i // B_k).sum())


def visible_keys(block_idx: np.ndarray, q_begin: int, N: int, B_k: int) -> np.ndarray:
    """Visible keys per (seq, row): block_idx [n_seq, n_rows, k] -> [n_seq, n_rows]."""
    n_rows = block_idx.shape[1]
    i = np.arange(q_begin, q_begin + n_rows, dtype=np.int64)[None, :, None]
    b = block_idx.astype(np.int64)
    lo = b * B_k
    hi = np.minimum(np.minimum(lo + B_k, N), i + 1)
    cnt = np.where(b >= 0, np.maximum(hi - lo, 0), 0)
    return cnt.sum(axis=2)


def main_flops(block_idx: np.ndarray, q_begin: int, N: int, B_k: int, G: int, d_h: int) -> float:
    return 4.0 * d_h * G * float(visible_keys(block_idx, q_begin, N, B_k).sum())


def backward_flops(block_idx: np.ndarray, q_begin: int, N: int, B_k: int, G: int, d_h: int,
                   d_idx: int, index: bool = True) -> tuple:
    """FLOPs of the backward pass as its kernels execute it, per visible
    (query, selection group, key): the main branch recomputes S and forms dP,
    dV, dK and dQ, 10 d_h per head (2.5x the forward's 4 d_h), and hands the
    teacher distribution (the mean of its heads' probabilities) to the index
    branch; the index branch computes the proxy scores twice (once in the proxy
    log-sum-exp pass, once beside the gradient) and forms dq_idx and dk_idx
    (8 d_idx in all).  Returns (main, index)."""
    vis = float(visible_keys(block_idx, q_begin, N, B_k).sum())
    main = 10.0 * d_h * G * vis
    idx = 8.0 * d_idx * vis if index else 0.0
    return main, idx


def dense_flops(q_begin: int, q_count: int, H_q: int, d_h: int, batch: int = 1) -> float:
    """Dense causal attention: 4 d_h FLOPs per (query head, key j <= i)."""
    i = np.arange(q_begin, q_begin + q_count, dtype=np.float64)
    return float(batch) * 4.0 * d_h * H_q * float((i + 1.0).sum())


def decode_bytes(batch: int, N: int, H_q: int, H_kv: int, d_h: int, d_idx: int, B_k: int, k: int,
                 valid_slots: int) -> int:
    """HBM bytes of one decode step (bf16), each tensor counted once: the
    K^idx scan of the L = (N - 1) // B_k earlier blocks, Q^idx and Q, the block
    scores written and read, K and V of every selected block (the last block
    partial), the partial outputs written and read by the merge, the selection,
    and O."""
    L = (N - 1) // B_k
    B = -(-N // B_k)
    G = H_q // H_kv
    scan = batch * L * B_k * d_idx * 2 + batch * H_kv * d_idx * 2
    scores = 2 * 4 * batch * H_kv * B
    kv = valid_slots * 2 * B_k * d_h * 2
    part = 2 * valid_slots * G * (2 * d_h + 4)
    return int(scan + scores + kv + part + 2 * 4 * batch * H_kv * k + 2 * batch * H_q * d_h * 2)


def partial_bytes(n_valid_slots: int, G: int, d_h: int) -> int:
    """Bytes of one partial output set: bf16 O-bar (2 d_h) + fp32 lse per head."""
    return n_valid_slots * G * (2 * d_h + 4)
