"""Plain CPU oracle for the MSA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code: this side decodes raw bf16 / fp8 storage itself and computes every step
from the definitions on the pages:

* block scores and top-k with the forced local block --
  "MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch Architecture and
  Training Stability Mechanisms; "Flash-MSA", Forward > Proxy attention;
* sparse main attention -- "MiniMax Sparse Attention", sec. 2.1 and 2.2;
* split-K log-sum-exp combine -- "MiniMax Sparse Attention (MSA)", Deep Dive >
  KV-Outer Sparse Attention (two-phase forward);
* block-index inversion -- "Flash-MSA", Backward;
* the backward pass: gradients of the sparse main attention and the KL
  alignment gradient of the index branch -- "MiniMax Sparse Attention (MSA)",
  Deep Dive > KL Alignment Loss; "Flash-MSA", Backward and KL Divergence Loss.

The forward arithmetic lives in ``msa_oracle.c`` (plain C, OpenMP over rows);
this module builds it with gcc and marshals numpy arrays through ctypes.  The
backward (``backward`` below) is plain numpy in float64, one (query, group)
at a time.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")

BF16, FP8 = 0, 1


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c99", "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_block_scores.argtypes = [i64, i32, i32, i32, i64, P, P, P, i64, P]
        L.oracle_block_scores.restype = None
        L.oracle_select.argtypes = [i64, i32, i64, i32, i32, P, P, P, P]
        L.oracle_select.restype = None
        L.oracle_attention.argtypes = [i64, i32, i32, i32, i32, i32, i32, i64, P, P, P, P,
                                       i32, f64, f64, f64, P, f64, P, P]
        L.oracle_attention.restype = None
        L.oracle_combine.argtypes = [i32, i32, i32, i32, i64, P, P, P, P, P]
        L.oracle_combine.restype = None
        L.oracle_invert.argtypes = [i64, i64, i32, i64, P, P, P]
        L.oracle_invert.restype = None
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_bf16.restype = ctypes.c_float
        L.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_decode_e4m3.restype = ctypes.c_double
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def block_scores(N, B_k, pos, q_idx_rows, k_idx):
    """Block scores M [n_rows, H_kv, B] (fp32, unscaled; +inf at the local block,
    -inf past it).  ``q_idx_rows`` [n_rows, H_kv, d_idx] and ``k_idx``
    [N, d_idx] hold raw bf16 bit patterns (uint16)."""
    pos, pp = _c(pos, np.int64)
    q, qp = _c(q_idx_rows, np.uint16)
    kk, kp = _c(k_idx, np.uint16)
    n_rows, H_kv, d_idx = q.shape
    assert kk.shape[1] == d_idx and kk.shape[0] >= N
    B = -(-N // B_k)
    M = np.empty((n_rows, H_kv, B), np.float32)
    lib().oracle_block_scores(N, H_kv, d_idx, B_k, n_rows, pp, qp, kp, B,
                              M.ctypes.data_as(ctypes.c_void_p))
    return M


def select(M, pos, B_k, k):
    """TopK with the forced local block.  Returns (block_idx [H_kv, n_rows, k]
    int32 ascending / -1 padded, rel_margin [H_kv, n_rows])."""
    M, mp = _c(M, np.float32)
    pos, pp = _c(pos, np.int64)
    n_rows, H_kv, B = M.shape
    out = np.empty((H_kv, n_rows, k), np.int32)
    marg = np.empty((H_kv, n_rows), np.float64)
    lib().oracle_select(n_rows, H_kv, B, B_k, k, pp, mp,
                        out.ctypes.data_as(ctypes.c_void_p),
                        marg.ctypes.data_as(ctypes.c_void_p))
    return out, marg


def index_topk(N, B_k, k, pos, q_idx_rows, k_idx, force_first=False, window=1):
    """Index branch for the given query rows: (block_idx, rel_margin, M).

    force_first / window > 1: the early-training variant ("MiniMax Sparse
    Attention", ablation of the forced first block and fixed local window):
    block 0 and the window - 1 blocks before the local one get score +inf
    before the selection, so they always take slots.  The returned M holds
    those +inf scores; a margin undefined because the (k-1)-th choice is
    itself forced is +inf (the selection is then unique)."""
    M = block_scores(N, B_k, pos, q_idx_rows, k_idx)
    if force_first or window > 1:
        pos = np.asarray(pos, np.int64)
        for n, i in enumerate(pos):
            L = int(i // B_k)
            if force_first and L >= 1:
                M[n, :, 0] = np.inf
            M[n, :, max(0, L - window + 1):L] = np.inf
    bi, marg = select(M, pos, B_k, k)
    marg = np.where(np.isnan(marg), np.inf, marg)
    return bi, marg, M


def window_selection(pos, B_k, k, H_kv):
    """FLOP-matched sliding-window selection ("MiniMax Sparse Attention",
    comparison with a fixed sparse pattern): block 0 and the k - 1 blocks
    ending at the local block L = i // B_k; every block 0 .. L when L < k.
    [H_kv, n_rows, k] int32, ascending, -1 padded."""
    pos = np.asarray(pos, np.int64)
    out = np.full((len(pos), k), -1, np.int32)
    for n, i in enumerate(pos):
        L = int(i // B_k)
        blocks = list(range(L + 1)) if L < k else [0] + list(range(L - k + 2, L + 1))
        out[n, :len(blocks)] = blocks
    return np.ascontiguousarray(np.broadcast_to(out[None], (H_kv, len(pos), k)))


def attention(N, B_k, pos, q_rows, K, V, block_idx, softmax_scale=None,
              dtype=BF16, q_scale=1.0, k_scale=1.0, v_scale=1.0):
    """Sparse main attention for the given query rows, fp64.

    q_rows [n_rows, H_q, d_h]; K, V [N, H_kv, d_h] as raw uint16 (bf16) or
    uint8 (fp8 e4m3) codes; block_idx [H_sel, n_rows, k]: one selection per
    index head, H_sel a multiple of H_kv dividing H_q (H_sel = H_kv: one per
    GQA group).  Returns (O [n_rows, H_q, d_h], lse [n_rows, H_q]) in
    float64."""
    st = np.uint16 if dtype == BF16 else np.uint8
    pos, pp = _c(pos, np.int64)
    q, qp = _c(q_rows, st)
    Kc, kp = _c(K, st)
    Vc, vp = _c(V, st)
    bi, bp = _c(block_idx, np.int32)
    n_rows, H_q, d_h = q.shape
    H_kv = Kc.shape[1]
    H_sel, k = bi.shape[0], bi.shape[2]
    assert bi.shape == (H_sel, n_rows, k) and H_sel % H_kv == 0 and H_q % H_sel == 0
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d_h)
    O = np.empty((n_rows, H_q, d_h), np.float64)
    lse = np.empty((n_rows, H_q), np.float64)
    lib().oracle_attention(N, H_q, H_kv, H_sel, d_h, B_k, k, n_rows, pp, qp, kp, vp, dtype,
                           float(q_scale), float(k_scale), float(v_scale), bp,
                           float(softmax_scale), O.ctypes.data_as(ctypes.c_void_p),
                           lse.ctypes.data_as(ctypes.c_void_p))
    return O, lse


def dense_attention(N, B_k, pos, q_rows, K, V, softmax_scale=None):
    """Dense causal GQA attention ("MiniMax Sparse Attention", sec. 2.1) for the
    given query rows, fp64: the sparse attention above with every block
    0 .. floor(i / B_k) selected, whose visible tokens are then exactly the
    j <= i of the dense causal form.  Returns (O [n_rows, H_q, d_h],
    lse [n_rows, H_q])."""
    pos = np.asarray(pos, np.int64)
    H_kv = np.asarray(K).shape[1]
    B = -(-N // B_k)
    L = pos // B_k
    sel = np.where(np.arange(B)[None, :] <= L[:, None], np.arange(B)[None, :], -1).astype(np.int32)
    sel = np.ascontiguousarray(np.broadcast_to(sel[None], (H_kv, len(pos), B)))
    return attention(N, B_k, pos, q_rows, K, V, sel, softmax_scale=softmax_scale)


def combine(block_idx, o_part, lse_part):
    """LSE merge.  block_idx [H_kv, n, k]; o_part [H_kv, n, k, G, d_h] bf16 bits;
    lse_part [H_kv, n, k, G] float32.  Returns (O [n, H_q, d_h], lse [n, H_q])."""
    bi, bp = _c(block_idx, np.int32)
    op_, opp = _c(o_part, np.uint16)
    lp, lpp = _c(lse_part, np.float32)
    H_kv, n, k, G, d_h = op_.shape
    O = np.empty((n, H_kv * G, d_h), np.float64)
    lse = np.empty((n, H_kv * G), np.float64)
    lib().oracle_combine(H_kv, G, d_h, k, n, bp, opp, lpp,
                         O.ctypes.data_as(ctypes.c_void_p),
                         lse.ctypes.data_as(ctypes.c_void_p))
    return O, lse


def invert(block_idx, B):
    """Stable counting-sort inversion.  block_idx [n_seq, n_rows, k] ->
    (offsets [n_seq, B + 1], entries [total]) with entry = row * k + slot."""
    bi, bp = _c(block_idx, np.int32)
    n_seq, n_rows, k = bi.shape
    offsets = np.empty((n_seq, B + 1), np.int32)
    entries = np.empty(max(int((bi >= 0).sum()), 1), np.int32)
    lib().oracle_invert(n_seq, n_rows, k, B, bp,
                        offsets.ctypes.data_as(ctypes.c_void_p),
                        entries.ctypes.data_as(ctypes.c_void_p))
    return offsets, entries[: int(offsets[-1, -1]) if n_seq else 0]


def decode_bf16(h: int) -> float:
    return float(lib().oracle_decode_bf16(h))


def decode_e4m3(c: int) -> float:
    return float(lib().oracle_decode_e4m3(c))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def _bf16_f64(h):
    """Raw bf16 bit patterns -> float64 (the bits are the top half of an IEEE
    binary32)."""
    h = np.ascontiguousarray(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _softmax(x):
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def backward(N, B_k, pos, q_rows, K, V, q_idx_rows, k_idx, block_idx, dO_rows,
             softmax_scale=None, kl_weight=1.0):
    """Backward pass of MSA for the given query rows, float64.

    Inputs are raw bf16 bit patterns (uint16): q_rows [n, H_q, d_h]; K, V
    [N, H_kv, d_h]; q_idx_rows [n, H_sel, d_idx]; k_idx [N, d_idx]; dO_rows
    [n, H_q, d_h] (the gradient of the loss with respect to the attention
    output).  block_idx [H_sel, n, k] is the forward's selection (-1 = empty
    slot).

    For query i and selection group r the token set T is the tokens of the
    selected blocks that are visible to i (j <= i) -- "MiniMax Sparse
    Attention", sec. 2.2.  With p_h = softmax over T of scale * Q_h . K_j for
    each head h of the group:

    * main branch (loss sum_h dO_h . O_h, O_h = sum_j p_hj V_j): the gradients
      of exact softmax attention restricted to T;
    * index branch ("MiniMax Sparse Attention (MSA)", Deep Dive > KL Alignment
      Loss): teacher P_j = mean over the group's heads of p_hj (held constant),
      proxy p_px = softmax over T of z_j = q_idx . k_idx_j / sqrt(d_idx), the
      per-row loss KL(P || p_px), and -- "Flash-MSA", KL Divergence Loss -- the
      gradient kl_weight * (p_px - P) on z, carried back to q_idx and k_idx.

    Returns a dict of float64 arrays: dq [n, H_q, d_h], dk, dv [N, H_kv, d_h]
    (contributions of these rows), dq_idx [n, H_sel, d_idx], dk_idx [N, d_idx],
    kl [H_sel, n] (per-row KL, not weighted), O [n, H_q, d_h], lse [n, H_q]."""
    q, Kf, Vf = _bf16_f64(q_rows), _bf16_f64(K), _bf16_f64(V)
    qi, ki, dO = _bf16_f64(q_idx_rows), _bf16_f64(k_idx), _bf16_f64(dO_rows)
    bi = np.asarray(block_idx)
    pos = np.asarray(pos, np.int64)
    n, H_q, d_h = q.shape
    H_kv = Kf.shape[1]
    H_sel = bi.shape[0]
    d_idx = qi.shape[2]
    G_sel = H_q // H_sel
    sel_per_kv = H_sel // H_kv
    scale = 1.0 / np.sqrt(d_h) if softmax_scale is None else float(softmax_scale)
    idx_scale = 1.0 / np.sqrt(d_idx)
    out = {
        "dq": np.zeros((n, H_q, d_h)), "dk": np.zeros((N, H_kv, d_h)),
        "dv": np.zeros((N, H_kv, d_h)), "dq_idx": np.zeros((n, H_sel, d_idx)),
        "dk_idx": np.zeros((N, d_idx)), "kl": np.zeros((H_sel, n)),
        "O": np.zeros((n, H_q, d_h)), "lse": np.zeros((n, H_q)),
    }
    for row in range(n):
        i = int(pos[row])
        for r in range(H_sel):
            blocks = [int(b) for b in bi[r, row] if b >= 0]
            T = np.concatenate([np.arange(b * B_k, min((b + 1) * B_k, N)) for b in blocks])
            T = T[T <= i]
            c = r // sel_per_kv                      # K/V head of group r
            heads = slice(r * G_sel, (r + 1) * G_sel)
            Kt, Vt, Qh, dOh = Kf[T, c], Vf[T, c], q[row, heads], dO[row, heads]
            s = scale * (Qh @ Kt.T)                  # [G_sel, |T|]
            p = _softmax(s)
            Oh = p @ Vt
            out["O"][row, heads] = Oh
            out["lse"][row, heads] = s.max(axis=1) + np.log(np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1))
            # main branch: dV = p^T dO, dP = dO V^T, dS = p (dP - rowsum(dO O))
            out["dv"][T, c] += p.T @ dOh
            dP = dOh @ Vt.T
            dS = p * (dP - (dOh * Oh).sum(axis=1, keepdims=True))
            out["dq"][row, heads] = scale * (dS @ Kt)
            out["dk"][T, c] += scale * (dS.T @ Qh)
            # index branch: KL(P || p_px) and its gradient on z
            z = idx_scale * (ki[T] @ qi[row, r])
            log_ppx = z - (z.max() + np.log(np.exp(z - z.max()).sum()))
            ppx = np.exp(log_ppx)
            P = p.mean(axis=0)
            nz = P > 0
            out["kl"][r, row] = np.sum(P[nz] * (np.log(P[nz]) - log_ppx[nz]))
            g = kl_weight * (ppx - P)
            out["dq_idx"][row, r] = idx_scale * (g @ ki[T])
            out["dk_idx"][T] += idx_scale * np.outer(g, qi[row, r])
    return out
