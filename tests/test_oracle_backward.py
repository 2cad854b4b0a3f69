"""Pins of the backward oracle (``oracle.backward``) against torch autograd.

The gradients are checked against reverse-mode differentiation of a forward
written with library routines (masked scaled-dot-product attention, log-softmax
and the KL divergence of torch.nn.functional) in float64 on the CPU, and against
exact invariants of the method, so that a dropped term (the rowsum of dO * O),
a wrong sign, a transposed operand or a wrong head / group index in the oracle
fails at least one test.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _f64(h):
    return synth.bf16_bits_to_f32(h).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _rand_selection(rng, N, H, B_k, k):
    bi = np.full((H, N, k), -1, np.int32)
    for r in range(H):
        for i in range(N):
            L = i // B_k
            others = rng.permutation(L)[: k - 1] if L else np.zeros(0, int)
            v = sorted(list(others) + [L])
            bi[r, i, : len(v)] = v
    return bi


def _inputs(seed, N, Hq, Hkv, Hsel, d, d_idx, B_k, k):
    rng = np.random.default_rng(seed)
    t = {
        "q": _rand_bf16(rng, (N, Hq, d)), "K": _rand_bf16(rng, (N, Hkv, d)),
        "V": _rand_bf16(rng, (N, Hkv, d)), "qi": _rand_bf16(rng, (N, Hsel, d_idx)),
        "ki": _rand_bf16(rng, (N, d_idx)), "dO": _rand_bf16(rng, (N, Hq, d)),
    }
    t["bi"] = _rand_selection(rng, N, Hsel, B_k, k)
    return t


def _autograd(t, N, B_k, scale, kl_weight):
    """Loss = sum(dO * O) + kl_weight * sum_{i,r} KL(P_teacher || p_px), the
    teacher detached, differentiated by torch (float64, CPU)."""
    q = torch.tensor(_f64(t["q"]), requires_grad=True)
    K = torch.tensor(_f64(t["K"]), requires_grad=True)
    V = torch.tensor(_f64(t["V"]), requires_grad=True)
    qi = torch.tensor(_f64(t["qi"]), requires_grad=True)
    ki = torch.tensor(_f64(t["ki"]), requires_grad=True)
    dO = torch.tensor(_f64(t["dO"]))
    bi = t["bi"]
    Hq, Hkv, Hsel = q.shape[1], K.shape[1], bi.shape[0]
    G, Gs = Hq // Hkv, Hq // Hsel
    blk = np.arange(N) // B_k
    mask_sel = np.zeros((Hsel, N, N), bool)
    for r in range(Hsel):
        for i in range(N):
            mask_sel[r, i] = np.isin(blk, bi[r, i][bi[r, i] >= 0]) & (np.arange(N) <= i)
    ms = torch.from_numpy(mask_sel)
    mh = ms.repeat_interleave(Gs, dim=0)                       # [Hq, N, N]
    Kr = K.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    Vr = V.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    O = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], Kr, Vr, attn_mask=mh[None],
                                       scale=scale)[0].permute(1, 0, 2)
    loss = (O * dO).sum()
    # teacher: the group's per-head softmax distributions, averaged, detached
    s = (q.permute(1, 0, 2) @ Kr[0].transpose(-1, -2)) * scale
    p = torch.softmax(s.masked_fill(~mh, float("-inf")), dim=-1)
    P = p.reshape(Hsel, Gs, N, N).mean(dim=1).detach()
    z = torch.einsum("nrd,md->rnm", qi, ki) / np.sqrt(qi.shape[2])
    logq = torch.log_softmax(z.masked_fill(~ms, float("-inf")), dim=-1)
    logq = torch.where(ms, logq, torch.zeros_like(logq))
    kl_rows = F.kl_div(logq, P, reduction="none").sum(dim=-1)  # [Hsel, N]
    (loss + kl_weight * kl_rows.sum()).backward()
    return {"dq": q.grad, "dk": K.grad, "dv": V.grad, "dq_idx": qi.grad, "dk_idx": ki.grad,
            "kl": kl_rows.detach(), "O": O.detach()}


CASES = [
    # N, Hq, Hkv, Hsel, d, d_idx, B_k, k, seed
    (300, 4, 2, 2, 16, 8, 64, 2, 1),        # sparse: 5 blocks, 2 slots
    (260, 4, 1, 1, 16, 16, 32, 3, 2),       # ragged last block, one group
    (200, 8, 2, 4, 8, 8, 32, 2, 3),         # more index heads than K/V heads
    (150, 2, 2, 2, 16, 8, 64, 4, 4),        # k * B_k >= N: dense causal
]


@pytest.mark.parametrize("N,Hq,Hkv,Hsel,d,d_idx,B_k,k,seed", CASES)
def test_backward_matches_autograd(N, Hq, Hkv, Hsel, d, d_idx, B_k, k, seed):
    t = _inputs(seed, N, Hq, Hkv, Hsel, d, d_idx, B_k, k)
    scale, w = 0.35, 0.7
    ref = _autograd(t, N, B_k, scale, w)
    got = oracle.backward(N, B_k, np.arange(N), t["q"], t["K"], t["V"], t["qi"], t["ki"], t["bi"],
                          t["dO"], softmax_scale=scale, kl_weight=w)
    for name in ("dq", "dk", "dv", "dq_idx", "dk_idx", "kl", "O"):
        r = ref[name].numpy()
        np.testing.assert_allclose(got[name], r, rtol=0, atol=1e-10 * max(1.0, np.abs(r).max()),
                                   err_msg=name)


def test_backward_invariants():
    """Softmax rows sum to one and dS rows sum to zero, so over all keys
    sum_j dK_j = 0, sum_j dk_idx_j = 0 and sum_j dV_j = sum over the rows and
    heads of dO; KL is non-negative."""
    N, Hq, Hkv, Hsel, d, d_idx, B_k, k = 256, 4, 2, 2, 16, 8, 32, 3
    t = _inputs(7, N, Hq, Hkv, Hsel, d, d_idx, B_k, k)
    got = oracle.backward(N, B_k, np.arange(N), t["q"], t["K"], t["V"], t["qi"], t["ki"], t["bi"],
                          t["dO"], kl_weight=1.3)
    assert np.abs(got["dk"].sum(axis=0)).max() < 1e-10
    assert np.abs(got["dk_idx"].sum(axis=0)).max() < 1e-10
    dO = _f64(t["dO"]).reshape(N, Hkv, Hq // Hkv, d).sum(axis=(0, 2))
    np.testing.assert_allclose(got["dv"].sum(axis=0), dO, rtol=0, atol=1e-9)
    assert (got["kl"] >= -1e-12).all() and got["kl"].max() > 0


def test_backward_kl_vanishes_when_proxy_equals_teacher():
    """One head per group, d_idx = d_h, the index inputs equal to the main Q
    and K and the index scale equal to the softmax scale: the proxy
    distribution is the teacher, so KL = 0 and both index gradients vanish."""
    N, d, B_k, k = 200, 16, 32, 3
    rng = np.random.default_rng(5)
    q = _rand_bf16(rng, (N, 1, d))
    K = _rand_bf16(rng, (N, 1, d))
    V = _rand_bf16(rng, (N, 1, d))
    dO = _rand_bf16(rng, (N, 1, d))
    bi = _rand_selection(rng, N, 1, B_k, k)
    got = oracle.backward(N, B_k, np.arange(N), q, K, V, q, K[:, 0], bi, dO,
                          softmax_scale=d ** -0.5, kl_weight=1.0)
    assert np.abs(got["kl"]).max() < 1e-12
    assert np.abs(got["dq_idx"]).max() < 1e-12 and np.abs(got["dk_idx"]).max() < 1e-12


def test_backward_first_query_has_no_query_gradient():
    """Query 0 sees only key 0: its softmax is the constant 1, so dQ and dq_idx
    of row 0 vanish, dV_0 gets dO_0 in full, and its KL is 0."""
    N, Hq, Hkv, d, d_idx, B_k, k = 64, 2, 1, 8, 8, 32, 2
    t = _inputs(9, N, Hq, Hkv, Hkv, d, d_idx, B_k, k)
    got = oracle.backward(N, B_k, np.array([0]), t["q"][:1], t["K"], t["V"], t["qi"][:1], t["ki"],
                          t["bi"][:, :1], t["dO"][:1])
    assert np.abs(got["dq"]).max() == 0 and np.abs(got["dq_idx"]).max() == 0
    np.testing.assert_allclose(got["dv"][0, 0], _f64(t["dO"])[0].sum(axis=0), rtol=0, atol=1e-14)
    assert abs(got["kl"][0, 0]) < 1e-15
