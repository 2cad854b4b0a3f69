"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a brute-force formulation on tiny inputs,
a library routine that the definition reduces to in a special case, a closed
form, or an exact invariant of the method, so that a dropped term, a wrong
index, a sign or a transposed operand in the oracle fails at least one test.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _f32(h):
    return synth.bf16_bits_to_f32(h).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_matches_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    ok = ~np.isnan(ref)
    got = np.array([oracle.decode_bf16(int(c)) for c in codes[ok][::97]])
    assert np.array_equal(got, ref[ok][::97])


def test_e4m3_decoder_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.decode_e4m3(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.decode_e4m3(0x7E) == 448.0


# ---------------------------------------------------------------- index branch

def brute_scores(N, B_k, q_idx, k_idx):
    """fp64 brute force: full score matrix, causal mask, block max-pool."""
    q = _f32(q_idx)                        # [N, H, d]
    kk = _f32(k_idx)                       # [N, d]
    H = q.shape[1]
    B = -(-N // B_k)
    S = np.einsum("ihd,jd->hij", q, kk)    # [H, N, N]
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    S = np.where(j <= i, S, -np.inf)
    pad = np.full((H, N, B * B_k), -np.inf)
    pad[:, :, :N] = S
    M = pad.reshape(H, N, B, B_k).max(axis=3)       # causal max over each block
    L = np.arange(N) // B_k
    M[:, np.arange(N), L] = np.inf                  # forced local block
    return M.transpose(1, 0, 2)                     # [N, H, B]


def brute_select(M, k):
    """Stable order by (-score, block id); keep the first k with finite score."""
    N, H, B = M.shape
    out = np.full((H, N, k), -1, np.int32)
    marg = np.full((H, N), np.inf)
    for r in range(H):
        for i in range(N):
            m = M[i, r]
            order = np.lexsort((np.arange(B), -m))
            keep = [b for b in order if np.isfinite(m[b]) or m[b] == np.inf][:k]
            keep = sorted(keep)
            out[r, i, : len(keep)] = keep
            cand = np.sort(m[np.isfinite(m)])[::-1]
            if len(cand) >= k and k >= 2:
                a, b = cand[k - 2], cand[k - 1]
                marg[r, i] = (a - b) / max(abs(a), abs(b), 1e-6)
    return out, marg


@pytest.mark.parametrize("N,H,d,k,seed,B_k", [
    (256, 1, 64, 1, 0, 128), (256, 2, 64, 2, 1, 128), (1000, 2, 128, 4, 2, 128), (1000, 1, 64, 16, 3, 128),
    (2048, 2, 64, 4, 4, 128), (2048, 1, 128, 8, 5, 128), (640, 3, 32, 3, 6, 128),
    (521, 2, 64, 2, 7, 32), (777, 1, 128, 2, 8, 32), (1000, 2, 64, 16, 9, 32),   # 32-token blocks
    (1200, 2, 128, 6, 10, 64), (200, 1, 64, 3, 11, 64),                           # 64-token blocks
])
def test_index_matches_brute_force(N, H, d, k, seed, B_k):
    rng = np.random.default_rng(seed)
    q = _rand_bf16(rng, (N, H, d))
    kk = _rand_bf16(rng, (N, d))
    pos = np.arange(N)
    bi, marg, M = oracle.index_topk(N, B_k, k, pos, q, kk)
    Mb = brute_scores(N, B_k, q, kk)
    fin = np.isfinite(Mb)
    assert np.array_equal(np.isinf(M), np.isinf(Mb))
    assert np.array_equal(np.sign(M[~fin]), np.sign(Mb[~fin]))
    np.testing.assert_allclose(M[fin], Mb[fin], rtol=2e-6, atol=2e-5)
    bb, mb = brute_select(Mb, k)
    # The margin decides which rows the GPU must match exactly: it is the
    # fp64 brute force's gap between the (k-1)-th and k-th best non-local
    # scores, over the larger magnitude.  Sorted values are continuous in the
    # scores, so fp32 and fp64 agree to the scores' rounding even at near ties.
    assert np.array_equal(np.isinf(marg), np.isinf(mb))
    fm = np.isfinite(mb)
    assert fm.any() == (k >= 2 and N > k * B_k)
    np.testing.assert_allclose(marg[fm], mb[fm], rtol=0, atol=1e-5)
    sure = (mb > 1e-5) & (marg > 1e-5)
    assert sure.mean() > 0.9
    assert np.array_equal(bi[sure], bb[sure])


@pytest.mark.parametrize("N,H,d,k,first,window,seed,B_k", [
    (2048, 2, 64, 6, True, 1, 20, 128), (2048, 1, 64, 6, False, 3, 21, 128), (1500, 2, 128, 8, True, 4, 22, 128),
    (1000, 1, 64, 4, True, 3, 23, 128),                 # all k - 1 choices forced
    (900, 2, 64, 6, True, 2, 24, 32), (1100, 1, 128, 5, True, 2, 25, 64),
])
def test_forced_selection_matches_brute_force(N, H, d, k, first, window, seed, B_k):
    """Forced first block / local window: the forced blocks are always chosen,
    the remaining slots go to the best others (fp64 brute force with the
    forced blocks removed from the candidates)."""
    rng = np.random.default_rng(seed)
    q = _rand_bf16(rng, (N, H, d))
    kk = _rand_bf16(rng, (N, d))
    pos = np.arange(N)
    bi, marg, _ = oracle.index_topk(N, B_k, k, pos, q, kk, force_first=first, window=window)
    Mb = brute_scores(N, B_k, q, kk)
    checked = 0
    for r in range(H):
        for i in pos:
            L = i // B_k
            forced = ({0} if first and L >= 1 else set()) | set(range(max(0, L - window + 1), L + 1))
            got = [int(b) for b in bi[r, i] if b >= 0]
            assert got == sorted(got) and forced <= set(got), (r, i, got, forced)
            rest = [b for b in range(L) if b not in forced]
            free = min(k - len(forced), len(rest))
            order = sorted(rest, key=lambda b: (-Mb[i, r, b], b))
            cand = [Mb[i, r, b] for b in order]
            # margin: the gap between the last free choice and the best block
            # left out; +inf when no free slot or no block is left out
            if free < len(cand) and free > 0:
                a, b2 = cand[free - 1], cand[free]
                want = (a - b2) / max(abs(a), abs(b2), 1e-6)
                assert abs(marg[r, i] - want) <= 1e-5, (r, i, marg[r, i], want)
                if want <= 1e-5:
                    continue                            # near tie: fp32 vs fp64 order may differ
            else:
                assert marg[r, i] == np.inf, (r, i, marg[r, i])
            assert set(got) == forced | set(order[:free]), (r, i)
            assert len(got) == min(k, L + 1)
            checked += 1
    assert checked > 0.9 * H * N
    assert np.isfinite(marg).sum() + np.isinf(marg).sum() == marg.size   # no NaN margins


def test_margin_exact_values():
    """Hand-built score rows whose margin is known exactly: the (k-1)-th and
    k-th best non-local scores c_{k-1}, c_k give (c_{k-1} - c_k) /
    max(|c_{k-1}|, |c_k|, 1e-6).  Rows cover positive and negative scores,
    the 1e-6 floor, a tie (margin 0, smaller id kept), a forced block (+inf
    score) taking a slot, and too few candidates (+inf)."""
    inf = np.inf
    B_k = 128
    cases = [
        # scores of blocks 0..L-1, k, expected margin, expected ids
        ([3.0, -1.0, 2.0, 0.5, 2.5], 3, 0.5 / 2.5, [0, 4, 5]),
        ([-1.0, -4.0, -2.0], 2, 1.0 / 2.0, [0, 3]),
        ([-1.0, -4.0, -2.0], 3, 2.0 / 4.0, [0, 2, 3]),
        ([1e-7, 0.0, -1e-7], 2, 1e-7 / 1e-6, [0, 3]),
        ([0.25, 1.0, 0.25, -3.0], 3, 0.0, [0, 1, 4]),
        ([inf, 3.0, 1.0, 2.0], 3, 1.0 / 3.0, [0, 1, 4]),
        ([4.0, 8.0], 3, inf, [0, 1, 2]),
        ([4.0, 8.0, 1.0], 1, inf, [3]),
    ]
    for scores, k, want, ids in cases:
        L = len(scores)
        M = np.full((1, 1, L + 2), -inf, np.float32)
        M[0, 0, :L] = scores
        M[0, 0, L] = inf
        bi, marg = oracle.select(M, np.array([L * B_k + 5]), B_k, k)
        got = float(marg[0, 0])
        if np.isinf(want):
            assert got == inf, (scores, k, got)
        else:
            # the scores are stored in fp32 (1e-7 is not exact there); the
            # margin is fp64 arithmetic on them
            assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), (scores, k, got, want)
        assert bi[0, 0].tolist() == ids + [-1] * (k - len(ids)), (scores, k, bi[0, 0])


def test_window_selection_closed_form():
    """The sliding-window selection: block 0 plus the k - 1 blocks ending at L,
    k blocks in all (the top-k budget), or every block when L < k."""
    B_k, k = 128, 5
    pos = np.array([0, 127, 128, 600, 639, 640, 5000, 70000])
    sel = oracle.window_selection(pos, B_k, k, 3)
    assert sel.shape == (3, len(pos), k)
    for n, i in enumerate(pos):
        L = i // B_k
        row = [int(b) for b in sel[0, n] if b >= 0]
        assert row[0] == 0 and row[-1] == L and row == sorted(set(row))
        assert len(row) == min(k, L + 1)
        if L >= k:
            assert row[1:] == list(range(L - k + 2, L + 1))
        assert (sel[1, n] == sel[0, n]).all() and (sel[2, n] == sel[0, n]).all()


def test_selection_closed_forms():
    rng = np.random.default_rng(7)
    N, H, d, B_k = 1000, 2, 64, 128
    q = _rand_bf16(rng, (N, H, d))
    kk = _rand_bf16(rng, (N, d))
    pos = np.arange(N)
    L = pos // B_k
    # k >= L + 1: everything causal is selected
    bi, _, _ = oracle.index_topk(N, B_k, 8, pos, q, kk)
    for i in range(N):
        row = bi[:, i, :]
        assert np.array_equal(row[:, : L[i] + 1], np.tile(np.arange(L[i] + 1), (H, 1)))
        assert (row[:, L[i] + 1:] == -1).all()
    # k = 1: only the local block
    bi, marg, _ = oracle.index_topk(N, B_k, 1, pos, q, kk)
    assert np.array_equal(bi[:, :, 0], np.tile(L, (H, 1)))
    assert np.isinf(marg).all()
    # general k: ascending, unique, local block is the last valid entry
    bi, _, _ = oracle.index_topk(N, B_k, 3, pos, q, kk)
    for r in range(H):
        for i in range(N):
            v = bi[r, i][bi[r, i] >= 0]
            assert len(v) == min(3, L[i] + 1)
            assert (np.diff(v) > 0).all() and v[-1] == L[i]
            assert (bi[r, i][len(v):] == -1).all()


def test_selection_planted_answer():
    """Q^idx = u, K^idx = 0 except block b* where it is 10 u: every query after
    block b* picks b*; the other picks are the smallest ids (all tied at 0)."""
    N, H, d, B_k, k, bstar = 2048, 2, 64, 128, 4, 6
    u = np.zeros(d, np.float32)
    u[::3] = 0.5
    q = np.tile(synth.f32_to_bf16_bits(u), (N, H, 1))
    kk = np.zeros((N, d), np.uint16)
    kk[bstar * B_k:(bstar + 1) * B_k] = synth.f32_to_bf16_bits(10 * u)
    pos = np.arange(N)
    bi, _, _ = oracle.index_topk(N, B_k, k, pos, q, kk)
    for i in range(N):
        L = i // B_k
        if L > bstar:
            want = sorted([bstar] + [b for b in range(L) if b != bstar][: k - 2] + [L])
        else:
            want = list(range(min(L, k - 1))) + [L]
        assert bi[0, i].tolist() == want + [-1] * (k - len(want)), i


def test_scale_does_not_change_selection():
    """Selection is order-only: a positive rescale of Q^idx (by 2, exact in bf16)
    selects the same blocks."""
    rng = np.random.default_rng(8)
    N, H, d, B_k, k = 1536, 2, 64, 128, 5
    q = _rand_bf16(rng, (N, H, d))
    kk = _rand_bf16(rng, (N, d))
    q2 = synth.f32_to_bf16_bits(2 * synth.bf16_bits_to_f32(q))
    a, _, _ = oracle.index_topk(N, B_k, k, np.arange(N), q, kk)
    b, _, _ = oracle.index_topk(N, B_k, k, np.arange(N), q2, kk)
    assert np.array_equal(a, b)


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(9)
    N, H, d, B_k, k = 1300, 2, 64, 128, 4
    q = _rand_bf16(rng, (N, H, d))
    kk = _rand_bf16(rng, (N, d))
    full, _, _ = oracle.index_topk(N, B_k, k, np.arange(N), q, kk)
    rows = np.array([0, 5, 127, 128, 777, 1299])
    part, _, _ = oracle.index_topk(N, B_k, k, rows, q[rows], kk)
    assert np.array_equal(part, full[:, rows, :])


# ---------------------------------------------------------------- main branch

def _sdpa_masked(q, K, V, mask, scale):
    """Library attention (fp64, CPU).  q [n, Hq, d]; K, V [N, Hq, d] (already
    repeated per head); mask [Hq, n, N] boolean (True = attend)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask)[None], scale=scale)
    s = (qt @ kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.from_numpy(mask)[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def _make_attn_inputs(rng, N, Hq, Hkv, d):
    q = _rand_bf16(rng, (N, Hq, d))
    K = _rand_bf16(rng, (N, Hkv, d))
    V = _rand_bf16(rng, (N, Hkv, d))
    return q, K, V


def _rand_selection(rng, N, Hkv, B_k, k):
    bi = np.full((Hkv, N, k), -1, np.int32)
    for r in range(Hkv):
        for i in range(N):
            L = i // B_k
            others = rng.permutation(L)[: k - 1] if L else np.zeros(0, int)
            v = sorted(list(others) + [L])
            bi[r, i, : len(v)] = v
    return bi


def test_attention_full_budget_is_dense_causal_gqa():
    """k * B_k >= N selects every causal block: MSA equals dense causal GQA."""
    rng = np.random.default_rng(10)
    N, Hq, Hkv, d, B_k, k = 700, 4, 2, 32, 128, 6
    G = Hq // Hkv
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    bi = _rand_selection(rng, N, Hkv, B_k, k)          # k-1 >= L for all rows
    pos = np.arange(N)
    O, lse = oracle.attention(N, B_k, pos, q, K, V, bi, softmax_scale=d ** -0.5)
    qt = torch.from_numpy(_f32(q)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(_f32(K)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(_f32(V)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=d ** -0.5)
    np.testing.assert_allclose(O, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,Hq,Hkv,rows", [(300, 4, 2, None), (261, 8, 1, [0, 1, 127, 128, 200, 260]),
                                           (129, 2, 2, [128])])
def test_dense_attention_is_library_causal_gqa(N, Hq, Hkv, rows):
    """The dense baseline's oracle equals library causal attention with K/V
    repeated over each group's heads, for all rows or a subset (ragged N)."""
    rng = np.random.default_rng(N + Hq)
    d, B_k = 32, 128
    G = Hq // Hkv
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    pos = np.arange(N) if rows is None else np.array(rows)
    O, lse = oracle.dense_attention(N, B_k, pos, q[pos], K, V, softmax_scale=0.2)
    mask = np.tril(np.ones((N, N), bool))[None].repeat(Hq, axis=0)
    ref, ref_lse = _sdpa_masked(_f32(q), np.repeat(_f32(K), G, axis=1),
                                np.repeat(_f32(V), G, axis=1), mask, 0.2)
    np.testing.assert_allclose(O, ref[pos], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[pos], rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,Hq,Hkv,k,seed,B_k", [(900, 4, 2, 3, 11, 128), (1024, 6, 3, 2, 12, 128),
                                                (513, 2, 1, 4, 13, 128), (450, 4, 2, 3, 16, 32),
                                                (700, 2, 1, 5, 17, 64)])
def test_attention_matches_masked_library_attention(N, Hq, Hkv, k, seed, B_k):
    rng = np.random.default_rng(seed)
    d = 32
    G = Hq // Hkv
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    bi = _rand_selection(rng, N, Hkv, B_k, k)
    pos = np.arange(N)
    O, lse = oracle.attention(N, B_k, pos, q, K, V, bi, softmax_scale=0.3)
    mask = np.zeros((Hq, N, N), bool)
    blk = np.arange(N) // B_k
    for h in range(Hq):
        r = h // G
        for i in range(N):
            sel = bi[r, i][bi[r, i] >= 0]
            mask[h, i] = np.isin(blk, sel) & (np.arange(N) <= i)
    ref, ref_lse = _sdpa_masked(_f32(q), np.repeat(_f32(K), G, axis=1),
                                np.repeat(_f32(V), G, axis=1), mask, 0.3)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,Hq,Hkv,Hsel,k,seed", [(700, 8, 2, 4, 3, 31), (520, 8, 1, 8, 2, 32),
                                                 (900, 16, 4, 8, 4, 33)])
def test_attention_with_more_index_heads_than_kv_heads(N, Hq, Hkv, Hsel, k, seed):
    """H_sel index heads > H_kv: head h follows the selection of index head
    h // (Hq / Hsel) and reads K/V head h // (Hq / Hkv) (library attention with
    a per-head block mask)."""
    rng = np.random.default_rng(seed)
    d, B_k = 32, 128
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    bi = _rand_selection(rng, N, Hsel, B_k, k)
    pos = np.arange(N)
    O, lse = oracle.attention(N, B_k, pos, q, K, V, bi, softmax_scale=0.3)
    mask = np.zeros((Hq, N, N), bool)
    blk = np.arange(N) // B_k
    for h in range(Hq):
        m = h // (Hq // Hsel)
        for i in range(N):
            sel = bi[m, i][bi[m, i] >= 0]
            mask[h, i] = np.isin(blk, sel) & (np.arange(N) <= i)
    G = Hq // Hkv
    ref, ref_lse = _sdpa_masked(_f32(q), np.repeat(_f32(K), G, axis=1),
                                np.repeat(_f32(V), G, axis=1), mask, 0.3)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_attention_first_query_returns_first_value():
    rng = np.random.default_rng(14)
    N, Hq, Hkv, d, B_k, k = 300, 4, 2, 16, 128, 2
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    bi = _rand_selection(rng, N, Hkv, B_k, k)
    O, lse = oracle.attention(N, B_k, np.array([0]), q[:1], K, V, bi[:, :1], softmax_scale=0.25)
    for h in range(Hq):
        r = h // 2
        assert np.array_equal(O[0, h], _f32(V[0, r]))
        assert lse[0, h] == pytest.approx(0.25 * float(_f32(q[0, h]) @ _f32(K[0, r])), abs=1e-12)


def test_attention_fp8_decodes_with_scales():
    """fp8 path: codes times per-tensor scales; with all scales 1 it equals the
    bf16 path on the same (exactly representable) values."""
    rng = np.random.default_rng(15)
    N, Hq, Hkv, d, B_k, k = 400, 2, 1, 16, 128, 2
    codes = rng.integers(0, 256, size=(3, N, Hkv, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38            # drop NaN codes
    qc = rng.integers(0, 256, size=(N, Hq, d)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x38
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    qv = torch.from_numpy(qc).view(torch.float8_e4m3fn).float()
    to_bf = lambda t: t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bi = _rand_selection(rng, N, Hkv, B_k, k)
    pos = np.arange(N)
    O8, l8 = oracle.attention(N, B_k, pos, qc, codes[0], codes[1], bi, 0.01, dtype=oracle.FP8)
    Ob, lb = oracle.attention(N, B_k, pos, to_bf(qv), to_bf(vals[0]), to_bf(vals[1]), bi, 0.01)
    assert np.array_equal(O8, Ob) and np.array_equal(l8, lb)
    O8s, l8s = oracle.attention(N, B_k, pos, qc, codes[0], codes[1], bi, 0.01, dtype=oracle.FP8,
                                q_scale=0.5, k_scale=2.0, v_scale=0.25)
    np.testing.assert_allclose(O8s, 0.25 * Ob, rtol=1e-14, atol=0)
    np.testing.assert_allclose(l8s, lb, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- combine

def test_combine_reproduces_direct_softmax():
    """Attention split per selected block, merged by LSE, equals attention over
    the union (up to the bf16 rounding of the stored partials)."""
    rng = np.random.default_rng(16)
    N, Hq, Hkv, d, B_k, k = 1024, 4, 2, 32, 128, 5
    G = Hq // Hkv
    q, K, V = _make_attn_inputs(rng, N, Hq, Hkv, d)
    bi = _rand_selection(rng, N, Hkv, B_k, k)
    pos = np.arange(N)
    O, lse = oracle.attention(N, B_k, pos, q, K, V, bi, softmax_scale=0.2)
    # per-slot partials: attention restricted to one block each
    o_part = np.zeros((Hkv, N, k, G, d), np.uint16)
    l_part = np.zeros((Hkv, N, k, G), np.float32)
    exact = np.zeros((Hkv, N, k, G, d))
    for s in range(k):
        one = np.full_like(bi, -1)
        one[:, :, 0] = bi[:, :, s]
        valid = bi[:, :, s] >= 0
        one[:, :, 0] = np.where(valid, bi[:, :, s], bi[:, :, 0])   # placeholder for empty
        Os, ls = oracle.attention(N, B_k, pos, q, K, V, one, softmax_scale=0.2)
        for r in range(Hkv):
            exact[r, :, s] = Os[:, r * G:(r + 1) * G]
            o_part[r, :, s] = synth.f32_to_bf16_bits(Os[:, r * G:(r + 1) * G].astype(np.float32))
            l_part[r, :, s] = ls[:, r * G:(r + 1) * G]
    Oc, lc = oracle.combine(bi, o_part, l_part)
    np.testing.assert_allclose(lc, lse, rtol=0, atol=2e-6)
    bound = np.abs(exact).max() * 2.0 ** -8 + 1e-6
    assert np.abs(Oc - O).max() <= bound


def test_combine_single_slot_and_equal_weights():
    rng = np.random.default_rng(17)
    Hkv, n, k, G, d = 2, 5, 3, 2, 8
    bi = np.full((Hkv, n, k), -1, np.int32)
    bi[:, :, 0] = 0
    o = synth.f32_to_bf16_bits(rng.standard_normal((Hkv, n, k, G, d)).astype(np.float32))
    lp = rng.standard_normal((Hkv, n, k, G)).astype(np.float32)
    O, lse = oracle.combine(bi, o, lp)
    for r in range(Hkv):
        assert np.array_equal(O[:, r * G:(r + 1) * G], _f32(o[r, :, 0]))
        assert np.array_equal(lse[:, r * G:(r + 1) * G], lp[r, :, 0].astype(np.float64))
    bi[:, :, 1] = 1
    lp[:, :, 1] = lp[:, :, 0]
    O, lse = oracle.combine(bi, o, lp)
    for r in range(Hkv):
        want = 0.5 * (_f32(o[r, :, 0]) + _f32(o[r, :, 1]))
        np.testing.assert_allclose(O[:, r * G:(r + 1) * G], want, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(lse[:, r * G:(r + 1) * G],
                                   lp[r, :, 0].astype(np.float64) + np.log(2), rtol=1e-15)


# ---------------------------------------------------------------- inversion

def test_inversion_matches_stable_sort():
    rng = np.random.default_rng(18)
    n_seq, n, k, B_k = 3, 777, 6, 128
    B = -(-n // B_k)
    bi = np.stack([_rand_selection(rng, n, 1, B_k, k)[0] for _ in range(n_seq)])
    off, ent = oracle.invert(bi, B)
    # library stable sort of the flat (seq, block) keys, in (row, slot) order
    flat = bi.reshape(n_seq, -1)
    want = []
    for q in range(n_seq):
        valid = np.nonzero(flat[q] >= 0)[0]
        order = np.argsort(flat[q][valid], kind="stable")
        want.append(valid[order])
    want = np.concatenate(want).astype(np.int32)
    assert np.array_equal(ent, want)
    counts = np.stack([np.bincount(flat[q][flat[q] >= 0], minlength=B) for q in range(n_seq)])
    assert np.array_equal(np.diff(off, axis=1), counts)
    assert off[0, 0] == 0 and (off[1:, 0] == off[:-1, -1]).all()
    assert off[-1, -1] == (bi >= 0).sum()
