"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Small cases compare every row; the full-size workloads compare sampled rows in
the same launch configuration the benchmark times (msa_forward over the whole
sequence, or over 32,768-row chunks for the 1M case).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_idx_amd as msa
import oracle
import synth
from gpu_util import (admissible, check_selection, compact_attention_rows, device_inputs,
                      dims_of, err_stats, log, opts_of, oracle_index_rows, sample_rows)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TINY = synth.TINY


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not msa.LIB_PATH or not __import__("os").path.exists(msa.LIB_PATH):
        pytest.fail("libmsa.so is not built")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- inputs

def test_device_generator_matches_host():
    for w in (TINY.with_(N=1000, plant=4), TINY.with_(N=640, dtype="fp8"),
              TINY.with_(N=768, plant=3, batch=3)):             # planting per sequence
        log(f"generator {w.name} N={w.N} dtype={w.dtype} plant={w.plant}")
        t = device_inputs(w, DEV)
        rows = np.array([0, 5, 127, 128, 300, w.N - 1])
        rows = np.concatenate([rows + b * w.N for b in range(w.batch)])
        for x in ("q", "k", "v", "q_idx", "k_idx"):
            dv = t[x]
            dv = dv.view(torch.int16) if dv.dtype == torch.bfloat16 else dv
            got = dv.cpu().numpy().reshape(w.batch * w.N, -1)[rows]
            want = synth.host_rows(w, x, rows).reshape(len(rows), -1)
            assert np.array_equal(got.view(want.dtype), want), x


# --------------------------------------------------------------------------- index branch

INDEX_CASES = [
    TINY,
    TINY.with_(N=1000),                                   # ragged last block
    TINY.with_(N=1),
    TINY.with_(N=100),
    TINY.with_(k=1),
    TINY.with_(k=2, d_idx=128),
    TINY.with_(k=16),                                     # k * B_k >= N: all causal blocks
    TINY.with_(N=5000, k=32, d_idx=128),
    TINY.with_(N=3000, k=7, H_q=4, H_kv=1),
    TINY.with_(N=2500, k=5, H_q=64, H_kv=4, d_idx=128),
    TINY.with_(N=2000, k=4, H_q=16, H_kv=2, H_idx=8),       # more index heads than K/V heads
    TINY.with_(N=1500, k=6, B_k=64),                        # 64-token blocks
    TINY.with_(N=1000, k=8, B_k=32, d_idx=128),             # 32-token blocks
    # 32-token blocks with one free slot: every score of the ring's blocks
    # decides the selection (the ring's buffer stride must hold the last DMA
    # instruction of a block, which reaches past a 4.5 / 8.5 KB tile)
    TINY.with_(N=521, k=2, H_q=4, H_kv=2, B_k=32, d_idx=64, batch=2),
    TINY.with_(N=777, k=2, B_k=32, d_idx=128),
    TINY.with_(batch=2, N=1300),
]


@pytest.mark.parametrize("w", INDEX_CASES, ids=lambda w: f"N{w.N}_hsel{w.H_sel}_d{w.d_idx}_k{w.k}_bk{w.B_k}_b{w.batch}")
def test_index_topk_parity(w):
    log(f"index_topk N={w.N} H_kv={w.H_kv} d_idx={w.d_idx} k={w.k} batch={w.batch}")
    t = device_inputs(w, DEV)
    d = dims_of(w)
    bi = msa.msa_index_topk(d, t["q_idx"], t["k_idx"]).cpu().numpy()
    rows = np.arange(w.N)
    for b in range(w.batch):
        ob, marg, M = oracle_index_rows(w, rows, bat=b)
        st = check_selection(bi[b], ob, marg, M, w.k, what=f"batch {b}")
        log(f"  batch {b}: {st}")


def test_index_topk_chunk_offsets():
    """A range [q_begin, q_begin + q_count) gives the rows of the full call."""
    w = TINY.with_(N=3000, k=6)
    t = device_inputs(w, DEV)
    d = dims_of(w)
    full = msa.msa_index_topk(d, t["q_idx"], t["k_idx"]).cpu().numpy()
    for qb, qn in ((0, 640), (640, 1000), (2048, 952), (2944, 56)):
        log(f"index_topk range {qb}+{qn}")
        part = msa.msa_index_topk(d, t["q_idx"], t["k_idx"], qb, qn).cpu().numpy()
        assert np.array_equal(part, full[:, :, qb:qb + qn])


# --------------------------------------------------------------------------- inversion

def _random_selection(rng, H, n, q_begin, B_k, k, hot=None):
    out = np.full((H, n, k), -1, np.int32)
    for r in range(H):
        for j in range(n):
            L = (q_begin + j) // B_k
            if L == 0:
                out[r, j, 0] = 0
                continue
            p = np.ones(L)
            if hot is not None:
                p[hot[hot < L]] *= 20.0
            p /= p.sum()
            others = rng.choice(L, size=min(k - 1, L), replace=False, p=p)
            v = np.sort(np.concatenate([others, [L]]))
            out[r, j, :len(v)] = v
    return out


@pytest.mark.parametrize("batch,H,N,q_begin,q_count,k,G", [
    (1, 2, 2048, 0, 2048, 4, 4), (1, 4, 3000, 0, 3000, 16, 16), (2, 2, 1500, 512, 988, 5, 2),
    (1, 1, 9000, 8192, 808, 8, 1), (1, 3, 700, 0, 700, 32, 8),
])
def test_invert_parity(batch, H, N, q_begin, q_count, k, G):
    log(f"invert batch={batch} H_kv={H} N={N} range={q_begin}+{q_count} k={k} G={G}")
    rng = np.random.default_rng(N + k)
    B_c = -(-(q_begin + q_count) // 128)
    hot = rng.choice(B_c, size=min(4, B_c), replace=False)
    sel = np.stack([_random_selection(rng, H, q_count, q_begin, 128, k, hot) for _ in range(batch)])
    d = msa.make_dims(batch, N, H * G, H, 128, 64, 128, k)
    bi = torch.from_numpy(sel).to(DEV)
    off, ent, sched = msa.msa_invert_blocks(d, bi, q_begin, q_count)
    assert msa.msa_invert_status(sched) == 0
    ooff, oent = oracle.invert(sel.reshape(batch * H, q_count, k), B_c)
    assert np.array_equal(off.cpu().numpy().reshape(batch * H, B_c + 1), ooff)
    assert np.array_equal(ent.cpu().numpy()[: len(oent)], oent)


def test_invert_counts_out_of_range_ids():
    w = TINY.with_(N=1024, k=4)
    rng = np.random.default_rng(3)
    sel = _random_selection(rng, 2, 1024, 0, 128, 4)
    sel[0, 500, 0] = 9          # beyond the row's local block
    sel[1, 7, 1] = -5           # negative, not the -1 padding
    d = dims_of(w)
    off, ent, sched = msa.msa_invert_blocks(d, torch.from_numpy(sel[None]).to(DEV))
    assert msa.msa_invert_status(sched) == 2
    keep = sel.copy()
    keep[0, 500, 0] = -1
    keep[1, 7, 1] = -1
    ooff, oent = oracle.invert(keep, 8)
    assert np.array_equal(off.cpu().numpy().reshape(2, 9), ooff)
    assert np.array_equal(ent.cpu().numpy()[: len(oent)], oent)


# --------------------------------------------------------------------------- attention + combine

ATTN_CASES = [
    TINY,
    TINY.with_(N=1000, k=3),
    TINY.with_(N=700, k=2, H_q=2, H_kv=2),               # G = 1
    TINY.with_(N=900, k=5, H_q=4, H_kv=2),               # G = 2
    TINY.with_(N=1200, k=4, H_q=16, H_kv=2),             # G = 8
    TINY.with_(N=1536, k=16, H_q=32, H_kv=2),            # G = 16, all causal blocks
    TINY.with_(N=777, k=4, dtype="fp8"),
    TINY.with_(N=1300, k=4, batch=2, H_q=16, H_kv=4),
    TINY.with_(N=1100, k=4, H_q=16, H_kv=2, H_idx=4),     # index heads: 2 per K/V head, G_sel = 4
    TINY.with_(N=900, k=3, H_q=16, H_kv=2, H_idx=16, batch=2),   # one index head per query head
    TINY.with_(N=1000, k=6, B_k=64),                      # 64-token blocks
    TINY.with_(N=700, k=9, B_k=32, H_q=32, H_kv=2),       # 32-token blocks, G = 16
]


def _oracle_partials(w, sel, rows):
    """Oracle partial (Obar, lse) of every (row, slot): attention over that one block."""
    H = w.H_sel
    code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
    sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
    q = synth.host_rows(w, "q", rows)
    K = synth.host_all(w, "k")[: w.N]
    V = synth.host_all(w, "v")[: w.N]
    parts = []
    for s in range(w.k):
        one = np.full((H, len(rows), w.k), -1, np.int32)
        one[:, :, 0] = sel[:, :, s]
        valid = sel[:, :, s] >= 0
        one[:, :, 0] = np.where(valid, sel[:, :, s], sel[:, :, 0])
        O, lse = oracle.attention(w.N, w.B_k, rows, q, K, V, one, dtype=code, q_scale=sc,
                                  k_scale=sc, v_scale=sc)
        parts.append((O, lse, valid))
    return parts


@pytest.mark.parametrize("w", ATTN_CASES, ids=lambda w: f"N{w.N}_G{w.G}_Gs{w.G_sel}_k{w.k}_bk{w.B_k}_{w.dtype}_b{w.batch}")
def test_attention_and_combine_parity(w):
    """Feed the oracle's selection to the GPU inversion, attention and combine."""
    log(f"attention N={w.N} H_q={w.H_q} H_kv={w.H_kv} k={w.k} dtype={w.dtype} batch={w.batch}")
    t = device_inputs(w, DEV)
    d, o = dims_of(w), opts_of(w)
    tol_max = 6e-2 if w.dtype == "fp8" else 2e-2
    rows = np.arange(w.N)
    sels = []
    for b in range(w.batch):
        ob, _, _ = oracle_index_rows(w, rows, bat=b)
        sels.append(ob)
    sel = np.stack(sels)
    bi = torch.from_numpy(sel).to(DEV)
    off, ent, sched = msa.msa_invert_blocks(d, bi)
    q, k, v = t["q"], t["k"], t["v"]
    opart, lpart = msa.msa_sparse_attn_fwd(d, o, q, k, v, off, ent, sched)
    out, lse = msa.msa_combine(d, bi, opart, lpart, want_lse=True)
    torch.cuda.synchronize()
    opart = opart.float().cpu().numpy()
    lpart = lpart.cpu().numpy()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    G = w.G_sel
    for b in range(w.batch):
        # partials per slot (batch 0 only: the oracle helper reads batch-0 rows)
        if b == 0:
            for s, (Os, ls, valid) in enumerate(_oracle_partials(w, sel[0], rows)):
                for r in range(w.H_sel):
                    m = valid[r]
                    if not m.any():                               # slot empty in every row
                        continue
                    got = opart[0, r, m, s]                       # [n, G, d_h]
                    ref = Os[m][:, r * G:(r + 1) * G]
                    mx, mn = err_stats(got, ref)
                    assert mx <= tol_max and mn <= 2e-3, (s, r, mx, mn)
                    lmx, _ = err_stats(lpart[0, r, m, s], ls[m][:, r * G:(r + 1) * G])
                    assert lmx <= 1e-3, (s, r, lmx)
        code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
        sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
        flat = b * w.N + rows
        O, L = oracle.attention(w.N, w.B_k, rows, synth.host_rows(w, "q", flat),
                                synth.host_rows(w, "k", b * w.N + np.arange(w.N)),
                                synth.host_rows(w, "v", b * w.N + np.arange(w.N)), sel[b],
                                dtype=code, q_scale=sc, k_scale=sc, v_scale=sc)
        mx, mn = err_stats(out[b], O, label="O")
        log(f"  batch {b}: output max abs {mx:.3g} mean abs {mn:.3g}")
        assert mx <= tol_max and mn <= 2e-3
        lmx, _ = err_stats(lse[b], L)
        assert lmx <= 1e-3


def test_fp8_every_code_attention_parity():
    """fp8 Q, K and V drawn uniformly from every finite e4m3 code (subnormals,
    zeros of both signs and +-448 included), so the score MFMAs, which take
    the codes as they are, meet every value; each row attends to all of its
    visible blocks (N = 500: a partial last block), G = 16."""
    N, H_q, H_kv, d_h, B_k, k = 500, 16, 1, 128, 128, 4
    log(f"fp8 every-code attention N={N} G={H_q // H_kv}")
    rng = np.random.default_rng(20261203)

    def codes(shape):
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] -= 1          # the two NaN codes become +-448
        return c

    q, kk, vv = codes((N, H_q, d_h)), codes((N, H_kv, d_h)), codes((N, H_kv, d_h))
    s = 1.0 / 256                            # decoded values within +-1.75
    rows = np.arange(N)
    sel = np.full((1, N, k), -1, np.int32)   # every visible block, ascending
    for i in rows:
        L = i // B_k
        sel[0, i, :L + 1] = np.arange(L + 1)
    d = msa.make_dims(1, N, H_q, H_kv, d_h, 128, B_k, k)
    o = msa.make_opts("fp8", q_scale=s, k_scale=s, v_scale=s)
    tq, tk, tv = (torch.from_numpy(x[None]).to(DEV) for x in (q, kk, vv))
    bi = torch.from_numpy(sel[None]).to(DEV)
    off, ent, sched = msa.msa_invert_blocks(d, bi)
    opart, lpart = msa.msa_sparse_attn_fwd(d, o, tq, tk, tv, off, ent, sched)
    out, lse = msa.msa_combine(d, bi, opart, lpart, want_lse=True)
    torch.cuda.synchronize()
    O, L = oracle.attention(N, B_k, rows, q, kk, vv, sel, dtype=oracle.FP8, q_scale=s, k_scale=s,
                            v_scale=s)
    mx, mn = err_stats(out[0].float().cpu().numpy(), O, label="O")
    log(f"  output max abs {mx:.3g} mean abs {mn:.3g}")
    assert mx <= 6e-2 and mn <= 2e-3
    lmx, _ = err_stats(lse[0].cpu().numpy(), L)
    assert lmx <= 1e-3


def test_combine_parity_random_partials():
    rng = np.random.default_rng(21)
    H, n, k, G = 2, 300, 6, 4
    w = TINY.with_(N=n, k=k, H_q=H * G, H_kv=H)
    sel = _random_selection(rng, H, n, 0, 128, k)
    op = synth.f32_to_bf16_bits(rng.standard_normal((H, n, k, G, 128)).astype(np.float32))
    lp = (3.0 * rng.standard_normal((H, n, k, G))).astype(np.float32)
    d = dims_of(w)
    bi = torch.from_numpy(sel[None]).to(DEV)
    opt = torch.from_numpy(op.view(np.int16)[None].copy()).to(DEV).view(torch.bfloat16)
    lpt = torch.from_numpy(lp[None]).to(DEV)
    out, lse = msa.msa_combine(d, bi, opt, lpt, want_lse=True)
    O, L = oracle.combine(sel, op, lp)
    mx, mn = err_stats(out.float().cpu().numpy()[0], O, label="O")
    assert mx <= 2e-2 and mn <= 2e-3
    lmx, _ = err_stats(lse.cpu().numpy()[0], L)
    assert lmx <= 1e-5


def test_combine_never_reads_invalid_slots():
    """Partial buffers prefilled with NaN: slots the attention pass does not
    write (-1 padding, an id past the row's local block, a negative id, a row
    with no valid slot) must never reach O.  O equals a run on zeroed buffers
    bit for bit and the oracle on the selection with those slots dropped."""
    w = TINY.with_(N=1500, k=6)
    log(f"NaN-poisoned partials N={w.N} H_q={w.H_q} H_kv={w.H_kv} k={w.k}")
    t = device_inputs(w, DEV)
    d, o = dims_of(w), opts_of(w)
    rows = np.arange(w.N)
    sel, _, _ = oracle_index_rows(w, rows)
    sel = sel.copy()
    assert (sel == -1).any()                     # early rows are padded
    sel[0, 700, 0] = 11                          # past the row's local block (5)
    sel[1, 900, 2] = -7                          # negative, not the -1 padding
    sel[0, 1000, :] = -1                         # no valid slot at all
    bi = torch.from_numpy(sel[None]).to(DEV)
    off, ent, sched = msa.msa_invert_blocks(d, bi)
    assert msa.msa_invert_status(sched) == 2
    shp = (1, w.H_sel, w.N, w.k, w.G_sel)
    outs = []
    for fill in (float("nan"), 0.0):
        op = torch.full(shp + (w.d_h,), fill, dtype=torch.bfloat16, device=DEV)
        lp = torch.full(shp, fill, dtype=torch.float32, device=DEV)
        msa.msa_sparse_attn_fwd(d, o, t["q"], t["k"], t["v"], off, ent, sched, o_part=op, lse_part=lp)
        out, lse = msa.msa_combine(d, bi, op, lp, want_lse=True)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    (o_nan, l_nan), (o_zero, l_zero) = outs
    assert np.array_equal(o_nan, o_zero)
    assert np.array_equal(l_nan.view(np.int32), l_zero.view(np.int32))
    of = synth.bf16_bits_to_f32(o_nan.view(np.uint16))[0]
    assert np.isfinite(of).all()
    G = w.G_sel
    assert (of[1000, 0:G] == 0).all() and np.isneginf(l_nan[0, 1000, 0:G]).all()
    clean = sel.copy()
    clean[0, 700, 0] = -1
    clean[1, 900, 2] = -1
    keep = np.setdiff1d(rows, [1000])
    O, L = oracle.attention(w.N, w.B_k, keep, synth.host_rows(w, "q", keep), synth.host_all(w, "k"),
                            synth.host_all(w, "v"), np.ascontiguousarray(clean[:, keep]))
    mx, mn = err_stats(of[keep], O, label="O")
    assert mx <= 2e-2 and mn <= 2e-3
    lmx, _ = err_stats(l_nan[0, keep], L)
    assert lmx <= 1e-3


# --------------------------------------------------------------------------- whole forward

FWD_CASES = [TINY, TINY.with_(N=1000, k=5), TINY.with_(N=2304, k=4, q_chunk=512),
             TINY.with_(N=3000, H_q=32, H_kv=2, k=8, d_idx=128, dtype="fp8"),
             TINY.with_(N=1800, H_q=32, H_kv=2, H_idx=8, k=5, q_chunk=768),
             TINY.with_(N=1300, k=10, B_k=64, q_chunk=512),
             TINY.with_(N=900, k=12, B_k=32, H_q=64, H_kv=4, d_idx=128)]


@pytest.mark.parametrize("w", FWD_CASES, ids=lambda w: f"N{w.N}_k{w.k}_{w.dtype}_chunk{w.q_chunk}")
def test_forward_parity(w):
    log(f"forward N={w.N} k={w.k} dtype={w.dtype} q_chunk={w.q_chunk}")
    t = device_inputs(w, DEV)
    d, o = dims_of(w), opts_of(w)
    bi = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_forward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"],
                                  block_idx_out=bi, want_lse=True)
    torch.cuda.synchronize()
    gsel = bi.cpu().numpy()[0]
    rows = np.arange(w.N)
    ob, marg, M = oracle_index_rows(w, rows)
    st = check_selection(gsel, ob, marg, M, w.k, what="forward")
    log(f"  selection: {st}")
    code = oracle.FP8 if w.dtype == "fp8" else oracle.BF16
    sc = synth.fp8_scale() if w.dtype == "fp8" else 1.0
    O, L = oracle.attention(w.N, w.B_k, rows, synth.host_all(w, "q"), synth.host_all(w, "k"),
                            synth.host_all(w, "v"), gsel, dtype=code, q_scale=sc, k_scale=sc,
                            v_scale=sc)
    mx, mn = err_stats(out.float().cpu().numpy()[0], O, label="O")
    log(f"  output max abs {mx:.3g} mean abs {mn:.3g}")
    assert mx <= (6e-2 if w.dtype == "fp8" else 2e-2) and mn <= 2e-3
    lmx, _ = err_stats(lse.cpu().numpy()[0], L)
    assert lmx <= 1e-3


def test_forward_chunked_equals_whole_and_deterministic():
    w = TINY.with_(N=2560, k=6)
    t = device_inputs(w, DEV)
    d = dims_of(w)
    args = (t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"])
    a, _, _ = msa.msa_forward(d, msa.make_opts(), *args)
    b, _, _ = msa.msa_forward(d, msa.make_opts(), *args)
    c, _, _ = msa.msa_forward(d, msa.make_opts(q_chunk=768), *args)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


DEFAULT_PASS_CASES = [
    TINY.with_(N=msa.DEFAULT_Q_CHUNK + 2560, k=6),
    TINY.with_(N=msa.DEFAULT_Q_CHUNK + 1000, H_q=32, H_kv=2, k=8, d_idx=128, dtype="fp8"),
    TINY.with_(N=2 * msa.DEFAULT_Q_CHUNK + 700, k=10, B_k=64),
    TINY.with_(N=msa.DEFAULT_Q_CHUNK + 300, H_q=32, H_kv=2, H_idx=8, k=5),
]


@pytest.mark.parametrize("w", DEFAULT_PASS_CASES, ids=lambda w: f"N{w.N}_k{w.k}_bk{w.B_k}_{w.dtype}_hidx{w.H_idx}")
def test_forward_default_chunks_equal_single_pass(w):
    """q_chunk 0 runs msa.DEFAULT_Q_CHUNK rows per pass (here two or three
    passes, the last ragged): output, LSE and selection bit for bit those of
    one pass over all rows."""
    log(f"forward default chunks N={w.N} k={w.k} B_k={w.B_k} {w.dtype} H_idx={w.H_idx}")
    t = device_inputs(w, DEV)
    d = dims_of(w)
    args = (t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"])
    runs = []
    one_pass = -(-w.N // w.B_k) * w.B_k        # a multiple of B_k covering all rows
    for qc in (0, one_pass):
        o = opts_of(w)
        o.q_chunk = qc
        bi = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
        out, lse, _ = msa.msa_forward(d, o, *args, block_idx_out=bi, want_lse=True)
        runs.append((out, lse, bi, msa.msa_workspace_size(d, o)))
    (a, la, ba, wa), (b, lb, bb, wb) = runs
    assert wa < wb
    assert torch.equal(ba, bb)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la, lb)


# --------------------------------------------------------------------------- selection variants

FORCED_CASES = [
    (TINY.with_(N=3000, k=6), True, 1),
    (TINY.with_(N=3000, k=6, d_idx=128), False, 3),
    (TINY.with_(N=2500, k=8, H_q=64, H_kv=4, d_idx=128, batch=2), True, 4),
    (TINY.with_(N=1000, k=4), True, 3),                 # every free slot forced
]


@pytest.mark.parametrize("w,first,window", FORCED_CASES,
                         ids=lambda x: f"N{x.N}_k{x.k}_b{x.batch}" if hasattr(x, "N") else str(x))
def test_forced_index_parity(w, first, window):
    log(f"forced index N={w.N} k={w.k} first={first} window={window} batch={w.batch}")
    t = device_inputs(w, DEV)
    bi = msa.msa_index_topk_forced(dims_of(w), t["q_idx"], t["k_idx"], force_first=first,
                                   local_window=window)
    torch.cuda.synchronize()
    gsel = bi.cpu().numpy()
    rows = np.arange(w.N)
    for b in range(w.batch):
        flat = b * w.N + rows
        ob, marg, M = oracle.index_topk(w.N, w.B_k, w.k, rows, synth.host_rows(w, "q_idx", flat),
                                        synth.host_rows(w, "k_idx", b * w.N + np.arange(w.N)),
                                        force_first=first, window=window)
        st = check_selection(gsel[b], ob, marg, M, w.k, what=f"forced b{b}")
        log(f"  batch {b}: {st}")
        L = rows // w.B_k
        for r in range(w.H_sel):
            if first:
                assert (gsel[b, r][L >= 1] == 0).any(axis=1).all()
            for back in range(1, window):
                need = L - back >= 0
                assert (gsel[b, r][need] == (L - back)[need][:, None]).any(axis=1).all()


WINDOW_CASES = [TINY.with_(N=3000, k=6), TINY.with_(N=1000, k=4, batch=2, H_q=32, H_kv=2),
                TINY.with_(N=900, k=5, B_k=64)]


@pytest.mark.parametrize("w", WINDOW_CASES, ids=lambda w: f"N{w.N}_k{w.k}_b{w.batch}")
def test_window_selection_attention_parity(w):
    """The sliding-window selection is bit-exact, and attention over it through
    the inversion, the KV-outer kernel and the combine matches the oracle."""
    log(f"window selection N={w.N} k={w.k} batch={w.batch}")
    t = device_inputs(w, DEV)
    d = dims_of(w)
    bi = msa.msa_window_select(d, device=DEV)
    off, ent, sched = msa.msa_invert_blocks(d, bi)
    opart, lpart = msa.msa_sparse_attn_fwd(d, msa.make_opts(), t["q"], t["k"], t["v"], off, ent, sched)
    out, lse = msa.msa_combine(d, bi, opart, lpart, want_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(w.N)
    want = oracle.window_selection(rows, w.B_k, w.k, w.H_sel)
    gsel = bi.cpu().numpy()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        assert np.array_equal(gsel[b], want)
        keys = b * w.N + np.arange(w.N)
        O, L = oracle.attention(w.N, w.B_k, rows, synth.host_rows(w, "q", b * w.N + rows),
                                synth.host_rows(w, "k", keys), synth.host_rows(w, "v", keys), want)
        mx, mn = err_stats(out[b], O, label="O")
        log(f"  batch {b}: output max abs {mx:.3g} mean abs {mn:.3g}")
        assert mx <= 2e-2 and mn <= 2e-3
        lmx, _ = err_stats(lse[b], L)
        assert lmx <= 1e-3


# --------------------------------------------------------------------------- dense baseline

DENSE_CASES = [
    TINY,                                    # G = 4
    TINY.with_(N=1000),                      # ragged last block and tile
    TINY.with_(N=1),
    TINY.with_(N=300, H_q=64, H_kv=4),       # G = 16
    TINY.with_(N=700, H_q=2, H_kv=2),        # G = 1: a tile spans two key blocks
    TINY.with_(N=520, H_q=4, H_kv=2),        # G = 2
    TINY.with_(N=900, H_q=16, H_kv=2),       # G = 8
    TINY.with_(N=640, batch=2),
]


def _dense_oracle(w, rows, bat=0):
    keys = bat * w.N + np.arange(w.N)
    return oracle.dense_attention(w.N, w.B_k, rows, synth.host_rows(w, "q", bat * w.N + rows),
                                  synth.host_rows(w, "k", keys), synth.host_rows(w, "v", keys))


@pytest.mark.parametrize("w", DENSE_CASES, ids=lambda w: f"N{w.N}_G{w.G}_b{w.batch}")
def test_dense_attention_parity(w):
    log(f"dense N={w.N} H_q={w.H_q} H_kv={w.H_kv} batch={w.batch}")
    t = device_inputs(w, DEV)
    out, lse = msa.msa_dense_attn_fwd(dims_of(w), msa.make_opts(), t["q"], t["k"], t["v"],
                                      want_lse=True)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = np.arange(w.N)
    for b in range(w.batch):
        O, L = _dense_oracle(w, rows, b)
        mx, mn = err_stats(out[b], O, label="O")
        log(f"  batch {b}: output max abs {mx:.3g} mean abs {mn:.3g}")
        assert mx <= 2e-2 and mn <= 2e-3
        lmx, _ = err_stats(lse[b], L)
        assert lmx <= 1e-3


def test_dense_attention_subrange_leaves_other_rows():
    """Rows [q_begin, q_begin + q_count) (unaligned) are written; the others keep
    what the caller put there."""
    w = TINY.with_(N=1500, H_q=32, H_kv=2)
    qb, qn = 333, 777
    log(f"dense subrange N={w.N} rows [{qb}, {qb + qn})")
    t = device_inputs(w, DEV)
    o = torch.full((1, w.N, w.H_q, w.d_h), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, w.N, w.H_q), -5.0, dtype=torch.float32, device=DEV)
    msa.msa_dense_attn_fwd(dims_of(w), msa.make_opts(), t["q"], t["k"], t["v"], qb, qn, o=o, lse=lse)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[0]
    lse = lse.cpu().numpy()[0]
    outside = np.r_[0:qb, qb + qn:w.N]
    assert (o[outside] == 7.0).all() and (lse[outside] == -5.0).all()
    rows = np.arange(qb, qb + qn)
    O, L = _dense_oracle(w, rows)
    mx, mn = err_stats(o[rows], O, label="O")
    assert mx <= 2e-2 and mn <= 2e-3
    lmx, _ = err_stats(lse[rows], L)
    assert lmx <= 1e-3


def test_dense_attention_full_size_sampled():
    """128K tokens, 64 query heads over 4 K/V heads: sampled rows against the oracle."""
    w = synth.P128K_HOT
    log(f"dense full-size {w.name}")
    t = device_inputs(w, DEV)
    out, lse = msa.msa_dense_attn_fwd(dims_of(w), msa.make_opts(), t["q"], t["k"], t["v"],
                                      want_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, w.B_k, 12, seed=w.seed)
    ridx = torch.from_numpy(rows).to(DEV)
    gout = out[0][ridx].float().cpu().numpy()
    glse = lse[0][ridx].cpu().numpy()
    del t, out, lse
    torch.cuda.empty_cache()
    log(f"dense full-size {w.name}: oracle on {len(rows)} rows")
    O, L = oracle.dense_attention(w.N, w.B_k, rows, synth.host_rows(w, "q", rows),
                                  synth.host_all(w, "k"), synth.host_all(w, "v"))
    mx, mn = err_stats(gout, O, label="O")
    log(f"  output max abs {mx:.3g} mean abs {mn:.3g}")
    assert mx <= 2e-2 and mn <= 2e-3
    lmx, _ = err_stats(glse, L)
    assert lmx <= 1e-3


def test_dense_attention_1m_last_rows():
    """1M tokens: the heaviest rows (the last 512, each over about a million
    keys), computed by one range launch, sampled against the oracle."""
    w = synth.P1M
    log(f"dense 1M last rows {w.name}")
    t = device_inputs(w, DEV)
    qb = w.N - 512
    out, lse = msa.msa_dense_attn_fwd(dims_of(w), msa.make_opts(), t["q"], t["k"], t["v"], q_begin=qb,
                                      q_count=512, want_lse=True)
    torch.cuda.synchronize()
    rows = np.array([qb, qb + 1, qb + 255, w.N - 2, w.N - 1])
    ridx = torch.from_numpy(rows).to(DEV)
    gout = out[0][ridx].float().cpu().numpy()
    glse = lse[0][ridx].cpu().numpy()
    del t, out, lse
    torch.cuda.empty_cache()
    log(f"dense 1M: oracle on {len(rows)} rows")
    O, L = oracle.dense_attention(w.N, w.B_k, rows, synth.host_rows(w, "q", rows),
                                  synth.host_all(w, "k"), synth.host_all(w, "v"))
    mx, mn = err_stats(gout, O, label="O")
    log(f"  output max abs {mx:.3g} mean abs {mn:.3g}")
    assert mx <= 2e-2 and mn <= 2e-3
    lmx, _ = err_stats(glse, L)
    assert lmx <= 1e-3


# --------------------------------------------------------------------------- decode

DECODE_CASES = [
    TINY,                                          # N = 2048, k = 4, d_idx = 64, G = 4
    TINY.with_(N=1),                               # no earlier block
    TINY.with_(N=128),                             # exactly one block
    TINY.with_(N=129, k=2),                        # local block of one token
    TINY.with_(N=1000, k=16),                      # k - 1 >= L: all blocks
    TINY.with_(N=3000, k=1, batch=2),              # local block only
    TINY.with_(N=2500, k=5, H_q=64, H_kv=4, d_idx=128, batch=3),
    TINY.with_(N=4000, k=32, H_q=2, H_kv=2, plant=4),   # G = 1, planted hot blocks
    TINY.with_(N=1500, k=7, H_q=32, H_kv=4, batch=2),   # G = 8
    TINY.with_(N=2200, k=6, H_q=32, H_kv=2, H_idx=8, batch=2),   # 4 index heads per K/V head
    TINY.with_(N=1999, k=8, B_k=64, batch=2),
    TINY.with_(N=1000, k=16, B_k=32, d_idx=128),
]


def _decode_inputs(w, t):
    """The last token's Q and Q^idx of every sequence, contiguous."""
    return t["q"][:, w.N - 1].contiguous(), t["q_idx"][:, w.N - 1].contiguous()


def _check_decode(w, t, out, lse, bi, tol_max=2e-2):
    last = np.array([w.N - 1])
    for b in range(w.batch):
        ob, marg, M = oracle_index_rows(w, last, bat=b)
        gsel = bi[b][:, None, :]                                   # [H_sel, 1, k]
        st = check_selection(gsel, ob, marg, M, w.k, what=f"decode b{b}")
        O, L = compact_attention_rows(w, last, gsel, bat=b)
        mx, mn = err_stats(out[b], O[0], label="O")
        log(f"  batch {b}: {st}; output max abs {mx:.3g} mean abs {mn:.3g}")
        assert mx <= tol_max and mn <= 2e-3
        lmx, _ = err_stats(lse[b], L[0])
        assert lmx <= 1e-3


@pytest.mark.parametrize("w", DECODE_CASES, ids=lambda w: f"N{w.N}_k{w.k}_G{w.G}_Hs{w.H_sel}_d{w.d_idx}_b{w.batch}")
def test_decode_parity(w):
    log(f"decode N={w.N} k={w.k} H_q={w.H_q} H_kv={w.H_kv} d_idx={w.d_idx} batch={w.batch}")
    t = device_inputs(w, DEV)
    q1, qi1 = _decode_inputs(w, t)
    bi = torch.empty((w.batch, w.H_sel, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_decode(dims_of(w), msa.make_opts(), q1, qi1, t["k"], t["v"], t["k_idx"],
                                 block_idx_out=bi, want_lse=True)
    torch.cuda.synchronize()
    _check_decode(w, t, out.float().cpu().numpy(), lse.cpu().numpy(), bi.cpu().numpy())


def test_decode_matches_forward_last_row():
    """Decode of token N - 1 equals the whole forward's row N - 1 (same
    selection; outputs within the bf16 rounding of two different kernels)."""
    w = TINY.with_(N=1792, k=5, batch=2)
    t = device_inputs(w, DEV)
    d = dims_of(w)
    bi_f = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
    of, lf, _ = msa.msa_forward(d, msa.make_opts(), t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"],
                                block_idx_out=bi_f, want_lse=True)
    q1, qi1 = _decode_inputs(w, t)
    bi_d = torch.empty((w.batch, w.H_sel, w.k), dtype=torch.int32, device=DEV)
    od, ld, _ = msa.msa_decode(d, msa.make_opts(), q1, qi1, t["k"], t["v"], t["k_idx"],
                               block_idx_out=bi_d, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(bi_d, bi_f[:, :, w.N - 1])
    mx, _ = err_stats(od.float().cpu().numpy(), of[:, w.N - 1].float().cpu().numpy())
    assert mx <= 1e-2
    lmx, _ = err_stats(ld.cpu().numpy(), lf[:, w.N - 1].cpu().numpy())
    assert lmx <= 1e-4


@pytest.mark.parametrize("w,lens", [
    (TINY.with_(N=3000, k=5, batch=5), [3000, 1, 128, 129, 2047]),
    (TINY.with_(N=2200, k=6, H_q=32, H_kv=2, H_idx=8, batch=3), [700, 2200, 1000]),
    (TINY.with_(N=1500, k=7, B_k=64, batch=2), [1500, 901]),
], ids=lambda x: f"N{x.N}_b{x.batch}" if hasattr(x, "N") else "lens")
def test_decode_ragged_lengths(w, lens):
    """Per-sequence lengths: sequence b decodes its token lens[b] - 1 against
    its first lens[b] cache slots (the rest of the cache is ignored)."""
    log(f"decode ragged N={w.N} lens={lens}")
    t = device_inputs(w, DEV)
    lens_np = np.array(lens, np.int64)
    ridx = torch.from_numpy(lens_np - 1).to(DEV)
    bidx = torch.arange(w.batch, device=DEV)
    q1 = t["q"][bidx, ridx].contiguous()
    qi1 = t["q_idx"][bidx, ridx].contiguous()
    bi = torch.empty((w.batch, w.H_sel, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_decode(dims_of(w), msa.make_opts(), q1, qi1, t["k"], t["v"], t["k_idx"],
                                 block_idx_out=bi, want_lse=True,
                                 seq_lens=torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    out, lse, bi = out.float().cpu().numpy(), lse.cpu().numpy(), bi.cpu().numpy()
    for b, n in enumerate(lens):
        row = np.array([n - 1])            # the sequence as a cache of its own length
        flat = b * w.N + row
        keys = b * w.N + np.arange(n)
        ob, marg, M = oracle.index_topk(n, w.B_k, w.k, row, synth.host_rows(w, "q_idx", flat),
                                        synth.host_rows(w, "k_idx", keys))
        gsel = bi[b][:, None, :]
        check_selection(gsel, ob, marg, M, w.k, what=f"ragged b{b}")
        O, L = oracle.attention(n, w.B_k, row, synth.host_rows(w, "q", flat), synth.host_rows(w, "k", keys),
                                synth.host_rows(w, "v", keys), gsel)
        mx, mn = err_stats(out[b], O[0], label="O")
        log(f"  seq {b} (len {n}): output max abs {mx:.3g} mean abs {mn:.3g}")
        assert mx <= 2e-2 and mn <= 2e-3
        lmx, _ = err_stats(lse[b], L[0])
        assert lmx <= 1e-3


@pytest.mark.parametrize("w", [synth.P128K_HOT.with_(batch=4), synth.P1M],
                         ids=lambda w: f"{w.name}_b{w.batch}")
def test_decode_full_size(w):
    log(f"decode full-size {w.name} batch={w.batch}: generating inputs")
    t = device_inputs(w, DEV)
    q1, qi1 = _decode_inputs(w, t)
    bi = torch.empty((w.batch, w.H_sel, w.k), dtype=torch.int32, device=DEV)
    out, lse, _ = msa.msa_decode(dims_of(w), msa.make_opts(), q1, qi1, t["k"], t["v"], t["k_idx"],
                                 block_idx_out=bi, want_lse=True)
    torch.cuda.synchronize()
    out, lse, bi = out.float().cpu().numpy(), lse.cpu().numpy(), bi.cpu().numpy()
    del t
    torch.cuda.empty_cache()
    _check_decode(w, None, out, lse, bi)


# --------------------------------------------------------------------------- full-size workloads

BIG = [(synth.P16K, 160), (synth.P128K_HOT, 48), (synth.P128K_FP8, 40), (synth.P1M, 32)]


@pytest.mark.parametrize("w,nrows", BIG, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_full_size_sampled_parity(w, nrows):
    log(f"full-size {w.name}: generating inputs")
    t = device_inputs(w, DEV)
    d, o = dims_of(w), opts_of(w)
    bi = torch.empty((w.batch, w.H_sel, w.N, w.k), dtype=torch.int32, device=DEV)
    log(f"full-size {w.name}: msa_forward q_chunk={w.q_chunk}")
    out, _, _ = msa.msa_forward(d, o, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"],
                                block_idx_out=bi)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, w.B_k, nrows, seed=w.seed)
    gsel = np.ascontiguousarray(bi[0][:, torch.from_numpy(rows).to(DEV)].cpu().numpy())
    gout = out[0][torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    del t, out, bi
    torch.cuda.empty_cache()
    log(f"full-size {w.name}: oracle index on {len(rows)} rows")
    ob, marg, M = oracle_index_rows(w, rows)
    st = check_selection(gsel, ob, marg, M, w.k, what=w.name)
    log(f"  selection: {st}")
    log(f"full-size {w.name}: oracle attention on {len(rows)} rows")
    O, _ = compact_attention_rows(w, rows, gsel)
    mx, mn = err_stats(gout, O, label="O")
    log(f"  output max abs {mx:.3g} mean abs {mn:.3g}")
    assert mx <= (6e-2 if w.dtype == "fp8" else 2e-2) and mn <= 2e-3
