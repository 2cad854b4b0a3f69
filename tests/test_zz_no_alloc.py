"""msa_decode_static (the decode step that allocates nothing, working in the
library's static device scratch) against msa_decode with a caller-allocated
workspace: two calls in a row, the second with a smaller step, each equal to
msa_decode bit for bit (same kernels, same inputs), and with ragged lengths.
The first call on the device also looks the scratch address up."""
import numpy as np
import pytest
import torch

import block_sparse_attention_idx_amd as msa
import synth
from gpu_util import device_inputs, dims_of, log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pair(w, seq_lens=None):
    t = device_inputs(w, DEV)
    if seq_lens is None:
        q1 = t["q"][:, w.N - 1].contiguous()
        qi1 = t["q_idx"][:, w.N - 1].contiguous()
        lens = None
    else:
        ridx = torch.tensor([n - 1 for n in seq_lens], device=DEV)
        bidx = torch.arange(w.batch, device=DEV)
        q1 = t["q"][bidx, ridx].contiguous()
        qi1 = t["q_idx"][bidx, ridx].contiguous()
        lens = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    d, o = dims_of(w), msa.make_opts()
    outs = []
    for fn in (msa.msa_decode, msa.msa_decode_static):
        bi = torch.full((w.batch, w.H_sel, w.k), -9, dtype=torch.int32, device=DEV)
        out, lse, _ = fn(d, o, q1, qi1, t["k"], t["v"], t["k_idx"], block_idx_out=bi, want_lse=True,
                         seq_lens=lens)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy().view(np.int32), bi.cpu().numpy()))
    (o_ref, l_ref, b_ref), (o_st, l_st, b_st) = outs
    assert np.array_equal(b_st, b_ref)
    assert np.array_equal(o_st, o_ref)
    assert np.array_equal(l_st, l_ref)
    assert np.isfinite(synth.bf16_bits_to_f32(o_st.view(np.uint16))).all()


def test_decode_static_two_calls_then_smaller():
    big = synth.P128K_HOT.with_(N=40000, batch=4)
    small = synth.TINY.with_(N=3000, k=5, batch=2)
    d = dims_of(big)
    ws = msa.msa_decode_workspace_size(d, msa.make_opts())
    assert ws <= msa.STATIC_SCRATCH_BYTES
    log(f"static decode: {big.name} N={big.N} batch={big.batch} ({ws} B of scratch)")
    _pair(big)
    log(f"static decode: smaller step N={small.N} batch={small.batch}")
    _pair(small)


def test_decode_static_ragged_after_other_calls():
    w = synth.TINY.with_(N=3000, k=5, batch=5)
    log("static decode: ragged lengths")
    _pair(w, seq_lens=[3000, 1, 128, 129, 2047])


def test_decode_static_rejects_too_large():
    w = synth.P1M.with_(batch=600)
    d = dims_of(w)
    assert msa.msa_decode_workspace_size(d, msa.make_opts()) > msa.STATIC_SCRATCH_BYTES
    z = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(msa.MSAError) as ei:
        msa.msa_decode_static(d, msa.make_opts(), z, z, z, z, z, o=z)
    assert ei.value.status == 7
