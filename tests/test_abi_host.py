"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects bad arguments before any
HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import block_sparse_attention_idx_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(msa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return msa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", msa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (msa_[a-z_0-9]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)
    assert set(msa.EXPORTS) <= set(names)


def test_identity(L):
    assert L.msa_abi_version() == 4
    assert L.msa_status_string(0) == b"ok"
    assert L.msa_status_string(5) == b"workspace too small"


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x10008)


def dims(**kw):
    base = dict(batch=1, N=2048, H_q=8, H_kv=2, d_h=128, d_idx=64, B_k=128, k=4)
    G = kw.pop("G", None)
    base.update(kw)
    d = msa.make_dims(**base)
    if G is not None:
        d.G = G
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=9), 2), (dict(G=3), 2), (dict(N=0), 2), (dict(k=0), 2), (dict(batch=0), 2),
    (dict(d_h=64), 3), (dict(B_k=96), 3), (dict(B_k=256), 3), (dict(d_idx=96), 3), (dict(k=33), 3),
    (dict(H_q=6, H_kv=2), 3), (dict(N=16384 * 128 + 1), 3),
])
def test_index_topk_rejects_bad_dims(L, kw, status):
    d = dims(**kw)
    assert L.msa_index_topk(ctypes.byref(d), FAKE, FAKE, 0, 16, FAKE, None) == status


@pytest.mark.parametrize("qb,qn,status", [(-128, 16, 2), (0, 0, 2), (64, 16, 2), (0, 2049, 2),
                                          (1920, 200, 2)])
def test_ranges(L, qb, qn, status):
    d = dims()
    assert L.msa_index_topk(ctypes.byref(d), FAKE, FAKE, qb, qn, FAKE, None) == status
    assert L.msa_combine(ctypes.byref(d), FAKE, FAKE, FAKE, qb, qn, FAKE, None, None) == status


def test_null_and_alignment(L):
    d = dims()
    assert L.msa_index_topk(ctypes.byref(d), None, FAKE, 0, 16, FAKE, None) == 1
    assert L.msa_index_topk(ctypes.byref(d), FAKE, ODD, 0, 16, FAKE, None) == 4
    assert L.msa_index_topk(None, FAKE, FAKE, 0, 16, FAKE, None) == 1
    assert L.msa_combine(ctypes.byref(d), FAKE, FAKE, FAKE, 0, 16, FAKE, ODD, None) == 4
    o = msa.make_opts()
    assert L.msa_sparse_attn_fwd(ctypes.byref(d), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None, 0, 16, FAKE, FAKE, None) == 1


def test_workspace_and_opts(L):
    d = dims()
    n = ctypes.c_size_t(0)
    assert L.msa_invert_workspace_size(ctypes.byref(d), 0, 2048, ctypes.byref(n)) == 0
    assert n.value > 0
    assert L.msa_invert_blocks(ctypes.byref(d), FAKE, 0, 2048, FAKE, FAKE, FAKE, n.value - 4,
                               None) == 5
    o = msa.make_opts()
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == 0
    ws = n.value
    # partial buffers dominate: k * G * (2 d_h + 4) bytes per (query, group)
    assert ws >= 2048 * 2 * 4 * 4 * (2 * 128 + 4)
    assert L.msa_forward(ctypes.byref(d), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         None, None, FAKE, ws - 256, None) == 5
    bad = msa.make_opts(q_chunk=100)
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(n)) == 2
    bad = msa.make_opts(dtype="fp8", q_scale=0.0)
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(n)) == 2
    d64 = dims(B_k=64)
    assert L.msa_workspace_size(ctypes.byref(d64), ctypes.byref(o), ctypes.byref(n)) == 0
    f8 = msa.make_opts(dtype="fp8")
    assert L.msa_workspace_size(ctypes.byref(d64), ctypes.byref(f8), ctypes.byref(n)) == 3
    bad = msa.make_opts()
    bad.qkv_dtype = 7
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(n)) == 3
    # chunking shrinks the workspace
    c = msa.make_opts(q_chunk=512)
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value < ws
    # q_chunk 0 takes msa_forward's default rows per pass (all rows when N is
    # at most that): the same workspace as asking for them explicitly
    big = dims(N=4 * msa.DEFAULT_Q_CHUNK)
    sizes = {}
    for qc in (0, msa.DEFAULT_Q_CHUNK, 4 * msa.DEFAULT_Q_CHUNK):
        assert L.msa_workspace_size(ctypes.byref(big), ctypes.byref(msa.make_opts(q_chunk=qc)),
                                    ctypes.byref(n)) == 0
        sizes[qc] = n.value
    assert sizes[0] == sizes[msa.DEFAULT_Q_CHUNK] < sizes[4 * msa.DEFAULT_Q_CHUNK]
    assert L.msa_workspace_size(ctypes.byref(d), ctypes.byref(msa.make_opts(q_chunk=d.N)),
                                ctypes.byref(n)) == 0
    assert n.value == ws  # N = 2048 is below the default: one pass either way


def test_dense_attn_validation(L):
    o = msa.make_opts()
    call = lambda d, o, qb, qn, q=FAKE, out=FAKE, lse=None: L.msa_dense_attn_fwd(
        ctypes.byref(d), ctypes.byref(o), q, FAKE, FAKE, qb, qn, out, lse, None)
    # d_idx, B_k and k are not used by the dense path
    assert call(dims(d_idx=96, B_k=64, k=0, N=0), o, 0, 16) == 2
    assert call(dims(H_q=9), o, 0, 16) == 2
    assert call(dims(d_h=64), o, 0, 16) == 3
    assert call(dims(H_q=6, H_kv=2), o, 0, 16) == 3
    assert call(dims(), o, -1, 16) == 2
    assert call(dims(), o, 0, 0) == 2
    assert call(dims(), o, 2000, 49) == 2
    assert call(dims(), msa.make_opts(dtype="fp8"), 0, 16) == 3
    assert call(dims(), o, 0, 16, q=None) == 1
    assert call(dims(), o, 0, 16, out=ODD) == 4
    assert call(dims(), o, 0, 16, lse=ODD) == 4
    assert L.msa_dense_attn_fwd(None, ctypes.byref(o), FAKE, FAKE, FAKE, 0, 16, FAKE, None, None) == 1


def test_decode_validation(L):
    o = msa.make_opts()
    n = ctypes.c_size_t(0)
    d = dims()
    assert L.msa_decode_workspace_size(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == 0
    ws = n.value
    # block scores, selection, partial outputs and their lse
    B = (2048 + 127) // 128
    assert ws >= 2 * B * 4 + 2 * 4 * 4 + 2 * 4 * 4 * 128 * 2 + 2 * 4 * 4 * 4
    call = lambda d, o, ws_bytes=ws, q=FAKE, out=FAKE, wsp=FAKE, lens=None: L.msa_decode(
        ctypes.byref(d), ctypes.byref(o), q, FAKE, FAKE, FAKE, FAKE, lens, out, None, None, wsp, ws_bytes,
        None)
    assert call(d, o, ws - 1) == 5
    assert call(d, msa.make_opts(dtype="fp8"), ws) == 3
    assert call(dims(H_q=66, H_kv=33), o) == 3
    assert call(dims(k=0), o) == 2
    assert call(d, o, q=None) == 1
    assert call(d, o, out=ODD) == 4
    assert call(d, o, wsp=ctypes.c_void_p(0x10010)) == 4     # workspace needs 256-byte alignment
    assert call(d, o, lens=ctypes.c_void_p(0x10002)) == 4    # lengths are int32
    assert L.msa_decode_workspace_size(ctypes.byref(d), ctypes.byref(o), None) == 1


def test_decode_static_validation(L):
    """msa_decode_static: the decode checks, then the static scratch limit, all
    before the device is touched."""
    o = msa.make_opts()
    call = lambda d, o=o, q=FAKE, out=FAKE, lse=None: L.msa_decode_static(
        ctypes.byref(d), ctypes.byref(o), q, FAKE, FAKE, FAKE, FAKE, None, out, lse, None, None)
    big = dims(N=1 << 20, H_q=64, H_kv=4, d_idx=128, k=16, batch=600)
    n = ctypes.c_size_t(0)
    assert L.msa_decode_workspace_size(ctypes.byref(big), ctypes.byref(o), ctypes.byref(n)) == 0
    assert n.value > msa.STATIC_SCRATCH_BYTES
    assert call(big) == 7
    assert L.msa_status_string(7).startswith(b"problem needs more than the static scratch")
    assert call(dims(), msa.make_opts(dtype="fp8")) == 3
    assert call(dims(k=0)) == 2
    assert call(dims(), q=None) == 1
    assert call(dims(), out=ODD) == 4
    assert call(dims(), lse=ODD) == 4
    assert L.msa_decode_static(None, ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                               None, None) == 1


@pytest.mark.parametrize("H_idx,status", [(-1, 2), (3, 2), (6, 2), (16, 0), (8, 0), (4, 0), (0, 0)])
def test_index_head_validation(L, H_idx, status):
    """H_idx: a multiple of H_kv = 2 dividing H_q = 16 (G_sel a power of two
    <= 16); 0 means H_kv."""
    d = dims(H_q=16, H_kv=2, H_idx=H_idx)
    n = ctypes.c_size_t(0)
    assert L.msa_invert_workspace_size(ctypes.byref(d), 0, 2048, ctypes.byref(n)) == status


def test_selection_variant_validation(L):
    d = dims(k=4)
    f = lambda first, window, d=d: L.msa_index_topk_forced(ctypes.byref(d), FAKE, FAKE, 0, 16, first,
                                                          window, FAKE, None)
    assert f(2, 1) == 2                      # force_first is 0 or 1
    assert f(0, 0) == 2                      # the window includes the local block
    assert f(1, 4) == 2                      # 1 + 3 forced > k - 1 = 3
    assert f(0, 5) == 2
    assert L.msa_index_topk_forced(ctypes.byref(d), FAKE, ODD, 0, 16, 1, 3, FAKE, None) == 4
    assert L.msa_index_topk_forced(ctypes.byref(d), None, FAKE, 0, 16, 1, 3, FAKE, None) == 1
    assert L.msa_window_select(ctypes.byref(d), 64, 16, FAKE, None) == 2   # q_begin % B_k
    assert L.msa_window_select(ctypes.byref(d), 0, 16, None, None) == 1
    assert L.msa_window_select(ctypes.byref(d), 0, 16, ODD, None) == 4


def test_binding_raises_when_library_missing(monkeypatch):
    monkeypatch.setattr(msa, "_lib", None)
    monkeypatch.setattr(msa, "LIB_PATH", "/nonexistent/libmsa.so")
    with pytest.raises(msa.MSAError):
        msa.lib()


def test_backward_validation(L):
    """msa_backward: bf16 and B_k = 128 only; required pointers; the index
    outputs come together; 16-byte alignment; a 256-byte aligned workspace of
    the queried size."""
    o = msa.make_opts()
    n = ctypes.c_size_t(0)
    d = dims()
    assert L.msa_backward_workspace_size(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == 0
    size = n.value
    assert size > 0
    assert L.msa_backward_workspace_size(ctypes.byref(dims(B_k=64)), ctypes.byref(o), ctypes.byref(n)) == 3
    fp8 = msa.make_opts("fp8")
    assert L.msa_backward_workspace_size(ctypes.byref(d), ctypes.byref(fp8), ctypes.byref(n)) == 3
    assert L.msa_backward_workspace_size(ctypes.byref(d), ctypes.byref(o), None) == 1

    def call(d=d, o=o, w=1.0, dqi=FAKE, dki=FAKE, kl=None, q=FAKE, wsp=ctypes.c_void_p(0x100000),
             nbytes=size, lse=FAKE):
        return L.msa_backward(ctypes.byref(d), ctypes.byref(o), w, q, FAKE, FAKE, FAKE, FAKE, FAKE, lse, FAKE,
                              FAKE, FAKE, FAKE, FAKE, dqi, dki, kl, wsp, nbytes, None)

    assert call(w=float("nan")) == 2
    assert call(q=None) == 1
    assert call(lse=None) == 1
    assert call(dqi=None) == 1             # dk_idx without dq_idx
    assert call(dqi=None, dki=None, kl=FAKE) == 1
    assert call(q=ODD) == 4
    assert call(kl=ODD) == 4
    assert call(wsp=ctypes.c_void_p(0x100010)) == 4
    assert call(nbytes=size - 1) == 5
    assert call(d=dims(B_k=32)) == 3


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(args, env):
    """The measurement is a one-GPU build: asked for several GPUs (flag or a
    launcher's WORLD_SIZE), bench.py exits with status 2 and says so before
    touching torch or the GPU."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    e = dict(os.environ)
    e.pop("WORLD_SIZE", None)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                       env=e, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
