"""Seeded synthetic inputs for the MSA forward pass.

This module holds no arithmetic of the method.  It is the one input generator
that both the oracle side (tests, CPU baseline) and the HIP side read, so that
both see bit-identical inputs.

Generator (counter based, so any element can be regenerated on its own):

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state increment 0x9E3779B97F4A7C15 and the
  finaliser with multipliers 0xBF58476D1CE4E5B9 / 0x94D049BB133111EB and
  shifts 30 / 27 / 31.  A tensor's stream key is the first output of a
  SplitMix64 generator seeded with ``seed << 16 | tensor_id``; element ``e`` of
  that tensor is output number ``e`` of a SplitMix64 generator seeded with the
  key (i.e. finaliser(key + (e + 1) * increment)).
* N(0, 1) values: the top 16 bits of the element's hash index a 65,536-entry
  quantile table, entry u = bf16(fp32(Phi^-1((u + 0.5) / 65536))) with
  round-to-nearest-even at each narrowing.  Integer hashing plus a table
  lookup means the GPU fill kernel and numpy give the same bits.
* fp8 inputs: per-tensor scale s = amax / 448 (amax = the table's largest
  magnitude), code = OCP e4m3fn round-to-nearest-even of fp32(x / s).
* planted "hot" blocks: 64 distinct blocks chosen by sorting block ids by
  their hash; a unit direction u from 128 table draws normalised in fp64 and
  rounded to fp32; 2.0 * u is added in fp32 to the index-key rows of hot
  blocks and to every index-query row before rounding to bf16.

Tensor ids: Q=0, K=1, V=2, Q^idx=3, K^idx=4, hot set=5, direction=6.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB

TID_Q, TID_K, TID_V, TID_QIDX, TID_KIDX, TID_HOT, TID_DIR, TID_DO = range(8)


def _fin_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * MUL1) & _MASK64
    z = ((z ^ (z >> 27)) * MUL2) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    return _fin_int(((seed << 16) | tensor_id) + GAMMA)


def hash_at(key: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 output number ``idx`` of the stream seeded with ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
        z = z ^ (z >> np.uint64(31))
    return z


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_TABLE: Optional[np.ndarray] = None


def normal_table() -> np.ndarray:
    """uint16[65536]: bf16 bits of the N(0,1) quantile at (u + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLE = f32_to_bf16_bits(ndtri(p).astype(np.float32))
    return _TABLE


def _e4m3_values() -> np.ndarray:
    """fp64 value of each e4m3fn code (NaN for the two NaN codes)."""
    c = np.arange(256)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e - 10.0))
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def fp8_scale() -> float:
    """Per-tensor fp32 scale amax / 448 of the generated distribution."""
    amax = np.float32(np.abs(bf16_bits_to_f32(normal_table())).max())
    return float(np.float32(amax / np.float32(448.0)))


_TABLE8: Optional[np.ndarray] = None


def fp8_table() -> np.ndarray:
    """uint8[65536]: e4m3fn code (RNE, saturating) of normal_table()/scale."""
    global _TABLE8
    if _TABLE8 is None:
        x = (bf16_bits_to_f32(normal_table()) / np.float32(fp8_scale())).astype(np.float64)
        vals = _e4m3_values()
        codes = np.arange(256)
        ok = ~np.isnan(vals)
        vals_ok, codes_ok = vals[ok], codes[ok]
        # nearest representable; ties to the even mantissa (code bit 0 clear)
        d = np.abs(x[:, None] - vals_ok[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        even = (codes_ok[None, :] & 1) == 0
        pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1),
                        np.argmax(cand, axis=1))
        # -0 and +0 are both nearest to 0: keep the sign of x
        out = codes_ok[pick].astype(np.uint8)
        out = np.where((vals_ok[pick] == 0) & (x < 0), np.uint8(0x80), out)
        _TABLE8 = out.astype(np.uint8)
    return _TABLE8


# --------------------------------------------------------------------------
# workloads

@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    N: int
    H_q: int
    H_kv: int
    d_h: int
    d_idx: int
    B_k: int
    k: int
    seed: int
    dtype: str = "bf16"          # "bf16" or "fp8" for Q, K, V
    plant: int = 0               # number of planted hot blocks (0 = none)
    plant_gain: float = 2.0
    q_chunk: int = 0             # 0 = the library default (msa_forward: passes of
                                 # 16,384 rows; msa_backward: one pass)
    H_idx: int = 0               # index (proxy) heads; 0 = H_kv

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def H_sel(self) -> int:
        """Index heads = selection groups."""
        return self.H_idx or self.H_kv

    @property
    def G_sel(self) -> int:
        """Query heads per selection group."""
        return self.H_q // self.H_sel

    @property
    def B(self) -> int:
        return -(-self.N // self.B_k)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny case, a 16K prefill, a 128K prefill with skewed
# block popularity, the 128K prefill with fp8 Q/K/V, and a chunked 1M prefill.
TINY = Workload("tiny_n2048_hq8_hkv2_didx64_k4", 1, 2048, 8, 2, 128, 64, 128, 4, seed=1)
P16K = Workload("prefill_n16384_hq64_hkv4_k16", 1, 16384, 64, 4, 128, 128, 128, 16, seed=2)
P128K_HOT = Workload("prefill_n131072_hq64_hkv4_k16_hot64", 1, 131072, 64, 4, 128, 128, 128, 16,
                     seed=3, plant=64)
P128K_FP8 = Workload("prefill_n131072_hq64_hkv4_k16_fp8", 1, 131072, 64, 4, 128, 128, 128, 16,
                     seed=4, dtype="fp8")
P1M = Workload("prefill_n1048576_hq64_hkv4_k16_chunk32768", 1, 1 << 20, 64, 4, 128, 128, 128, 16,
               seed=5, q_chunk=32768)
WORKLOADS = {w.name: w for w in (TINY, P16K, P128K_HOT, P128K_FP8, P1M)}


# --------------------------------------------------------------------------
# host-side generation (numpy)

def _codes(seed, tid, idx, fp8):
    h = hash_at(stream_key(seed, tid), idx)
    u = (h >> np.uint64(48)).astype(np.int64)
    return fp8_table()[u] if fp8 else normal_table()[u]


def hot_blocks(w: Workload) -> np.ndarray:
    """Sorted ids of the planted hot blocks (empty when not planted)."""
    if not w.plant:
        return np.zeros(0, np.int64)
    ids = np.arange(w.B, dtype=np.uint64)
    h = hash_at(stream_key(w.seed, TID_HOT), ids)
    order = np.lexsort((ids, h))
    return np.sort(order[: min(w.plant, w.B)].astype(np.int64))


def plant_vector(w: Workload) -> np.ndarray:
    """fp32 [d_idx]: gain * unit direction (zeros when not planted)."""
    if not w.plant:
        return np.zeros(w.d_idx, np.float32)
    v = bf16_bits_to_f32(_codes(w.seed, TID_DIR, np.arange(w.d_idx), False)).astype(np.float64)
    u = (v / np.sqrt((v * v).sum())).astype(np.float32)
    return (np.float32(w.plant_gain) * u).astype(np.float32)


def _planted(codes_bf16, cols, rows_hot, vec):
    """bf16(fp32(x) + vec[col]) where rows_hot, else x."""
    x = bf16_bits_to_f32(codes_bf16)
    y = f32_to_bf16_bits((x + vec[cols]).astype(np.float32))
    return np.where(rows_hot, y, codes_bf16)


def host_rows(w: Workload, which: str, rows) -> np.ndarray:
    """Regenerate whole token rows of one tensor on the host.

    which in {"q", "k", "v", "q_idx", "k_idx", "d_o"} ("d_o": a bf16 output
    gradient for the backward pass); rows are token positions of
    batch element 0.. (flattened as batch * N + i).  Returns raw codes with
    shape [len(rows), heads, dim] (k_idx: [len(rows), dim])."""
    rows = np.asarray(rows, dtype=np.int64)
    spec = {
        "q": (TID_Q, w.H_q, w.d_h, w.dtype == "fp8"),
        "k": (TID_K, w.H_kv, w.d_h, w.dtype == "fp8"),
        "v": (TID_V, w.H_kv, w.d_h, w.dtype == "fp8"),
        "q_idx": (TID_QIDX, w.H_sel, w.d_idx, False),
        "k_idx": (TID_KIDX, 1, w.d_idx, False),
        "d_o": (TID_DO, w.H_q, w.d_h, False),
    }[which]
    tid, heads, dim, fp8 = spec
    per_row = heads * dim
    idx = rows[:, None] * per_row + np.arange(per_row, dtype=np.int64)[None, :]
    codes = _codes(w.seed, tid, idx.reshape(-1), fp8).reshape(len(rows), heads, dim)
    if w.plant and which in ("q_idx", "k_idx"):
        vec = plant_vector(w)
        cols = np.broadcast_to(np.arange(dim), codes.shape)
        if which == "q_idx":
            hot = np.ones(codes.shape, bool)
        else:
            hb = np.zeros(w.B, bool)
            hb[hot_blocks(w)] = True
            tok = rows % w.N
            hot = np.broadcast_to(hb[tok // w.B_k][:, None, None], codes.shape)
        codes = _planted(codes, cols, hot, vec)
    if which == "k_idx":
        codes = codes[:, 0, :]
    return codes


def host_all(w: Workload, which: str) -> np.ndarray:
    """A whole tensor on the host (small workloads only)."""
    return host_rows(w, which, np.arange(w.batch * w.N))


# --------------------------------------------------------------------------
# device-side generation (HIP fill kernel, same bits)

_SRC = os.path.join(_HERE, "synth_fill.hip")
_LIB = os.path.join(_HERE, "libmsa_synth.so")
_lib = None


def build() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           _SRC, "-o", _LIB + ".tmp"]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _dlib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError("libmsa_synth.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.synth_fill.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int64,
                                 P, P, ctypes.c_int, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, P]
        L.synth_fill.restype = ctypes.c_int
        _lib = L
    return _lib


def device_tensor(w: Workload, which: str, device="cuda"):
    """Generate a whole input tensor directly in device memory (torch tensor of
    raw codes: uint16 for bf16 (viewable as torch.bfloat16), uint8 for fp8)."""
    import torch
    tid, heads, dim, fp8 = {
        "q": (TID_Q, w.H_q, w.d_h, w.dtype == "fp8"),
        "k": (TID_K, w.H_kv, w.d_h, w.dtype == "fp8"),
        "v": (TID_V, w.H_kv, w.d_h, w.dtype == "fp8"),
        "q_idx": (TID_QIDX, w.H_sel, w.d_idx, False),
        "k_idx": (TID_KIDX, 1, w.d_idx, False),
        "d_o": (TID_DO, w.H_q, w.d_h, False),
    }[which]
    shape = (w.batch, w.N, heads, dim) if which != "k_idx" else (w.batch, w.N, dim)
    n = int(np.prod(shape))
    table = torch.from_numpy((fp8_table() if fp8 else normal_table()).view(
        np.uint8 if fp8 else np.int16).copy()).to(device)
    out = torch.empty(shape, dtype=torch.uint8 if fp8 else torch.int16, device=device)
    vec_t = mask_t = None
    mode = 0
    if w.plant and which in ("q_idx", "k_idx"):
        vec_t = torch.from_numpy(plant_vector(w)).to(device)
        if which == "q_idx":
            mode = 1
        else:
            mode = 2
            hb = np.zeros(w.B, np.uint8)
            hb[hot_blocks(w)] = 1
            mask_t = torch.from_numpy(hb).to(device)
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = _dlib().synth_fill(
        ctypes.c_void_p(out.data_ptr()), 1 if fp8 else 2, n,
        stream_key(w.seed, tid), 0, ctypes.c_void_p(table.data_ptr()),
        ctypes.c_void_p(vec_t.data_ptr() if vec_t is not None else 0), dim,
        ctypes.c_void_p(mask_t.data_ptr() if mask_t is not None else 0),
        w.B_k * dim, w.N * dim, mode, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed with HIP error {rc}")
    # keep table / vector alive until the fill has run
    torch.cuda.current_stream(out.device).synchronize()
    if not fp8:
        out = out.view(torch.bfloat16)
    return out
