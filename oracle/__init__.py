"""CPU oracle for the slot-indexed Gated DeltaNet state path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package. It shares no
code with the HIP library; the C source is `gdn_oracle.c` next to this file.

All arrays are numpy; bf16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = C.CDLL(_LIB_PATH)
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.orc_f32_to_bf16.argtypes = [p, p, i64]
        L.orc_bf16_to_f32.argtypes = [p, p, i64]
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_gdn_layer.argtypes = [p, i64, i64, i64, i64,
                                    i32, i32, i32, i32, i32, i32,
                                    i32, p, p, p, p, p, p, p, p, C.c_double, C.c_double, p, p]
        L.orc_gdn_layer.restype = C.c_int
        L.orc_restore.argtypes = [p, i32, i64, i64, i64, i64, i64, i64, p, p, p, i32, p]
        L.orc_restore.restype = C.c_int
        L.orc_gather.argtypes = [p, i64, i64, i64, i64, i64, i64, p, i32, p, p]
        L.orc_scatter.argtypes = [p, i64, i64, i64, i64, i64, i64, p, i32, p, p]
        L.orc_conv_silu.argtypes = [i32, i32, i32, p, p, p, p, p]
        L.orc_delta_rule.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def f32_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().orc_bf16_to_f32(_ptr(b), _ptr(out), b.size)
    return out


def conv_silu(window, x, conv_w, conv_b=None):
    """Conv + SiLU over a sequence. window: bf16 [W-1, C] (updated copy is
    returned), x: bf16 [L, C]. Returns (y float64 [L, C], new window)."""
    win = _c(window, np.uint16).copy()
    x = _c(x, np.uint16)
    w = _c(conv_w, np.uint16)
    b = None if conv_b is None else _c(conv_b, np.uint16)
    L, C_ = x.shape
    W = w.shape[1]
    y = np.empty((L, C_), dtype=np.float64)
    lib().orc_conv_silu(L, C_, W, _ptr(win), _ptr(x), _ptr(w), _ptr(b), _ptr(y))
    return y, win


def delta_rule(S, q_hat, k_hat, v, alpha, beta):
    """Gated delta rule for one head over L tokens. S: fp32 [dk, dv] (a new
    array is returned), q_hat, k_hat: [L, dk], v: [L, dv], alpha, beta: [L].
    Returns (S_final fp32, out64 [L, dv], out16 [L, dv])."""
    S = _c(S, np.float32).copy()
    q = _c(q_hat, np.float64)
    k = _c(k_hat, np.float64)
    v = _c(v, np.float64)
    a = _c(alpha, np.float32)
    b = _c(beta, np.float32)
    L, dk = q.shape
    dv = v.shape[1]
    o64 = np.empty((L, dv), dtype=np.float64)
    o16 = np.empty((L, dv), dtype=np.uint16)
    lib().orc_delta_rule(L, dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                         _ptr(o64), _ptr(o16))
    return S, o64, o16


def region_bytes(C_: int, W: int, Hv: int, dk: int, dv: int):
    """(state bytes, conv-window bytes) of one page: Hv*dk*dv fp32 and
    (W-1)*C bf16."""
    return Hv * dk * dv * 4, (W - 1) * C_ * 2


def gdn_layer(pool: np.ndarray, geom, cu_seqlens, state_indices, has_initial_state,
              x, conv_w, conv_b, alpha, beta, scale=1.0, eps=1e-6):
    """Run one GDN layer over the batch; `pool` ([num_slots, page_stride] uint8)
    is updated in place. Returns (out64 [T,Hv,dv] float64, out16 [T,Hv,dv] uint16)."""
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    cu = _c(cu_seqlens, np.int32)
    idx = _c(state_indices, np.int32)
    hs = _c(has_initial_state, np.uint8)
    x = _c(x, np.uint16)
    w = _c(conv_w, np.uint16)
    b = None if conv_b is None else _c(conv_b, np.uint16)
    a = _c(alpha, np.float32)
    be = _c(beta, np.float32)
    T = int(cu[-1])
    out64 = np.zeros((T, geom.Hv, geom.dv), dtype=np.float64)
    out16 = np.zeros((T, geom.Hv, geom.dv), dtype=np.uint16)
    rc = lib().orc_gdn_layer(_ptr(pool), pool.shape[0], geom.page_stride, geom.ssm_off,
                             geom.conv_off, geom.C, geom.W, geom.Hk, geom.Hv, geom.dk,
                             geom.dv, len(idx), _ptr(cu), _ptr(idx), _ptr(hs), _ptr(x),
                             _ptr(w), _ptr(b), _ptr(a), _ptr(be), float(scale), float(eps),
                             _ptr(out64), _ptr(out16))
    if rc != 0:
        raise ValueError("oracle rejected the layer arguments")
    return out64, out16


def decode(pool, geom, state_indices, has_initial_state, x, conv_w, conv_b, alpha, beta,
           scale=1.0, eps=1e-6):
    """One decode step: every row is a sequence of one token."""
    rows = len(state_indices)
    cu = np.arange(rows + 1, dtype=np.int32)
    return gdn_layer(pool, geom, cu, state_indices, has_initial_state, x, conv_w, conv_b,
                     alpha, beta, scale, eps)


def restore(layer_pools: Sequence[Optional[np.ndarray]], geom, ops, hs) -> int:
    """Apply restore ops [n,3] = (dst, src, requested) to the host pools
    (None = attention-only layer); `hs` (uint8 [n]) is updated in place.
    Returns 1 on the soft failure (a hit copied no layer), else 0."""
    ops = _c(ops, np.int32).reshape(-1, 3)
    dst = _c(ops[:, 0], np.int32)
    src = _c(ops[:, 1], np.int32)
    req = _c(ops[:, 2] != 0, np.uint8)
    assert hs.dtype == np.uint8 and hs.flags["C_CONTIGUOUS"]
    ptrs = (C.c_void_p * len(layer_pools))(
        *[None if p is None else p.ctypes.data for p in layer_pools])
    num_slots = geom.num_slots
    ssm_b, conv_b = region_bytes(geom.C, geom.W, geom.Hv, geom.dk, geom.dv)
    rc = lib().orc_restore(ptrs, len(layer_pools), num_slots, geom.page_stride, geom.ssm_off,
                           ssm_b, geom.conv_off, conv_b, _ptr(dst), _ptr(src), _ptr(req),
                           len(dst), _ptr(hs))
    if rc < 0:
        raise ValueError("oracle restore: slot out of range")
    return rc


def gather(pool: np.ndarray, geom, idx):
    idx = _c(idx, np.int32)
    ssm_b, conv_b = region_bytes(geom.C, geom.W, geom.Hv, geom.dk, geom.dv)
    sd = np.empty((len(idx), ssm_b), dtype=np.uint8)
    cd = np.empty((len(idx), conv_b), dtype=np.uint8)
    lib().orc_gather(_ptr(pool), pool.shape[0], geom.page_stride, geom.ssm_off, ssm_b,
                     geom.conv_off, conv_b, _ptr(idx), len(idx), _ptr(sd), _ptr(cd))
    return sd, cd


def scatter(pool: np.ndarray, geom, idx, ssm_dense, conv_dense) -> None:
    idx = _c(idx, np.int32)
    ssm_b, conv_b = region_bytes(geom.C, geom.W, geom.Hv, geom.dk, geom.dv)
    sd = _c(ssm_dense, np.uint8).reshape(len(idx), ssm_b)
    cd = _c(conv_dense, np.uint8).reshape(len(idx), conv_b)
    lib().orc_scatter(_ptr(pool), pool.shape[0], geom.page_stride, geom.ssm_off, ssm_b,
                      geom.conv_off, conv_b, _ptr(idx), len(idx), _ptr(sd), _ptr(cd))
