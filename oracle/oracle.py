"""ctypes wrapper over oracle/liboracle.so (plain C, fp64).

TEST INFRASTRUCTURE ONLY.  The wrapper only marshals arguments: every step of
the arithmetic lives in lora_oracle.c, in the pages' order.  Input conversion
to fp64 (to_f64) is exact for fp32, fp16 and bf16.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

BASE_ONLY = -1
MODE_NONE, MODE_FUSED, MODE_SEPARATE = 0, 1, 2
POLICY_AUTO, POLICY_FUSED, POLICY_SEPARATE = 0, 1, 2

_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def load():
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_route.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _i32p,
                                 ctypes.c_int, ctypes.c_int,
                                 _i32p, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_apply.restype = ctypes.c_long
    lib.oracle_apply.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 _f64p, _f64p, _i32p, _i32p, _i32p, _f64p,
                                 _f64p, _i64p, _f64p, _i64p,
                                 _f64p, _i32p, ctypes.c_int]
    _lib = lib
    return lib


def to_f64(a):
    """Exact conversion of a torch tensor (any device) or array to fp64 numpy."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu").to(torch.float64).numpy())
    except ImportError:  # pragma: no cover - torch is part of the image
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def route(idx, n_slots, active, policy=POLICY_AUTO, theta=16):
    """Counting sort of one call's tokens by adapter key (see oracle_route)."""
    lib = load()
    idx = _i32(idx).reshape(-1)
    active = _i32(active).reshape(-1)
    S = int(n_slots)
    assert active.shape[0] == S
    T = idx.shape[0]
    counts = np.zeros(S + 2, np.int32)
    offsets = np.zeros(S + 3, np.int32)
    perm = np.zeros(max(T, 1), np.int32)
    segs = np.zeros((S + 2) * 4, np.int32)
    n_seg = np.zeros(1, np.int32)
    rc = lib.oracle_route(idx, T, S, active, int(policy), int(theta),
                          counts, offsets, perm, segs, n_seg)
    if rc != 0:
        raise MemoryError("oracle_route failed")
    n = int(n_seg[0])
    return {"counts": counts, "offsets": offsets, "perm": perm[:T],
            "segs": segs.reshape(S + 2, 4)[:n].copy(), "n_seg": n}


def apply(x, W, idx, n_slots, adapters, n_threads=0):
    """Per-token y = x W^T + (alpha/r) (x A^T) B^T in fp64 (see oracle_apply).

    x: [T][d_in], W: [d_out][d_in] (fp64-convertible).
    adapters: {slot: (A [r][d_in], B [d_out][r], r, alpha)} -- registered slots.
    Returns (y [T][d_out] fp64, invalid [T] int32).
    """
    lib = load()
    x = to_f64(x)
    W = to_f64(W)
    idx = _i32(idx).reshape(-1)
    T, d_in = x.shape
    d_out = W.shape[0]
    assert W.shape[1] == d_in and idx.shape[0] == T
    S = int(n_slots)
    active = np.zeros(S, np.int32)
    rank = np.zeros(S, np.int32)
    alpha = np.zeros(S, np.float64)
    a_off = np.zeros(S, np.int64)
    b_off = np.zeros(S, np.int64)
    a_parts, b_parts = [], []
    a_pos = b_pos = 0
    for slot, (A, B, r, al) in sorted(adapters.items()):
        A = to_f64(A)
        B = to_f64(B)
        r = int(r)
        assert A.shape == (r, d_in), (A.shape, r, d_in)
        assert B.shape == (d_out, r), (B.shape, d_out, r)
        active[slot] = 1
        rank[slot] = r
        alpha[slot] = float(al)
        a_off[slot] = a_pos
        b_off[slot] = b_pos
        a_parts.append(A.reshape(-1))
        b_parts.append(B.reshape(-1))
        a_pos += A.size
        b_pos += B.size
    A_cat = np.ascontiguousarray(np.concatenate(a_parts) if a_parts else np.zeros(1))
    B_cat = np.ascontiguousarray(np.concatenate(b_parts) if b_parts else np.zeros(1))
    y = np.zeros((T, d_out), np.float64)
    invalid = np.zeros(max(T, 1), np.int32)
    rc = lib.oracle_apply(T, d_in, d_out, S, x, W, idx, active, rank, alpha,
                          A_cat, a_off, B_cat, b_off, y, invalid, int(n_threads))
    if rc < 0:
        raise MemoryError("oracle_apply failed")
    return y, invalid[:T]
