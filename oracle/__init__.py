"""fp64 CPU attention-forward oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It computes the plain definition of attention forward
(Q·Kᵀ -> scale -> mask -> softmax as Map(exp) -> Reduce(+) -> Zip(/) -> ×V,
"CS149 L11: Programming Specialized Hardware", section 5, slides 48 and 54)
in fp64 C code (``attn_oracle.c``), and shares nothing with the HIP library.

Functions:
    attention_fp64(q, k, v, causal, scale, rows=None, threads=0, drop_thr=0, seed=0)
        q: [B, H_q, N_q, d_qk], k: [B, H_kv, N_kv, d_qk], v: [B, H_kv, N_kv, d_v]
        (torch tensors or numpy arrays of any float dtype; values are widened
        to fp32, which is exact for bf16 and fp32 inputs).
        scale: the fp32 softmax scale (widened to fp64 inside).
        rows: optional int array of shape [R, 3] holding (b, h, i) triples; then
        O is [R, d_v] and lse is [R]. Without rows, O is [B, H_q, N_q, d_v]
        and lse is [B, H_q, N_q].
        Returns (O, lse, threads_used) as float64 numpy arrays and an int.
        drop_thr (1..255) applies dropout at probability drop_thr / 256: each
        p_j is kept (and scaled by 256 / (256 - drop_thr)) when its byte of
        the counter-based generator Philox4x32-10 is >= drop_thr; lse is that
        of the softmax before dropout.
    philox4x32_10(ctr, key): one block of that generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind_lib(path: str):
    lib = ctypes.CDLL(path)
    f = lib.attn_oracle_fp64
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    I = ctypes.c_int64
    f.argtypes = [P, P, P, I, I, I, I, I, I, I, ctypes.c_int, ctypes.c_float,
                  P, I, P, P, ctypes.c_int]
    f = lib.attn_oracle_dropout_fp64
    f.restype = ctypes.c_int
    f.argtypes = [P, P, P, I, I, I, I, I, I, I, ctypes.c_int, ctypes.c_float,
                  P, I, P, P, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64]
    f = lib.oracle_philox4x32_10
    f.restype = None
    f.argtypes = [P, P, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = _bind_lib(_LIB)
    return _lib


def _as_f32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def philox4x32_10(ctr, key) -> np.ndarray:
    """The oracle's Philox4x32-10 block: 4 uint32 counter words, 2 key words
    -> 4 uint32 output words."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.empty(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def attention_fp64(q, k, v, causal: bool, scale: float, rows=None, threads: int = 0,
                   lib_path: str | None = None, drop_thr: int = 0, seed: int = 0):
    """See the module docstring. ``lib_path`` binds another build of the same
    C source (the test suite uses it for deliberately broken copies).
    ``drop_thr`` in 1..255 applies dropout at probability drop_thr / 256 with
    the generator seed ``seed`` (0 = no dropout)."""
    lib = _bind_lib(lib_path) if lib_path else _load()
    Q, K, V = _as_f32(q), _as_f32(k), _as_f32(v)
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, dqk = Q.shape
    Bk, Hkv, Nkv, dk = K.shape
    Bv, Hv, Nv, dv = V.shape
    if (Bk, dk) != (B, dqk) or (Bv, Hv, Nv) != (Bk, Hkv, Nkv):
        raise ValueError("shape mismatch between q, k, v")
    if rows is None:
        n_rows = B * Hq * Nq
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n_rows = rows_arr.shape[0]
        rows_ptr = rows_arr.ctypes.data
    O = np.empty((n_rows, dv), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    if drop_thr:
        rc = lib.attn_oracle_dropout_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                          B, Hq, Hkv, Nq, Nkv, dqk, dv, int(bool(causal)),
                                          float(np.float32(scale)), rows_ptr, n_rows,
                                          O.ctypes.data, lse.ctypes.data, int(threads),
                                          int(drop_thr), int(seed) & (2 ** 64 - 1))
    else:
        rc = lib.attn_oracle_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                  B, Hq, Hkv, Nq, Nkv, dqk, dv, int(bool(causal)),
                                  float(np.float32(scale)), rows_ptr, n_rows,
                                  O.ctypes.data, lse.ctypes.data, int(threads))
    if rc <= 0:
        raise ValueError("attn_oracle_fp64 failed with code %d" % rc)
    if rows is None:
        O = O.reshape(B, Hq, Nq, dv)
        lse = lse.reshape(B, Hq, Nq)
    return O, lse, rc
