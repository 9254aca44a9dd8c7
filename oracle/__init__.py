"""Float64 CPU oracle for NSA selection attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports, links or calls it, and it never imports the product package.

The arithmetic lives in ``nsa_oracle.c`` (plain C, float64, optional OpenMP
over rows/keys); this file builds it with gcc, loads it with ctypes and adds
the packed-sequence split: a packed batch is, by definition, independent
dense B=1 problems, one per sequence (page 3 of the reference text, the
cudnn-frontend backward pull request, passes cumulative sequence lengths for
packed THD tensors; no key crosses a sequence boundary).

Where the method's source pages are silent the oracle takes these readings:
  * a row's key set is the union of the listed blocks (set semantics: a block
    listed twice counts once); negative or >= NB entries are skipped;
  * causality applies to every listed block (key j <= query t), so a listed
    future block adds nothing; an empty row gives o = 0, lse = -inf, dq = 0;
  * scale defaults to 1/sqrt(D); lse is natural-log and includes the scale;
  * an optional sliding window W (keys t - W < j <= t), a mask on keys only;
  * dense problems may have Tk >= T keys (k/v [B, Hkv, Tk, D]): the queries
    are the last T key positions (bottom-right causal alignment, one of the
    backward flavours page 3 lists), query t at position t + Tk - T, which
    replaces t in the causal and window limits;
  * an optional attention sink (page 3 names a dSink backward step, nothing
    more): a per-head logit, no scale, in every row's softmax denominator
    with no value; lse includes it, dq/dk/dv keep their formulas with that
    lse, and dsink[h] = -sum over head h's rows of exp(sink[h] - lse) Delta.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile nsa_oracle.c with gcc -O2 (no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    i, d, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
    shape = [i, i, i, i, i, i, i, d, dp, i, i]
    lib.nsa_oracle_fwd_rows.argtypes = shape + [dp, dp, dp, ip, i64, lp, dp, dp]
    lib.nsa_oracle_bwd_rows.argtypes = shape + [dp, dp, dp, dp, ip, i64, lp, dp, dp, dp]
    lib.nsa_oracle_dkdv_keys.argtypes = shape + [dp, dp, dp, dp, ip, dp, dp, i64, lp, dp, dp]
    lib.nsa_oracle_invert.argtypes = [i, i, i, i, i, i, i, ip, ip, ip, i64]
    lib.nsa_oracle_invert.restype = i64
    lib.nsa_oracle_count_pairs.argtypes = [i, i, i, i, i, i, i, ip]
    lib.nsa_oracle_count_pairs.restype = i64
    lib.nsa_oracle_num_threads.restype = i
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().nsa_oracle_num_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.int32)


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _shape(q, k, idx, block_size, scale, sink=None, window=0):
    """The C shape arguments; sink (per-head logits) is passed as a pointer
    to a float64 copy that the returned tuple keeps alive."""
    B, Hq, T, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    S = idx.shape[-1]
    if scale is None:
        scale = D ** -0.5
    if k.shape != (B, Hkv, Tk, D) or Tk < T or idx.shape != (B, Hkv, T, S) or Hq % Hkv:
        raise ValueError("inconsistent shapes")
    sk = None if sink is None else _f64(sink).reshape(-1)
    if sk is not None and sk.shape != (Hq,):
        raise ValueError("sink must hold one logit per query head")
    ptr = None if sk is None else _ptr(sk, ctypes.c_double)
    if window is None or window < 0:
        raise ValueError("window must be >= 0 (0: none)")
    return _Shape((B, Hq, Hkv, T, D, S, int(block_size), float(scale), ptr, int(window), Tk), sk)


class _Shape(tuple):
    """Shape arguments plus the sink array they point into."""
    def __new__(cls, args, keep):
        t = super().__new__(cls, args)
        t.keep = keep
        return t


def fwd_rows(q, k, v, block_idx, block_size, rows=None, scale=None, sink=None, window=0):
    """Forward of the listed flat rows ((b*Hq + h)*T + t); all rows if None.
    Returns (o [n, D], lse [n])."""
    q, k, v, idx = _f64(q), _f64(k), _f64(v), _i32(block_idx)
    sh = _shape(q, k, idx, block_size, scale, sink, window)
    n = q.shape[0] * q.shape[1] * q.shape[2] if rows is None else len(rows)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    o = np.zeros((n, sh[4]))
    lse = np.zeros(n)
    rc = _load().nsa_oracle_fwd_rows(*sh, _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                     _ptr(v, ctypes.c_double), _ptr(idx, ctypes.c_int32), n,
                                     None if r is None else _ptr(r, ctypes.c_int64),
                                     _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc:
        raise RuntimeError(f"oracle fwd failed ({rc})")
    return o, lse


def bwd_rows(q, k, v, dO, block_idx, block_size, rows=None, scale=None, want_dq=True,
             sink=None, window=0):
    """lse, Delta and dq of the listed rows.  Returns (lse [n], delta [n], dq [n, D])."""
    q, k, v, dO, idx = _f64(q), _f64(k), _f64(v), _f64(dO), _i32(block_idx)
    sh = _shape(q, k, idx, block_size, scale, sink, window)
    n = q.shape[0] * q.shape[1] * q.shape[2] if rows is None else len(rows)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    lse, delta = np.zeros(n), np.zeros(n)
    dq = np.zeros((n, sh[4])) if want_dq else None
    rc = _load().nsa_oracle_bwd_rows(*sh, _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                     _ptr(v, ctypes.c_double), _ptr(dO, ctypes.c_double),
                                     _ptr(idx, ctypes.c_int32), n,
                                     None if r is None else _ptr(r, ctypes.c_int64),
                                     _ptr(lse, ctypes.c_double), _ptr(delta, ctypes.c_double),
                                     None if dq is None else _ptr(dq, ctypes.c_double))
    if rc:
        raise RuntimeError(f"oracle bwd failed ({rc})")
    return lse, delta, dq


def dkdv_keys(q, k, v, dO, block_idx, block_size, row_lse, row_delta, keys=None, scale=None,
              window=0):
    """dk, dv of the listed flat keys ((b*Hkv + hkv)*Tk + j); all keys if None.
    row_lse/row_delta: every row, shaped or flat [B*Hq*T]."""
    q, k, v, dO, idx = _f64(q), _f64(k), _f64(v), _f64(dO), _i32(block_idx)
    sh = _shape(q, k, idx, block_size, scale, None, window)
    lse, delta = _f64(row_lse).reshape(-1), _f64(row_delta).reshape(-1)
    n = k.shape[0] * k.shape[1] * k.shape[2] if keys is None else len(keys)
    kk = None if keys is None else np.ascontiguousarray(keys, dtype=np.int64)
    dk, dv = np.zeros((n, sh[4])), np.zeros((n, sh[4]))
    rc = _load().nsa_oracle_dkdv_keys(*sh, _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                      _ptr(v, ctypes.c_double), _ptr(dO, ctypes.c_double),
                                      _ptr(idx, ctypes.c_int32), _ptr(lse, ctypes.c_double),
                                      _ptr(delta, ctypes.c_double), n,
                                      None if kk is None else _ptr(kk, ctypes.c_int64),
                                      _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc:
        raise RuntimeError(f"oracle dkdv failed ({rc})")
    return dk, dv


def fwd(q, k, v, block_idx, block_size, scale=None, sink=None, window=0):
    """Dense forward: o like q, lse [B, Hq, T] (sink: optional [Hq] logits;
    window: sliding-window width, 0 for none)."""
    B, Hq, T, D = np.shape(q)
    o, lse = fwd_rows(q, k, v, block_idx, block_size, None, scale, sink, window)
    return o.reshape(B, Hq, T, D), lse.reshape(B, Hq, T)


def bwd(q, k, v, dO, block_idx, block_size, scale=None, sink=None, window=0):
    """Dense backward: (dq, dk, dv, lse, delta); lse includes the sink if any."""
    B, Hq, T, D = np.shape(q)
    Hkv, Tk = np.shape(k)[1], np.shape(k)[2]
    lse, delta, dq = bwd_rows(q, k, v, dO, block_idx, block_size, None, scale, sink=sink,
                              window=window)
    dk, dv = dkdv_keys(q, k, v, dO, block_idx, block_size, lse, delta, None, scale, window)
    return (dq.reshape(B, Hq, T, D), dk.reshape(B, Hkv, Tk, D), dv.reshape(B, Hkv, Tk, D),
            lse.reshape(B, Hq, T), delta.reshape(B, Hq, T))


def dsink(sink, lse, delta, head_axis: int):
    """Gradient of the per-head sink logits: dsink[h] = -sum over the rows of
    head h of exp(sink[h] - lse) * Delta (o moves by -P_sink * o when the sink
    logit grows, so <dO, do> = -P_sink <dO, o> = -P_sink Delta).  lse/delta:
    the backward's row arrays; head_axis: their query-head axis (1 for dense
    [B, Hq, T], 0 for packed [Hq, Ttot])."""
    sk = _f64(sink).reshape(-1)
    lse, delta = _f64(lse), _f64(delta)
    shp = [1] * lse.ndim
    shp[head_axis] = -1
    p_sink = np.exp(sk.reshape(shp) - lse)
    axes = tuple(a for a in range(lse.ndim) if a != head_axis)
    return -(p_sink * delta).sum(axis=axes)


def invert(block_idx, block_size, window: int = 0, Tk: Optional[int] = None
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Brute-force block -> token lists: for block u the ascending tokens
    whose key position p = t + Tk - T is >= u*bs and that list u (with a
    window W, only those whose window reaches a key of u: (u+1)*bs - 1 >
    p - W).  Tk defaults to T.  Returns (counts [B,Hkv,NB], tokens) with the
    lists concatenated in (b, hkv, u) order, NB = ceil(Tk / bs)."""
    idx = _i32(block_idx)
    B, Hkv, T, S = idx.shape
    Tk = T if Tk is None else int(Tk)
    NB = -(-Tk // block_size)
    counts = np.zeros((B, Hkv, NB), dtype=np.int32)
    cap = max(1, B * Hkv * T * min(S, NB))
    tokens = np.zeros(cap, dtype=np.int32)
    n = _load().nsa_oracle_invert(B, Hkv, T, Tk, S, int(block_size), int(window),
                                  _ptr(idx, ctypes.c_int32), _ptr(counts, ctypes.c_int32),
                                  _ptr(tokens, ctypes.c_int32), cap)
    if n < 0:
        raise RuntimeError("oracle invert: capacity exceeded")
    return counts, tokens[:n].copy()


def count_pairs(block_idx, Hq: int, block_size: int, Tk: Optional[int] = None) -> int:
    """Useful (query-head row, key) pair count N = sum over rows of |A|
    (Tk keys per group, default T)."""
    idx = _i32(block_idx)
    B, Hkv, T, S = idx.shape
    Tk = T if Tk is None else int(Tk)
    return int(_load().nsa_oracle_count_pairs(B, Hq, Hkv, T, Tk, S, int(block_size),
                                              _ptr(idx, ctypes.c_int32)))


# ---- packed (THD) helpers: one dense B=1 problem per sequence -------------

def _seq(x_thd: np.ndarray, a: int, b: int) -> np.ndarray:
    """[Ttot, H, D] slice of one sequence -> [1, H, L, D]."""
    return np.ascontiguousarray(np.asarray(x_thd)[a:b].transpose(1, 0, 2))[None]


def fwd_thd(q, k, v, block_idx, cu_seqlens, block_size, scale=None, sink=None, window=0):
    """Packed forward: q [Ttot,Hq,D], k/v [Ttot,Hkv,D], block_idx [Hkv,Ttot,S].
    Returns (o [Ttot,Hq,D], lse [Hq,Ttot])."""
    Ttot, Hq, D = np.shape(q)
    o = np.zeros((Ttot, Hq, D))
    lse = np.zeros((Hq, Ttot))
    for z in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[z]), int(cu_seqlens[z + 1])
        if b == a:
            continue
        oz, lz = fwd(_seq(q, a, b), _seq(k, a, b), _seq(v, a, b),
                     np.asarray(block_idx)[:, a:b][None], block_size, scale, sink, window)
        o[a:b] = oz[0].transpose(1, 0, 2)
        lse[:, a:b] = lz[0]
    return o, lse


def bwd_thd(q, k, v, dO, block_idx, cu_seqlens, block_size, scale=None, sink=None, window=0):
    """Packed backward: (dq, dk, dv) in the packed layouts, plus lse, delta [Hq,Ttot]."""
    Ttot, Hq, D = np.shape(q)
    Hkv = np.shape(k)[1]
    dq, dk, dv = np.zeros((Ttot, Hq, D)), np.zeros((Ttot, Hkv, D)), np.zeros((Ttot, Hkv, D))
    lse, delta = np.zeros((Hq, Ttot)), np.zeros((Hq, Ttot))
    for z in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[z]), int(cu_seqlens[z + 1])
        if b == a:
            continue
        r = bwd(_seq(q, a, b), _seq(k, a, b), _seq(v, a, b), _seq(dO, a, b),
                np.asarray(block_idx)[:, a:b][None], block_size, scale, sink, window)
        dq[a:b] = r[0][0].transpose(1, 0, 2)
        dk[a:b] = r[1][0].transpose(1, 0, 2)
        dv[a:b] = r[2][0].transpose(1, 0, 2)
        lse[:, a:b] = r[3][0]
        delta[:, a:b] = r[4][0]
    return dq, dk, dv, lse, delta


def count_pairs_thd(block_idx, cu_seqlens, Hq: int, block_size: int) -> int:
    n = 0
    for z in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[z]), int(cu_seqlens[z + 1])
        if b > a:
            n += count_pairs(np.asarray(block_idx)[:, a:b][None], Hq, block_size)
    return n
