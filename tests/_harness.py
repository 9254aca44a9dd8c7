"""Shared helpers of the GPU tests: upload a seeded draw, run the C-ABI path,
and compute oracle values for full problems or sampled rows/keys."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_attention_nsa_amd as nsa
import oracle
import workloads

TOL = {"f32": 2e-3, "bf16": 6e-2}  # max-abs gates of page 1's TOL table (atol)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(w: workloads.Workload, dev="cuda"):
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt).contiguous()
    d = dict(q=t(w.q), k=t(w.k), v=t(w.v), dO=t(w.dO),
             idx=torch.from_numpy(np.ascontiguousarray(w.block_idx, dtype=np.int32)).to(dev),
             cu=None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev))
    return d


def run_gpu(w: workloads.Workload, d=None, stream=None):
    """fwd + bwd through the C ABI; returns float64 numpy outputs."""
    d = d or to_dev(w)
    ms = None if not w.packed else w.max_seqlen
    o, lse = nsa.nsa_sel_fwd(d["q"], d["k"], d["v"], d["idx"], w.block_size, w.scale, d["cu"], ms)
    dq, dk, dv = nsa.nsa_sel_bwd(d["q"], d["k"], d["v"], o, lse, d["dO"], d["idx"], w.block_size,
                                 w.scale, d["cu"], ms)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    return dict(o=f(o), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv))


def oracle_full(w: workloads.Workload):
    """Full float64 oracle outputs in the workload's layout."""
    if w.packed:
        o, lse = oracle.fwd_thd(w.q, w.k, w.v, w.block_idx, w.cu_seqlens, w.block_size, w.scale)
        dq, dk, dv, _, _ = oracle.bwd_thd(w.q, w.k, w.v, w.dO, w.block_idx, w.cu_seqlens,
                                          w.block_size, w.scale)
    else:
        o, lse = oracle.fwd(w.q, w.k, w.v, w.block_idx, w.block_size, w.scale)
        dq, dk, dv, _, _ = oracle.bwd(w.q, w.k, w.v, w.dO, w.block_idx, w.block_size, w.scale)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def dsink_bound(w, got, ref, sink, lse_ref, delta_ref):
    """Per-head bound on |dsink_gpu - dsink_oracle| derived from the arithmetic
    the GPU performs on the o and lse it produced itself (the pages fix no
    dsink tolerance).  Per row r of head h the GPU adds P_g * Delta_g with
    Delta_g = fp32 sum of dO * o_gpu and P_g = exp(sink[h] - lse_gpu) in fp32;
    the oracle adds P_r * Delta_r in float64.  With u = 2^-24:
      |Delta_g - Delta_r| <= |<dO, o_gpu - o_ref>| + D u sum|dO o_gpu|
      |P_g - P_r|         <= P_r (exp(|lse_gpu - lse_ref| + 8u) - 1)
    and the fixed-order fp32 sum over the head's rows adds at most
    rows * u * sum|P_r Delta_g|.  Returns [Hq] bounds.
    got/ref: GPU / oracle o (and dO from w) in the workload layout;
    lse_ref / delta_ref: the oracle backward's row arrays."""
    u = 2.0 ** -24
    f = lambda x: np.asarray(x, np.float64)
    if w.packed:   # [T, Hq, D] -> [Hq, T, D]; lse [Hq, T]
        o_g, o_r, dO = (f(x).transpose(1, 0, 2) for x in (got["o"], ref["o"], w.dO))
        lse_g, lse_r, dl_r = f(got["lse"]), f(lse_ref), f(delta_ref)
    else:          # [B, Hq, T, D] -> [Hq, B*T, D]; lse [B, Hq, T] -> [Hq, B*T]
        hm = lambda x: f(x).transpose(1, 0, 2, 3).reshape(w.Hq, -1, w.D)
        o_g, o_r, dO = hm(got["o"]), hm(ref["o"]), hm(w.dO)
        hl = lambda x: f(x).transpose(1, 0, 2).reshape(w.Hq, -1)
        lse_g, lse_r, dl_r = hl(got["lse"]), hl(lse_ref), hl(delta_ref)
    sk = f(sink)[:, None]
    P_r = np.exp(sk - lse_r)
    dl_g = np.sum(dO * o_g, axis=-1)
    e_dl = np.abs(np.sum(dO * (o_g - o_r), axis=-1)) + w.D * u * np.sum(np.abs(dO * o_g), axis=-1)
    e_dl = np.maximum(e_dl, np.abs(dl_g - dl_r))
    e_p = P_r * np.expm1(np.abs(lse_g - lse_r) + 8 * u)
    rows = lse_r.shape[1]
    term = P_r * e_dl + np.abs(dl_g) * e_p
    return term.sum(axis=1) + rows * u * np.sum(np.abs(P_r * dl_g), axis=1)


def max_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0, bool(np.isnan(d).any())


def assert_close(name, got, ref, tol):
    err, nan = max_err(got, ref)
    mag = float(np.max(np.abs(np.where(np.isinf(ref), 0, ref)))) if np.size(ref) else 0.0
    say(f"  {name}: max|err| = {err:.3e} (tol {tol:g}, max|ref| = {mag:.3g})")
    assert not nan, f"{name}: NaN in comparison"
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol}"


# ---- sampled oracle values on one dense (b) slice or one packed sequence ----

def dense_view(w: workloads.Workload, z: int):
    """(q, k, v, dO, block_idx) of batch entry / sequence z as a dense B=1 problem."""
    if not w.packed:
        sl = slice(z, z + 1)
        return w.q[sl], w.k[sl], w.v[sl], w.dO[sl], w.block_idx[sl]
    a, b = int(w.cu_seqlens[z]), int(w.cu_seqlens[z + 1])
    tr = lambda x: np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]
    return tr(w.q), tr(w.k), tr(w.v), tr(w.dO), np.ascontiguousarray(w.block_idx[:, a:b])[None]


def gpu_rows(w, out, z, h, t):
    """GPU values of query rows (z, h, t[]) from full outputs."""
    if w.packed:
        tok = int(w.cu_seqlens[z]) + np.asarray(t)
        return out["o"][tok, h], out["lse"][h, tok], out["dq"][tok, h]
    return out["o"][z, h, t], out["lse"][z, h, t], out["dq"][z, h, t]


def gpu_keys(w, out, z, hkv, j):
    if w.packed:
        tok = int(w.cu_seqlens[z]) + np.asarray(j)
        return out["dk"][tok, hkv], out["dv"][tok, hkv]
    return out["dk"][z, hkv, j], out["dv"][z, hkv, j]


def oracle_rows(w, z, h, t):
    q, k, v, dO, idx = dense_view(w, z)
    T = q.shape[2]
    rows = h * T + np.asarray(t, dtype=np.int64)
    o, lse = oracle.fwd_rows(q, k, v, idx, w.block_size, rows, w.scale)
    _, _, dq = oracle.bwd_rows(q, k, v, dO, idx, w.block_size, rows, w.scale)
    return o, lse, dq


def oracle_block_keys(w, z, hkv, u):
    """dk, dv of every key of block u (of batch entry / sequence z, KV head
    hkv).  Only the rows that attend to block u get their lse/Delta computed:
    membership is read from block_idx here, not from any GPU structure."""
    q, k, v, dO, idx = dense_view(w, z)
    T = q.shape[2]
    G = w.Hq // w.Hkv
    bs = w.block_size
    toks = [t for t in range(u * bs, T) if u in set(idx[0, hkv, t].tolist())]
    heads = np.arange(hkv * G, (hkv + 1) * G)
    rows = (heads[None, :] * T + np.asarray(toks, dtype=np.int64)[:, None]).reshape(-1)
    lse_all = np.full(w.Hq * T, np.nan)
    dl_all = np.full(w.Hq * T, np.nan)
    if len(rows):
        lse_r, dl_r, _ = oracle.bwd_rows(q, k, v, dO, idx, bs, rows, w.scale, want_dq=False)
        lse_all[rows] = lse_r
        dl_all[rows] = dl_r
    j = np.arange(u * bs, min((u + 1) * bs, T))
    keys = hkv * T + j
    dk, dv = oracle.dkdv_keys(q, k, v, dO, idx, bs, lse_all, dl_all, keys, w.scale)
    return j, dk, dv, len(toks)
