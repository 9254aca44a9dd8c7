"""NSA selection attention on MI355X (gfx950): a thin binding over the C ABI
of libnsa_sel.so (include/nsa_sel.h).

The binding only marshals arguments: it reads shapes from torch tensors,
allocates outputs and the backward workspace with torch (device memory), and
passes raw pointers and the current HIP stream to the library.  Every step of
the computation runs in the library's HIP kernels; there is no other path.

Layouts (page 1 of the reference text, run_one): dense q/dO [B, Hq, T, D],
k/v [B, Hkv, T, D], block_idx [B, Hkv, T, S] int32.  Packed sequences
(page 3, cumulative sequence lengths): q [T, Hq, D], k/v [T, Hkv, D],
block_idx [Hkv, T, S] with sequence-local block numbers, cu_seqlens int32
[n_seqs + 1] on the device.  q, k, v, o, dO and the gradients may be strided
views (e.g. a [B, T, H, D] buffer transposed to [B, H, T, D]) as long as the
last dimension is contiguous: their strides are passed to the library, which
checks them.  block_idx, lse and cu_seqlens must be contiguous.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

__all__ = [
    "nsa_sel_fwd",
    "nsa_sel_bwd",
    "BwdStages",
    "nsa_sel_delta",
    "nsa_sel_invert",
    "nsa_sel_check_block_idx",
    "bwd_workspace_bytes",
    "make_problem",
    "set_strides",
    "wait_timeouts",
    "ds_handoff",
    "build_git",
    "selection_attn",
    "SelectionAttn",
]

_DTYPES = {torch.float32: _lib.NSA_F32, torch.bfloat16: _lib.NSA_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


_STRIDE_FIELDS = {"q": "stride_q", "k": "stride_k", "v": "stride_v", "o": "stride_o",
                  "dO": "stride_do", "dq": "stride_dq", "dk": "stride_dk", "dv": "stride_dv"}


def set_strides(p: _lib.Problem, **tensors: Optional[torch.Tensor]) -> _lib.Problem:
    """Record the (batch entry, head, token) element strides of the given
    tensors (names q, k, v, o, dO, dq, dk, dv) in the problem and mark it
    strided.  Dense tensors are [B, H, T, D] views, packed ones [T, H, D]."""
    p.strided = 1
    for name, t in tensors.items():
        if t is None:
            continue
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous (stride {t.stride(-1)})")
        arr = getattr(p, _STRIDE_FIELDS[name])
        if t.dim() == 4:
            arr[0], arr[1], arr[2] = t.stride(0), t.stride(1), t.stride(2)
        else:
            arr[0], arr[1], arr[2] = 0, t.stride(1), t.stride(0)
    return p


def make_problem(q: torch.Tensor, k: torch.Tensor, block_idx: torch.Tensor, block_size: int,
                 scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
                 max_seqlen: Optional[int] = None, window: int = 0) -> _lib.Problem:
    """The nsa_sel_problem describing these tensors (contiguous layouts until
    set_strides records the actual strides).  Dense k may hold more tokens
    than q (Tk >= T): the queries are then the last T key positions
    (bottom-right causal alignment)."""
    if q.dtype not in _DTYPES:
        raise TypeError(f"q dtype {q.dtype} is not float32 or bfloat16")
    p = _lib.Problem()
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4 or block_idx.dim() != 4:
            raise ValueError("dense layout needs q/k [B, H, T, D] and block_idx [B, Hkv, T, S]")
        p.layout = _lib.NSA_DENSE
        p.B, p.Hq, p.T, p.D = q.shape
        p.Hkv = k.shape[1]
        p.Tk = k.shape[2]
        p.S = block_idx.shape[-1]
        p.n_seqs, p.max_seqlen = 0, 0
    else:
        if q.dim() != 3 or k.dim() != 3 or block_idx.dim() != 3:
            raise ValueError("packed layout needs q/k [T, H, D] and block_idx [Hkv, T, S]")
        p.layout = _lib.NSA_PACKED
        p.B = 1
        p.T, p.Hq, p.D = q.shape
        p.Hkv = k.shape[1]
        p.S = block_idx.shape[-1]
        p.n_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if p.n_seqs else 0
        p.max_seqlen = int(max_seqlen)
    p.block_size = int(block_size)
    p.dtype = _DTYPES[q.dtype]
    p.scale = float(q.shape[-1] ** -0.5 if scale is None else scale)
    p.window = int(window)
    return p


def _check_tensors(q, k, v, block_idx, cu_seqlens, p: _lib.Problem):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    if block_idx.dtype != torch.int32 or not block_idx.is_contiguous():
        raise TypeError("block_idx must be a contiguous int32 tensor")
    dense = cu_seqlens is None
    want_k = (p.B, p.Hkv, p.Tk, p.D) if dense else (p.T, p.Hkv, p.D)
    want_i = (p.B, p.Hkv, p.T, p.S) if dense else (p.Hkv, p.T, p.S)
    if tuple(k.shape) != want_k or tuple(block_idx.shape) != want_i:
        raise ValueError(f"shape mismatch: k {tuple(k.shape)} (want {want_k}), "
                         f"block_idx {tuple(block_idx.shape)} (want {want_i})")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous()):
        raise TypeError("cu_seqlens must be a contiguous int32 tensor")


def _lse_shape(q, cu_seqlens):
    return tuple(q.shape[:3]) if cu_seqlens is None else (q.shape[1], q.shape[0])


def _check_sink(sink, p: _lib.Problem):
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() != p.Hq:
        raise ValueError("sink must be a contiguous float32 tensor of Hq logits")


def nsa_sel_fwd(q, k, v, block_idx, block_size, scale=None, cu_seqlens=None, max_seqlen=None,
                out=None, lse=None, sink=None, window=0) -> Tuple[torch.Tensor, torch.Tensor]:
    """o, lse = forward (nsa_sel_fwd; nsa_sel_fwd_sink with per-head sink
    logits); window > 0: sliding window of that many keys."""
    p = make_problem(q, k, block_idx, block_size, scale, cu_seqlens, max_seqlen, window)
    _check_tensors(q, k, v, block_idx, cu_seqlens, p)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    lse_t = torch.empty(_lse_shape(q, cu_seqlens), dtype=torch.float32, device=q.device) if lse is None else lse
    if not lse_t.is_contiguous():
        raise ValueError("lse must be contiguous")
    set_strides(p, q=q, k=k, v=v, o=o)
    lib = _lib.load()
    if sink is None:
        st = lib.nsa_sel_fwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(cu_seqlens),
                             _ptr(o), _ptr(lse_t), _stream())
        _lib.check("nsa_sel_fwd", st)
    else:
        _check_sink(sink, p)
        st = lib.nsa_sel_fwd_sink(p, _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(cu_seqlens),
                                  _ptr(sink), _ptr(o), _ptr(lse_t), _stream())
        _lib.check("nsa_sel_fwd_sink", st)
    return o, lse_t


def bwd_workspace_bytes(p: _lib.Problem) -> int:
    n = _lib.load().nsa_sel_bwd_workspace_bytes(p)
    err = _lib.last_error()
    if err:
        raise _lib.NsaError("nsa_sel_bwd_workspace_bytes", _lib.NSA_ERR_INVALID_ARG, err)
    return int(n)


def ds_handoff(p: _lib.Problem) -> bool:
    """Whether the backward of this problem hands dS from dK/dV over to dQ
    (nsa_sel_bwd_ds_handoff)."""
    r = _lib.load().nsa_sel_bwd_ds_handoff(p)
    if r < 0:
        raise _lib.NsaError("nsa_sel_bwd_ds_handoff", _lib.NSA_ERR_INVALID_ARG, _lib.last_error())
    return bool(r)


def build_git() -> str:
    """The commit the loaded library was built from (nsa_build_git)."""
    return _lib.load().nsa_build_git().decode()


def nsa_sel_bwd(q, k, v, o, lse, dO, block_idx, block_size, scale=None, cu_seqlens=None,
                max_seqlen=None, workspace=None, dq=None, dk=None, dv=None, sink=None, window=0,
                sched_policy=0):
    """dq, dk, dv = backward (nsa_sel_bwd); with sink logits (lse from the
    sink forward) also dsink, from nsa_sel_bwd_dsink on the same workspace:
    dq, dk, dv, dsink.  sched_policy: nsa_sel_problem.sched_policy."""
    p = make_problem(q, k, block_idx, block_size, scale, cu_seqlens, max_seqlen, window)
    p.sched_policy = int(sched_policy)
    _check_tensors(q, k, v, block_idx, cu_seqlens, p)
    for name, t in (("o", o), ("dO", dO)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    nbytes = bwd_workspace_bytes(p)
    ws = workspace
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    set_strides(p, q=q, k=k, v=v, o=o, dO=dO, dq=dq, dk=dk, dv=dv)
    st = _lib.load().nsa_sel_bwd(p, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                 _ptr(block_idx), _ptr(cu_seqlens), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(ws), ws.numel(), _stream())
    _lib.check("nsa_sel_bwd", st)
    if sink is None:
        return dq, dk, dv
    _check_sink(sink, p)
    dsink = torch.empty_like(sink)
    st = _lib.load().nsa_sel_bwd_dsink(p, _ptr(lse), _ptr(sink), _ptr(cu_seqlens), _ptr(dsink),
                                       _ptr(ws), ws.numel(), _stream())
    _lib.check("nsa_sel_bwd_dsink", st)
    return dq, dk, dv, dsink


class BwdStages:
    """The backward as its three C-ABI stages on one workspace
    (nsa_sel_bwd_prepare, nsa_sel_bwd_dkdv, nsa_sel_bwd_dq); calling them in
    that order equals nsa_sel_bwd (dq may read the dS the dK/dV stage hands
    over, so it comes last).  Buffers are allocated once here."""

    def __init__(self, q, k, v, block_idx, block_size, scale=None, cu_seqlens=None,
                 max_seqlen=None, window=0, sched_policy=0):
        self.p = make_problem(q, k, block_idx, block_size, scale, cu_seqlens, max_seqlen, window)
        self.p.sched_policy = int(sched_policy)
        _check_tensors(q, k, v, block_idx, cu_seqlens, self.p)
        self.q, self.k, self.v, self.idx, self.cu = q, k, v, block_idx, cu_seqlens
        self.ws = torch.empty(max(bwd_workspace_bytes(self.p), 1), dtype=torch.uint8,
                              device=q.device)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        set_strides(self.p, q=q, k=k, v=v, dq=self.dq, dk=self.dk, dv=self.dv)
        self.lib = _lib.load()
        self.ds_handoff = ds_handoff(self.p)

    def prepare(self, o, dO):
        set_strides(self.p, o=o, dO=dO)
        st = self.lib.nsa_sel_bwd_prepare(self.p, _ptr(o), _ptr(dO), _ptr(self.idx),
                                          _ptr(self.cu), _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_prepare", st)

    def prepare_lists(self):
        """The inversion and dK/dV plan alone (nsa_sel_bwd_prepare_lists):
        needs only block_idx, so it may run during the forward."""
        st = self.lib.nsa_sel_bwd_prepare_lists(self.p, _ptr(self.idx), _ptr(self.cu),
                                                _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_prepare_lists", st)

    def prepare_delta(self, o, dO):
        """Delta alone (nsa_sel_bwd_prepare_delta); with prepare_lists it
        equals prepare."""
        set_strides(self.p, o=o, dO=dO)
        st = self.lib.nsa_sel_bwd_prepare_delta(self.p, _ptr(o), _ptr(dO), _ptr(self.cu),
                                                _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_prepare_delta", st)

    def dq_stage(self, dO, lse):
        set_strides(self.p, dO=dO)
        st = self.lib.nsa_sel_bwd_dq(self.p, _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(dO),
                                     _ptr(lse), _ptr(self.idx), _ptr(self.cu), _ptr(self.dq),
                                     _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_dq", st)
        return self.dq

    def dkdv_stage(self, dO, lse):
        set_strides(self.p, dO=dO)
        st = self.lib.nsa_sel_bwd_dkdv(self.p, _ptr(self.q), _ptr(self.k), _ptr(self.v),
                                       _ptr(dO), _ptr(lse), _ptr(self.cu), _ptr(self.dk),
                                       _ptr(self.dv), _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_dkdv", st)
        return self.dk, self.dv

    def dkdv_blocks(self, dO, lse):
        """First kernel of the dK/dV stage (nsa_sel_bwd_dkdv_blocks)."""
        set_strides(self.p, dO=dO)
        st = self.lib.nsa_sel_bwd_dkdv_blocks(self.p, _ptr(self.q), _ptr(self.k), _ptr(self.v),
                                              _ptr(dO), _ptr(lse), _ptr(self.cu), _ptr(self.dk),
                                              _ptr(self.dv), _ptr(self.ws), self.ws.numel(),
                                              _stream())
        _lib.check("nsa_sel_bwd_dkdv_blocks", st)

    def dkdv_reduce(self):
        """Second kernel of the dK/dV stage (nsa_sel_bwd_dkdv_reduce)."""
        st = self.lib.nsa_sel_bwd_dkdv_reduce(self.p, _ptr(self.cu), _ptr(self.dk), _ptr(self.dv),
                                              _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_dkdv_reduce", st)
        return self.dk, self.dv

    def dsink_stage(self, lse, sink, out=None):
        """Sink-logit gradient from the prepared workspace (nsa_sel_bwd_dsink)."""
        _check_sink(sink, self.p)
        ds = torch.empty_like(sink) if out is None else out
        st = self.lib.nsa_sel_bwd_dsink(self.p, _ptr(lse), _ptr(sink), _ptr(self.cu), _ptr(ds),
                                        _ptr(self.ws), self.ws.numel(), _stream())
        _lib.check("nsa_sel_bwd_dsink", st)
        return ds


def nsa_sel_delta(o, dO, block_size, block_idx, k, scale=None, cu_seqlens=None, max_seqlen=None):
    """Delta = rowsum(dO * o) (nsa_sel_delta), laid out like lse."""
    p = make_problem(o, k, block_idx, block_size, scale, cu_seqlens, max_seqlen)
    set_strides(p, o=o, dO=dO)
    delta = torch.empty(_lse_shape(o, cu_seqlens), dtype=torch.float32, device=o.device)
    st = _lib.load().nsa_sel_delta(p, _ptr(o), _ptr(dO), _ptr(cu_seqlens), _ptr(delta), _stream())
    _lib.check("nsa_sel_delta", st)
    return delta


def nsa_sel_invert(q, k, block_idx, block_size, cu_seqlens=None, max_seqlen=None, window=0):
    """Block -> query lists (nsa_sel_invert): (offsets [Z, Hkv, NBmax+1], tokens)."""
    p = make_problem(q, k, block_idx, block_size, None, cu_seqlens, max_seqlen, window)
    lib = _lib.load()
    cap = int(lib.nsa_sel_invert_tokens_capacity(p))
    Z = p.B if cu_seqlens is None else p.n_seqs
    kmax = (p.Tk or p.T) if cu_seqlens is None else p.max_seqlen  # keys: blocks are key blocks
    nb = -(-kmax // p.block_size)
    offsets = torch.empty((Z, p.Hkv, nb + 1), dtype=torch.int32, device=block_idx.device)
    tokens = torch.empty(max(cap, 1), dtype=torch.int32, device=block_idx.device)
    nbytes = bwd_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=block_idx.device)
    st = lib.nsa_sel_invert(p, _ptr(block_idx), _ptr(cu_seqlens), _ptr(offsets), _ptr(tokens),
                            _ptr(ws), ws.numel(), _stream())
    _lib.check("nsa_sel_invert", st)
    return offsets, tokens


def nsa_sel_check_block_idx(q, k, block_idx, block_size, cu_seqlens=None, max_seqlen=None):
    """Entry counts of block_idx (nsa_sel_check_block_idx): a dict with the
    numbers of padding, out-of-range, future and repeated entries."""
    p = make_problem(q, k, block_idx, block_size, None, cu_seqlens, max_seqlen)
    counts = torch.empty(4, dtype=torch.int64, device=block_idx.device)
    st = _lib.load().nsa_sel_check_block_idx(p, _ptr(block_idx), _ptr(cu_seqlens), _ptr(counts),
                                             _stream())
    _lib.check("nsa_sel_check_block_idx", st)
    c = counts.cpu().tolist()
    return {"padding": c[0], "out_of_range": c[1], "future": c[2], "repeated": c[3]}


def wait_timeouts() -> int:
    """Bounded in-kernel waits that gave up on the current device since the
    library was loaded (nsa_sel_wait_timeouts); 0 is the only healthy value.
    Synchronises the device."""
    import ctypes
    n = ctypes.c_uint64(0)
    st = _lib.load().nsa_sel_wait_timeouts(ctypes.byref(n))
    _lib.check("nsa_sel_wait_timeouts", st)
    return int(n.value)


class SelectionAttn(torch.autograd.Function):
    """o = selection attention; backward through nsa_sel_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, block_idx, block_size, scale, cu_seqlens, max_seqlen, sink=None,
                window=0):
        o, lse = nsa_sel_fwd(q, k, v, block_idx, block_size, scale, cu_seqlens, max_seqlen,
                             sink=sink, window=window)
        ctx.save_for_backward(q, k, v, o, lse, block_idx, cu_seqlens, sink)
        ctx.cfg = (block_size, scale, max_seqlen, window)
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse, block_idx, cu_seqlens, sink = ctx.saved_tensors
        block_size, scale, max_seqlen, window = ctx.cfg
        g = nsa_sel_bwd(q, k, v, o, lse, dO.contiguous(), block_idx, block_size, scale,
                        cu_seqlens, max_seqlen, sink=sink, window=window)
        dsink = g[3] if sink is not None else None
        return g[0], g[1], g[2], None, None, None, None, None, dsink, None


def selection_attn(q, k, v, block_idx, block_size, scale=None, cu_seqlens=None, max_seqlen=None,
                   sink=None, window=0):
    """Differentiable NSA selection attention (page 1's selection_attn call);
    sink: optional per-head sink logits [Hq] float32 (differentiable);
    window > 0: sliding window of that many keys."""
    return SelectionAttn.apply(q, k, v, block_idx, block_size, scale, cu_seqlens, max_seqlen, sink,
                               window)
