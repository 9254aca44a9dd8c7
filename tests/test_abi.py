"""C-ABI checks that need no GPU: the library loads, exports every function
include/nsa_sel.h declares, and refuses bad arguments with the documented
status before making any HIP call (fake non-null pointers are never
dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_nsa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa_sel.h")

FAKE = 0x10000  # 64 KiB-aligned, never dereferenced


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (nsa_\w+)", out))
    assert set(names) <= exported


def test_problem_struct_matches_header():
    text = open(HEADER).read()
    body = text[text.index("typedef struct nsa_sel_problem"):]
    body = body[:body.index("} nsa_sel_problem;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for ty, names in re.findall(r"(int32_t|int64_t|float)\s+([^;]+);", body):
        for n in names.split(","):
            m = re.match(r"\s*(\w+)(?:\[(\d+)\])?", n)
            fields.append((m.group(1), ty, int(m.group(2) or 1)))
    assert [f for f, _, _ in fields] == [f for f, _ in _lib.Problem._fields_]
    size = {"int32_t": 4, "float": 4, "int64_t": 8}
    off = 0
    for (name, ty, n), (_, ct) in zip(fields, _lib.Problem._fields_):
        off = -(-off // size[ty]) * size[ty]
        assert getattr(_lib.Problem, name).offset == off, name
        assert ctypes.sizeof(ct) == size[ty] * n, name
        off += size[ty] * n
    assert ctypes.sizeof(_lib.Problem) == -(-off // 8) * 8


def _prob(**kw):
    p = _lib.Problem()
    base = dict(layout=0, B=1, T=256, Hq=2, Hkv=1, D=32, S=4, block_size=16, n_seqs=0,
                max_seqlen=0, dtype=0, scale=32 ** -0.5)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def _fwd(p, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cu=None, o=FAKE, lse=FAKE):
    return _lib.load().nsa_sel_fwd(p, q, k, v, idx, cu, o, lse, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hq=3, Hkv=2), _lib.NSA_ERR_INVALID_ARG, "multiple"),
    (dict(dtype=7), _lib.NSA_ERR_INVALID_ARG, "dtype"),
    (dict(layout=5), _lib.NSA_ERR_INVALID_ARG, "layout"),
    (dict(S=0), _lib.NSA_ERR_INVALID_ARG, "S="),
    (dict(block_size=0), _lib.NSA_ERR_INVALID_ARG, "block_size"),
    (dict(T=-1), _lib.NSA_ERR_INVALID_ARG, "T="),
    (dict(scale=float("nan")), _lib.NSA_ERR_INVALID_ARG, "scale"),
    (dict(sched_policy=2), _lib.NSA_ERR_INVALID_ARG, "sched_policy"),
    (dict(sched_policy=-1), _lib.NSA_ERR_INVALID_ARG, "sched_policy"),
    (dict(dtype=1, D=48), _lib.NSA_ERR_UNSUPPORTED, "D in"),
    (dict(dtype=1, D=64, block_size=8), _lib.NSA_ERR_UNSUPPORTED, "block_size in"),
    (dict(D=24), _lib.NSA_ERR_UNSUPPORTED, "D in"),
    (dict(T=1 << 20, block_size=16), _lib.NSA_ERR_UNSUPPORTED, "8192"),
    (dict(S=5000), _lib.NSA_ERR_UNSUPPORTED, "slots"),
    (dict(dtype=1, D=128, block_size=64, T=64 * 7000), _lib.NSA_ERR_UNSUPPORTED, "LDS"),
    (dict(B=9000, Hkv=1, Hq=1), _lib.NSA_ERR_UNSUPPORTED, "exceeds 8192"),
    (dict(layout=1, B=2), _lib.NSA_ERR_INVALID_ARG, "B == 1"),
    (dict(layout=1, n_seqs=2, max_seqlen=300), _lib.NSA_ERR_INVALID_ARG, "max_seqlen"),
])
def test_bad_problem_rejected_before_any_hip_call(kw, status, word):
    st = _fwd(_prob(**kw), cu=FAKE if kw.get("layout") == 1 else None)
    assert st == status
    assert word in _lib.last_error()


def test_null_and_misaligned_pointers_rejected():
    assert _fwd(_prob(), q=None) == _lib.NSA_ERR_INVALID_ARG
    assert "q is NULL" in _lib.last_error()
    assert _fwd(_prob(dtype=1, D=64, block_size=32), k=FAKE + 8) == _lib.NSA_ERR_INVALID_ARG
    assert "k is not 16-byte aligned" in _lib.last_error()
    assert _fwd(_prob(), cu=FAKE) == _lib.NSA_ERR_INVALID_ARG
    assert "dense" in _lib.last_error()
    assert _fwd(_prob(layout=1, n_seqs=2, max_seqlen=200)) == _lib.NSA_ERR_INVALID_ARG
    assert "cu_seqlens is NULL" in _lib.last_error()


def test_workspace_checked_before_launch():
    lib = _lib.load()
    p = _prob(dtype=1, D=64, block_size=32, Hq=6, Hkv=2, T=1024, B=2, S=8)
    need = lib.nsa_sel_bwd_workspace_bytes(p)
    assert need > 0 and _lib.last_error() == ""
    st = lib.nsa_sel_bwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                         FAKE, need - 1, None)
    assert st == _lib.NSA_ERR_WORKSPACE
    st = lib.nsa_sel_bwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                         FAKE + 64, need, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "256-byte" in _lib.last_error()
    assert lib.nsa_sel_bwd_workspace_bytes(_prob(Hq=3, Hkv=2)) == 0
    assert "multiple" in _lib.last_error()


def test_sink_and_check_calls_validate_before_any_hip_call():
    """The sink forward, dsink and block_idx check reject bad arguments on the
    host (no GPU here: a launch would fail differently)."""
    lib = _lib.load()
    p = _prob(dtype=1, D=64, block_size=32, Hq=6, Hkv=2, T=1024, B=2, S=8)
    st = lib.nsa_sel_fwd_sink(p, FAKE, FAKE, FAKE, FAKE, None, FAKE + 2, FAKE, FAKE, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "sink is not 4-byte aligned" in _lib.last_error()
    need = lib.nsa_sel_bwd_workspace_bytes(p)
    st = lib.nsa_sel_bwd_dsink(p, FAKE, None, None, FAKE, FAKE, need, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "sink is NULL" in _lib.last_error()
    st = lib.nsa_sel_bwd_dsink(p, FAKE, FAKE, None, FAKE, FAKE, need - 1, None)
    assert st == _lib.NSA_ERR_WORKSPACE
    st = lib.nsa_sel_bwd_dsink(p, FAKE, FAKE, None, None, FAKE, need, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "dsink is NULL" in _lib.last_error()
    st = lib.nsa_sel_check_block_idx(p, FAKE, None, FAKE + 4, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "counts is not 8-byte aligned" in _lib.last_error()
    st = lib.nsa_sel_check_block_idx(_prob(Hq=3, Hkv=2), FAKE, None, FAKE, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "multiple" in _lib.last_error()


def test_status_strings():
    for s in range(5):
        assert _lib.status_string(s)
    assert _lib.status_string(99) == "unknown status"


def test_empty_problem_is_a_no_op():
    # T = 0: nothing to read or write, so NULL buffers are fine and no HIP call happens.
    assert _fwd(_prob(T=0), q=None, k=None, v=None, idx=None, o=None, lse=None) == _lib.NSA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def _strided(p, **strides):
    """Mark p strided with contiguous dense strides, then override some."""
    H = {"q": p.Hq, "o": p.Hq, "do": p.Hq, "dq": p.Hq, "k": p.Hkv, "v": p.Hkv, "dk": p.Hkv,
         "dv": p.Hkv}
    p.strided = 1
    for name, h in H.items():
        arr = getattr(p, "stride_" + name)
        arr[0], arr[1], arr[2] = h * p.T * p.D, p.T * p.D, p.D
    for name, st in strides.items():
        arr = getattr(p, "stride_" + name)
        arr[0], arr[1], arr[2] = st
    return p


def _bwd_small_ws(p):
    """nsa_sel_bwd with every tensor given and a workspace one byte short:
    NSA_ERR_WORKSPACE means every tensor check passed (no HIP call made)."""
    lib = _lib.load()
    need = lib.nsa_sel_bwd_workspace_bytes(p)
    assert need > 0, _lib.last_error()
    return lib.nsa_sel_bwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                           FAKE, need - 1, None)


def test_declared_strides_accepted():
    """BTHD buffers viewed as BHTD, a KV head repeated over the batch (batch
    stride 0 on an input), and gradients written into a wider buffer."""
    B, Hq, Hkv, T, D = 2, 4, 2, 96, 64
    p = _prob(dtype=1, B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, S=4, block_size=32)
    _strided(p, q=(T * Hq * D, D, Hq * D), o=(T * Hq * D, D, Hq * D),
             k=(0, T * D, D), v=(T * Hkv * D, D, Hkv * D),
             dq=(T * Hq * 2 * D, 2 * D, Hq * 2 * D), dk=(Hkv * T * D, T * D, D))
    assert _bwd_small_ws(p) == _lib.NSA_ERR_WORKSPACE, _lib.last_error()
    p2 = _prob(dtype=1, layout=1, B=1, Hq=Hq, Hkv=Hkv, T=T, D=D, S=4, block_size=32, n_seqs=2,
               max_seqlen=64)
    _strided(p2, q=(12345, D, Hq * D), dq=(0, 2 * D, Hq * 2 * D))   # packed: [0] unread
    lib = _lib.load()
    need = lib.nsa_sel_bwd_workspace_bytes(p2)
    st = lib.nsa_sel_bwd(p2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, need - 1, None)
    assert st == _lib.NSA_ERR_WORKSPACE, _lib.last_error()


@pytest.mark.parametrize("which,st,status,word", [
    ("q", (-8, 64, 64 * 4), _lib.NSA_ERR_INVALID_ARG, ">= 0"),
    ("k", (96 * 64, 96 * 64 + 4, 64), _lib.NSA_ERR_INVALID_ARG, "multiples of 8"),
    ("v", (0, 64, 1 << 23), _lib.NSA_ERR_UNSUPPORTED, "token stride"),
    ("dO", (0, 1 << 30, 64), _lib.NSA_ERR_UNSUPPORTED, "2^31"),
    ("o", (4 * 96 * 64, 0, 64), _lib.NSA_ERR_INVALID_ARG, "overlapping"),   # heads alias
    ("dq", (4 * 96 * 64, 96 * 64, 32), _lib.NSA_ERR_INVALID_ARG, "overlapping"),  # rows overlap
    ("dk", (0, 96 * 64, 64), _lib.NSA_ERR_INVALID_ARG, "overlapping"),      # batch entries alias
    ("dv", (2 * 96 * 64, 2 * 96 * 64, 64), _lib.NSA_ERR_INVALID_ARG, "overlapping"),  # head 1 = entry 1
])
def test_bad_strides_rejected_before_any_hip_call(which, st, status, word):
    p = _prob(dtype=1, B=2, Hq=4, Hkv=2, T=96, D=64, S=4, block_size=32)
    _strided(p, **{which.lower() if which != "dO" else "do": st})
    assert _bwd_small_ws(p) == status
    assert word in _lib.last_error() and which in _lib.last_error()


def test_inputs_may_overlap_outputs_may_not():
    """A zero head stride is a valid input (one row shared by every head) but
    an invalid output."""
    p = _prob(dtype=1, B=1, Hq=4, Hkv=1, T=64, D=64, S=2, block_size=32)
    _strided(p, q=(0, 0, 64))
    assert _bwd_small_ws(p) == _lib.NSA_ERR_WORKSPACE, _lib.last_error()
    _strided(p, dq=(0, 0, 64))
    assert _bwd_small_ws(p) == _lib.NSA_ERR_INVALID_ARG and "overlapping" in _lib.last_error()


def test_list_entry_bound():
    """max length * min(S, NBmax) inverted-list entries per (batch, KV head)
    must stay below 2^31 (32-bit list offsets): the last accepted length and
    the first refused one."""
    lib = _lib.load()
    ok = _prob(dtype=0, D=16, T=(1 << 19) - 1, block_size=64, S=4096, Hq=1, Hkv=1)
    assert lib.nsa_sel_bwd_workspace_bytes(ok) > 0, _lib.last_error()
    bad = _prob(dtype=0, D=16, T=1 << 19, block_size=64, S=4096, Hq=1, Hkv=1)
    assert lib.nsa_sel_bwd_workspace_bytes(bad) == 0
    assert "list entries" in _lib.last_error()


def test_noalloc_backward_checks_before_any_hip_call():
    """nsa_sel_bwd_noalloc refuses bad tensors and problems whose workspace
    exceeds its built-in 64 MiB scratch on the host, before any HIP call."""
    lib = _lib.load()
    ok = _prob(dtype=1, D=64, block_size=32, Hq=6, Hkv=2, T=1024, B=2, S=8)
    st = lib.nsa_sel_bwd_noalloc(ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                                 FAKE, None)
    assert st == _lib.NSA_ERR_INVALID_ARG and "dq is NULL" in _lib.last_error()
    big = _prob(dtype=1, D=128, block_size=64, Hq=32, Hkv=2, T=8192, B=1, S=16)
    assert lib.nsa_sel_bwd_workspace_bytes(big) > 64 << 20
    st = lib.nsa_sel_bwd_noalloc(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                 FAKE, None)
    assert st == _lib.NSA_ERR_WORKSPACE and str(64 << 20) in _lib.last_error()


def test_ds_handoff_query():
    """nsa_sel_bwd_ds_handoff states when dK/dV hands dS over to dQ: bf16,
    G = 4, 8 or a multiple of 16, block_size >= 32, S <= 64, no window,
    lists that cannot cover whole causal prefixes (S * block_size < length)
    and a per-(batch, KV head) dS region below 2^31 bytes."""
    lib = _lib.load()
    q = lambda **kw: lib.nsa_sel_bwd_ds_handoff(_prob(**kw))
    cfg2 = dict(dtype=1, D=128, block_size=64, Hq=32, Hkv=2, T=8192, B=1, S=16)
    assert q(**cfg2) == 1, _lib.last_error()
    assert q(**{**cfg2, "Hq": 64}) == 1                      # G = 32
    assert q(**{**cfg2, "S": 128}) == 0                      # whole prefixes possible
    assert q(**{**cfg2, "dtype": 0, "D": 64}) == 0           # f32 path
    assert q(**{**cfg2, "Hq": 6}) == 0                       # G = 3
    assert q(**{**cfg2, "Hq": 8}) == 1                       # G = 4
    assert q(**{**cfg2, "Hq": 16}) == 1                      # G = 8
    assert q(**{**cfg2, "Hq": 4}) == 0                       # G = 2
    assert q(**{**cfg2, "Hq": 24}) == 0                      # G = 12
    # dS region of one (batch, KV head): T * S * block_size * G * 2 bytes
    assert q(**{**cfg2, "T": (1 << 16) - 64}) == 1
    assert q(**{**cfg2, "T": 1 << 16}) == 0
    assert q(**{**cfg2, "block_size": 16, "S": 64}) == 0     # 16-key blocks
    assert q(**{**cfg2, "S": 65}) == 0                       # more than 64 slots
    assert q(**{**cfg2, "window": 512}) == 0
    assert q(**{**cfg2, "Hq": 33}) == -1 and _lib.last_error()  # invalid problem


def test_build_git_reported():
    s = _lib.load().nsa_build_git().decode()
    assert s == "unknown" or re.fullmatch(r"[0-9a-f]{4,40}(\+dirty)?", s), s


def test_key_length_checks():
    """Tk (keys per (batch entry, KV head)) must be 0 (= T) or >= T for dense
    problems and 0 or T for packed ones; k-like tensors span Tk rows."""
    lib = _lib.load()
    ok = _prob(dtype=1, D=64, block_size=32, Hq=4, Hkv=2, T=100, S=4)
    ok.Tk = 300
    assert lib.nsa_sel_bwd_workspace_bytes(ok) > 0, _lib.last_error()
    bad = _prob(dtype=1, D=64, block_size=32, Hq=4, Hkv=2, T=100, S=4)
    bad.Tk = 99
    assert _fwd(bad) == _lib.NSA_ERR_INVALID_ARG and "Tk" in _lib.last_error()
    neg = _prob(dtype=1, D=64, block_size=32, Hq=4, Hkv=2, T=100, S=4)
    neg.Tk = -1
    assert _fwd(neg) == _lib.NSA_ERR_INVALID_ARG
    packed = _prob(layout=1, dtype=1, D=64, block_size=32, Hq=4, Hkv=2, T=100, S=4, n_seqs=1,
                   max_seqlen=100)
    packed.Tk = 200
    assert _fwd(packed, cu=FAKE) == _lib.NSA_ERR_INVALID_ARG and "Tk" in _lib.last_error()
    packed.Tk = 100
    assert lib.nsa_sel_bwd_workspace_bytes(packed) > 0, _lib.last_error()
    # key blocks: 8192 blocks of keys at most, whatever the query count
    many = _prob(dtype=1, D=64, block_size=32, Hq=4, Hkv=2, T=10, S=4)
    many.Tk = 32 * 8192 + 1
    assert lib.nsa_sel_bwd_workspace_bytes(many) == 0 and "8192" in _lib.last_error()
