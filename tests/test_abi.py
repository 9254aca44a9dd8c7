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
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in _lib.Problem._fields_]
    assert ctypes.sizeof(_lib.Problem) == 4 * len(fields)


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
    (dict(dtype=1, D=48), _lib.NSA_ERR_UNSUPPORTED, "D in"),
    (dict(dtype=1, D=64, block_size=16), _lib.NSA_ERR_UNSUPPORTED, "block_size in"),
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
