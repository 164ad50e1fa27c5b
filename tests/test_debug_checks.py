"""The SA_DEBUG precondition checks, driven through the C ABI on the host.

Both libraries export sa_debug_check_host, which runs the same rules as the
SA_DEBUG build's device-side check kernels on host arrays; here every rule is
given a bad value and must name it.  No GPU is needed."""
import ctypes

import numpy as np
import pytest

from sparse_attention_relu_amd import _lib
from tests.test_abi import declared_functions

MAX_SEQ_LEN = 3728270      # position * 1152 + 1151 < 2^32


@pytest.fixture(scope="module", params=["release", "debug"])
def L(request):
    return _lib.lib() if request.param == "release" else _lib.debug_lib()


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def batch(n_q=3):
    seq_start = np.array([0, 100, 150], dtype=np.int64)
    seq_len = np.array([100, 50, 70], dtype=np.int32)
    q_seq = np.array([0, 1, 2], dtype=np.int32)[:n_q]
    q_pos = np.array([99, 10, 69], dtype=np.int32)[:n_q]
    return dict(seq_start=seq_start, seq_len=seq_len, q_seq=q_seq, q_pos=q_pos, ld=100)


def run(L, b, idx=None, k=0, n_seq=None):
    n_seq = len(b["seq_start"]) if n_seq is None else n_seq
    rc = L.sa_debug_check_host(_p(b["seq_start"]), _p(b["seq_len"]), _p(b["q_seq"]), _p(b["q_pos"]),
                               len(b["q_seq"]), n_seq, b["ld"], _p(idx), k)
    return rc, L.sa_last_error_message().decode()


def test_debug_library_exports_everything():
    D = _lib.debug_lib()
    for n in declared_functions():
        assert hasattr(D, n), n
    assert D.sa_debug_enabled() == 1
    assert _lib.lib().sa_debug_enabled() == 0


def test_release_debug_check_is_unsupported():
    R = _lib.lib()
    assert R.sa_debug_check(None) == -2
    assert b"SA_DEBUG" in R.sa_last_error_message()


def test_valid_batch_passes(L):
    b = batch()
    idx = np.array([[0, 99, -1], [10, 3, -1], [-1, -1, -1]], dtype=np.int32)
    assert run(L, b, idx, 3) == (0, run(L, b, idx, 3)[1])
    assert run(L, b)[0] == 0


@pytest.mark.parametrize("field,i,value,text", [
    ("q_seq", 1, 3, "q_seq outside"),
    ("q_seq", 0, -1, "q_seq outside"),
    ("q_pos", 2, -4, "q_pos negative"),
    ("q_pos", 1, 50, "seq_len"),           # sequence 1 holds 50 keys: positions 0..49
    ("q_pos", 2, 69, None),                # the last key of sequence 2 is valid ...
    ("seq_len", 2, MAX_SEQ_LEN + 1, "SA_MAX_SEQ_LEN"),
    ("seq_len", 1, -1, "SA_MAX_SEQ_LEN"),
    ("seq_start", 2, -5, "seq_start negative"),
])
def test_each_batch_rule(L, field, i, value, text):
    b = batch()
    b[field] = b[field].copy()
    b[field][i] = value
    rc, msg = run(L, b)
    if text is None:
        assert rc == 0, msg
        return
    assert rc == -5, (field, value, msg)
    assert text in msg and f"value {value}" in msg, msg


def test_q_pos_beyond_ld(L):
    b = batch()
    b["ld"] = 60                            # query 0 sits at 99
    rc, msg = run(L, b)
    assert rc == -5 and "below ld" in msg and "item 0" in msg


@pytest.mark.parametrize("t,j,value", [(0, 1, 100), (1, 0, 11), (2, 2, -2), (0, 2, MAX_SEQ_LEN)])
def test_each_index_rule(L, t, j, value):
    b = batch()
    idx = np.full((3, 3), -1, dtype=np.int32)
    idx[t, j] = value
    rc, msg = run(L, b, idx, 3)
    assert rc == -5 and "idx entry" in msg and f"item {t}, slot {j}, value {value}" in msg, msg


def test_first_violation_reported_and_all_counted(L):
    b = batch()
    b["q_pos"] = np.array([-1, 60, 70], dtype=np.int32)   # three violations; query 0 is first
    rc, msg = run(L, b)
    assert rc == -5 and "q_pos negative" in msg and "item 0" in msg and "3 violation(s)" in msg, msg


def test_null_arrays_rejected(L):
    assert L.sa_debug_check_host(None, None, None, None, 2, 1, 10, None, 0) == -1
    assert L.sa_debug_check_host(None, None, None, None, 0, 0, 10, None, 0) == 0
    b = batch()
    assert L.sa_debug_check_host(_p(b["seq_start"]), _p(b["seq_len"]), _p(b["q_seq"]), _p(b["q_pos"]), -1, 3, 10,
                                 None, 0) == -1
