"""The host-side table checks (kvfp4_check_*_tables): every value a call
would read out of range is reported with its element and value, valid
workload tables pass, and bad arguments are refused. The tests call the C
functions directly, so the same tests also run against a sanitizer build
of the checks (tests/test_sanitizers.py sets KVFP4_TABLE_CHECKS_LIB)."""
import ctypes as C
import os

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EVALUE = 0, 1, 6
(T_OK, T_START, T_ORDER, T_PAGE, T_BATCH, T_POS, T_LAST, T_DUP, T_LEN, T_RES, T_OUT, T_STEP) = range(12)


class Report(C.Structure):
    _fields_ = [("problem", C.c_int32), ("index", C.c_int64), ("value", C.c_int64)]


@pytest.fixture(scope="module")
def lib():
    path = os.environ.get("KVFP4_TABLE_CHECKS_LIB")
    if path is None:
        from kv_cache_quantization_paged_amd import _binding
        path = _binding.LIB_PATH
    lib = C.CDLL(path)
    P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.kvfp4_check_append_tables.restype = i32
    lib.kvfp4_check_append_tables.argtypes = [P, P, i64, P, P, P, i32, i32, i32, P, C.POINTER(Report)]
    lib.kvfp4_check_paged_tables.restype = i32
    lib.kvfp4_check_paged_tables.argtypes = [P, i32, i64, i32, P, i32, i32, i32, i32, C.POINTER(Report)]
    lib.kvfp4_check_materialize_tables.restype = i32
    lib.kvfp4_check_materialize_tables.argtypes = [P, i32, i64, i64, i32, P, P, i32, i32, i32, i32, i64,
                                                   C.POINTER(Report)]
    lib.kvfp4_check_step_rows.restype = i32
    lib.kvfp4_check_step_rows.argtypes = [P, P, i64, P, i32, P, C.POINTER(Report)]
    lib.kvfp4_table_problem_string.restype = C.c_char_p
    lib.kvfp4_table_problem_string.argtypes = [i32]
    return lib


def ptr(a):
    return C.c_void_p(a.ctypes.data) if a is not None and a.size else None


def append(lib, bi, pos, ind, indptr, last, ps, P, dup=True):
    bi, pos = np.ascontiguousarray(bi, np.int32), np.ascontiguousarray(pos, np.int32)
    ind, indptr, last = (np.ascontiguousarray(x, np.int32) for x in (ind, indptr, last))
    scratch = np.zeros(len(bi), np.int64) if dup else None
    r = Report()
    st = lib.kvfp4_check_append_tables(ptr(bi), ptr(pos), len(bi), ptr(ind), ptr(indptr), ptr(last), len(indptr) - 1,
                                       ps, P, ptr(scratch), C.byref(r))
    return st, (r.problem, r.index, r.value)


def paged(lib, bt, lens, ps, P, T=2 ** 31 - 1):
    bt = np.ascontiguousarray(bt)
    lens = np.ascontiguousarray(lens, np.int32)
    r = Report()
    st = lib.kvfp4_check_paged_tables(ptr(bt), 1 if bt.dtype == np.int64 else 0, bt.shape[1], bt.shape[1], ptr(lens),
                                      len(lens), ps, P, T, C.byref(r))
    return st, (r.problem, r.index, r.value)


def mat(lib, bt, lens, indptr, ps, P, maxp, n_out, shared):
    bt = np.ascontiguousarray(bt, np.int32)
    lens, indptr = np.ascontiguousarray(lens, np.int32), np.ascontiguousarray(indptr, np.int32)
    cols = bt.shape[-1]
    row, kvs = (cols, 0) if shared else (2 * cols, cols)
    r = Report()
    st = lib.kvfp4_check_materialize_tables(ptr(bt), int(shared), row, kvs, cols, ptr(lens), ptr(indptr), len(lens),
                                            ps, P, maxp, n_out, C.byref(r))
    return st, (r.problem, r.index, r.value)


def decode_tables():
    rng = np.random.default_rng(1002)
    return W.decode_append_tables(rng, 64, 4096, 20000, 16)


def test_raw_workload_tables_pass(lib):
    old, new_len, ind, indptr, last, bt = decode_tables()
    assert append(lib, np.arange(64), old, ind, indptr, last, 16, 20000)[0] == OK
    # every history row of every request, in any order
    hb, hp = W.rows_for_positions(np.zeros(64, np.int64), new_len)
    order = np.random.default_rng(0).permutation(len(hb))
    assert append(lib, hb[order], hp[order], ind, indptr, last, 16, 20000)[0] == OK
    assert paged(lib, bt, new_len, 16, 20000, int(new_len.max()))[0] == OK
    assert paged(lib, bt, new_len, 16, 20000)[0] == OK                          # attention: no clamp
    assert paged(lib, bt.astype(np.int64), new_len, 16, 20000)[0] == OK
    lens, P, maxp, mbt, mptr = W.materialize_tables(np.random.default_rng(1004))
    assert mat(lib, mbt, lens, mptr, 16, P, maxp, P + 1, False)[0] == OK
    lens, P, maxp, mbt, mptr = W.materialize_tables(np.random.default_rng(7), shared=True, compact=False)
    assert mat(lib, mbt, lens, mptr, 16, P, maxp, int(mptr[-1]) + 1, True)[0] == OK


def test_raw_append_problems(lib):
    old, new_len, ind, indptr, last, bt = decode_tables()
    bi = np.arange(64)
    args = lambda **kw: {**dict(bi=bi, pos=old, ind=ind, indptr=indptr, last=last, ps=16, P=20000), **kw}  # noqa
    run = lambda **kw: append(lib, **args(**kw))                                                       # noqa
    p = indptr.copy(); p[0] = 1
    assert run(indptr=p) == (EVALUE, (T_START, 0, 1))
    p = indptr.copy(); p[10] = p[9] - 1
    assert run(indptr=p) == (EVALUE, (T_ORDER, 10, p[10]))
    i = ind.copy(); i[77] = 20000
    assert run(ind=i) == (EVALUE, (T_PAGE, 77, 20000))
    i = ind.copy(); i[5] = -3
    assert run(ind=i) == (EVALUE, (T_PAGE, 5, -3))
    l2 = last.copy(); l2[3] = 0
    assert run(last=l2) == (EVALUE, (T_LAST, 3, 0))
    l2 = last.copy(); l2[3] = 17
    assert run(last=l2) == (EVALUE, (T_LAST, 3, 17))
    b2 = bi.copy(); b2[9] = 64
    assert run(bi=b2) == (EVALUE, (T_BATCH, 9, 64))
    b2 = bi.copy(); b2[9] = -1
    assert run(bi=b2) == (EVALUE, (T_BATCH, 9, -1))
    # the last valid position of request 20 passes, the next one does not
    space = (indptr[21] - indptr[20] - 1) * 16 + last[20]
    q = old.copy(); q[20] = space - 1
    assert run(pos=q)[0] == OK
    q[20] = space
    assert run(pos=q) == (EVALUE, (T_POS, 20, space))
    q[20] = -1
    assert run(pos=q) == (EVALUE, (T_POS, 20, -1))
    # two rows of request 4 at the same position race
    b2, q = np.concatenate([bi, [4]]), np.concatenate([old, [old[4]]])
    assert run(bi=b2, pos=q) == (EVALUE, (T_DUP, 4, old[4]))
    assert append(lib, b2, q, ind, indptr, last, 16, 20000, dup=False)[0] == OK   # that check skipped


def test_raw_paged_problems(lib):
    old, new_len, ind, indptr, last, bt = decode_tables()
    T = int(new_len.max())
    l2 = new_len.copy(); l2[7] = -1
    assert paged(lib, bt, l2, 16, 20000, T) == (EVALUE, (T_LEN, 7, -1))
    l2 = new_len.copy(); l2[7] = bt.shape[1] * 16 + 1          # needs one more column than the table has
    assert paged(lib, bt, l2, 16, 20000) == (EVALUE, (T_LEN, 7, l2[7]))
    assert paged(lib, bt, l2, 16, 20000, T)[0] == OK           # ... but dequant clamps to max_seq_len
    b2 = bt.copy()
    need = (new_len[30] + 15) // 16
    b2[30, need - 1] = 20000
    assert paged(lib, b2, new_len, 16, 20000, T) == (EVALUE, (T_PAGE, 30 * bt.shape[1] + need - 1, 20000))
    b2 = bt.copy()
    b2[30, need] = -5                                           # a column the request does not use
    assert paged(lib, b2, new_len, 16, 20000, T)[0] == OK
    assert paged(lib, b2.astype(np.int64) + (1 << 40), new_len, 16, 20000, T)[1][0] == T_PAGE


@pytest.mark.parametrize("shared", [False, True])
def test_raw_materialize_problems(lib, shared):
    lens, P, maxp, bt, indptr = W.materialize_tables(np.random.default_rng(1004), shared=shared)
    n_out = P + 1
    run = lambda bt=bt, lens=lens, indptr=indptr, n_out=n_out: mat(lib, bt, lens, indptr, 16, P, maxp, n_out, shared)  # noqa
    assert run()[0] == OK
    assert run(n_out=P) == (EVALUE, (T_OUT, 32, P))
    p = indptr.copy(); p[0] = 2
    assert run(indptr=p)[1][0] == T_START
    p = indptr.copy(); p[5] = p[4] - 1
    assert run(indptr=p) == (EVALUE, (T_ORDER, 5, p[5]))
    need = (lens + 15) // 16
    p = indptr.copy(); p[6:] -= 1                               # request 5 reserves one page too few
    assert run(indptr=p) == (EVALUE, (T_RES, 5, need[5] - 1))
    l2 = lens.copy(); l2[11] = maxp * 16 + 1
    assert run(lens=l2)[1][:2] == (T_LEN, 11)
    l2 = lens.copy(); l2[11] = -2
    assert run(lens=l2) == (EVALUE, (T_LEN, 11, -2))
    b2 = bt.copy()
    if shared:
        b2[3, need[3] - 1] = P
        assert run(bt=b2) == (EVALUE, (T_PAGE, 3 * bt.shape[1] + need[3] - 1, P))
    else:
        b2[3, 1, need[3] - 1] = P                               # a V page
        assert run(bt=b2) == (EVALUE, (T_PAGE, 3 * 2 * bt.shape[2] + bt.shape[2] + need[3] - 1, P))


def test_raw_bad_arguments(lib):
    r = Report()
    z = np.zeros(4, np.int32)
    assert lib.kvfp4_check_append_tables(None, None, 0, None, ptr(z), ptr(z), 1, 16, 4, None, None) == EINVAL
    assert lib.kvfp4_check_append_tables(None, None, 0, None, ptr(z), ptr(z), 1, 0, 4, None, C.byref(r)) == EINVAL
    assert lib.kvfp4_check_append_tables(None, None, 2, None, ptr(z), ptr(z), 1, 16, 4, None, C.byref(r)) == EINVAL
    assert lib.kvfp4_check_paged_tables(ptr(z), 7, 2, 2, ptr(z), 2, 16, 4, 10, C.byref(r)) == EINVAL
    assert lib.kvfp4_check_paged_tables(ptr(z), 0, 1, 2, ptr(z), 2, 16, 4, 10, C.byref(r)) == EINVAL
    assert lib.kvfp4_check_materialize_tables(ptr(z), 1, 2, 0, 2, ptr(z), ptr(z), 2, 16, 4, 3, 10,
                                              C.byref(r)) == EINVAL          # fewer columns than max_pages_per_seq
    assert lib.kvfp4_check_materialize_tables(ptr(z), 1, 2, 0, 2, ptr(z), ptr(z), 2, 16, 4, 2, 0,
                                              C.byref(r)) == EINVAL          # no output page
    for p in range(11):
        assert lib.kvfp4_table_problem_string(p) != b"unknown problem"
    assert lib.kvfp4_table_problem_string(99) == b"unknown problem"


def test_python_wrappers_raise_with_the_location():
    import kv_cache_quantization_paged_amd as K
    old, new_len, ind, indptr, last, bt = decode_tables()
    K.check_append_tables(np.arange(64), old, ind, indptr, last, 16, 20000)
    K.check_paged_tables(bt, new_len, 16, 20000, int(new_len.max()))
    bad = ind.copy()
    bad[100] = 20001
    with pytest.raises(K.TableError) as e:
        K.check_append_tables(np.arange(64), old, bad, indptr, last, 16, 20000)
    assert (e.value.problem, e.value.index, e.value.value) == (T_PAGE, 100, 20001)
    lens, P, maxp, mbt, mptr = W.materialize_tables(np.random.default_rng(1004))
    K.check_materialize_tables(mbt, lens, mptr, 16, P, maxp, P + 1, uses_shared_paged_kv_idx=False)
    with pytest.raises(K.TableError):
        K.check_materialize_tables(mbt, lens, mptr, 16, P, maxp, P, uses_shared_paged_kv_idx=False)


def step_rows(lib, bi, pos, lens, dup=True, nnz=None):
    bi, pos, lens = (np.ascontiguousarray(x, np.int32) for x in (bi, pos, lens))
    scratch = np.zeros(len(lens), np.int64) if dup else None
    r = Report()
    st = lib.kvfp4_check_step_rows(ptr(bi), ptr(pos), len(bi) if nnz is None else nnz, ptr(lens), len(lens),
                                   ptr(scratch), C.byref(r))
    return st, (r.problem, r.index, r.value)


def test_step_rows(lib):
    """the one-launch decode step's rows: one per request, at its newest
    token; the decode workload's step passes"""
    old, new_len, *_ = decode_tables()
    rng = np.random.default_rng(5)
    order = rng.permutation(64)
    assert step_rows(lib, order, old[order], new_len)[0] == OK
    assert step_rows(lib, np.arange(64), old, new_len)[0] == OK
    pos = old.copy()
    pos[9] -= 1                                            # not the newest token
    assert step_rows(lib, np.arange(64), pos, new_len) == (EVALUE, (T_STEP, 9, int(pos[9])))
    bi = np.arange(64)
    bi[3] = 64                                             # request out of range
    assert step_rows(lib, bi, old, new_len)[1][:2] == (T_BATCH, 3)
    bi = np.arange(64)
    bi[40] = 7                                             # request 7 twice, request 40 missing
    pos = old[bi]
    assert step_rows(lib, bi, pos, new_len) == (EVALUE, (T_DUP, 40, 7))
    assert step_rows(lib, bi, pos, new_len, dup=False)[0] == OK      # without scratch: not checked
    assert step_rows(lib, np.arange(64), old, new_len, nnz=63)[0] == EINVAL   # rows != requests
    assert step_rows(lib, np.zeros(0), np.zeros(0), np.zeros(0))[0] == OK
    assert lib.kvfp4_table_problem_string(T_STEP).decode() != "unknown problem"
