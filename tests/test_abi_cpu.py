"""C-ABI checks that need no GPU: the library loads and exports every function
include/wfst.h declares, and graph validation (pure host code, run before any
device call) rejects corrupt graphs with WFST_ECORRUPT and a message."""

import ctypes
import os
import re

import numpy as np
import pytest

import wfst_beam_search_amd as wb
from cases import graph_from_states

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WFST_ECORRUPT = -2
WFST_EINVAL = -1


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "wfst.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wfst_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wb.library_path()):
        pytest.fail("libwfst_mi355x.so is not built (run __graft_entry__.build())")
    return wb.load_library()


def test_header_and_library_agree(lib):
    declared = _declared_functions()
    assert declared == sorted(wb.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


_CTYPES = {"float": ctypes.c_float, "int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64}


@pytest.mark.parametrize("name,cls", [("wfst_decoder_config", wb._Config), ("wfst_graph_desc", wb._GraphDesc)])
def test_binding_structs_match_header(name, cls):
    """The binding's ctypes structs list the header's fields in the same order
    with the same types, so the C library reads what Python writes."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "wfst.h")).read(), flags=re.S)
    body = re.search(r"typedef struct " + name + r"\s*\{(.*?)\}\s*" + name + ";", src, flags=re.S).group(1)
    fields = re.findall(r"([A-Za-z_][A-Za-z0-9_ ]*?[\s*]+)([a-z_]+)\s*;", body)
    assert [f for _, f in fields] == [f for f, _ in cls._fields_]
    for (ctype, fname), (pname, ptype) in zip(fields, cls._fields_):
        ctype = ctype.strip()
        if "*" in ctype:
            assert ptype is ctypes.c_void_p, fname
        else:
            assert _CTYPES[ctype] is ptype, fname


def _good_spec():
    return {"start": 0, "vocab": 3, "epsilon_id": -1,
            "states": [[[1, 1, 5, -0.5], [0, 2, 0, -1.0], [2, -1, 0, 0.0]],
                       [[1, 0, 0, -0.25], [2, -1, 0, 0.0]], []]}


def _upload_rc(g, lib):
    arrays = [np.ascontiguousarray(x) for x in (g.row_splits, g.dest, g.ilabel, g.olabel, g.weight)]
    desc = wb._GraphDesc(int(g.num_states), int(g.dest.shape[0]), int(g.start), int(g.vocab),
                         int(g.epsilon_id), *[a.ctypes.data if a.size else None for a in arrays])
    h = ctypes.c_void_p()
    rc = lib.wfst_graph_upload(ctypes.byref(desc), 0, ctypes.byref(h))
    msg = lib.wfst_last_error().decode()
    if rc == 0:
        lib.wfst_graph_release(h)
    return rc, msg


def _mutations():
    out = []

    def m(name, fn):
        g = graph_from_states(_good_spec())
        fn(g)
        out.append((name, g))

    m("rowsplits_decrease", lambda g: g.row_splits.__setitem__(1, 4))
    m("rowsplits_end", lambda g: g.row_splits.__setitem__(3, 4))
    m("dest_out_of_range", lambda g: g.dest.__setitem__(0, 7))
    m("dest_negative", lambda g: g.dest.__setitem__(0, -1))
    m("ilabel_ge_vocab", lambda g: g.ilabel.__setitem__(0, 3))
    m("ilabel_below_minus_one", lambda g: g.ilabel.__setitem__(0, -2))
    m("final_not_last", lambda g: (g.ilabel.__setitem__(0, -1), g.dest.__setitem__(0, 2),
                                    g.ilabel.__setitem__(2, 1), g.dest.__setitem__(2, 1)))
    m("final_not_to_superfinal", lambda g: g.dest.__setitem__(2, 1))
    m("emitting_into_superfinal", lambda g: g.dest.__setitem__(0, 2))
    m("nan_weight", lambda g: g.weight.__setitem__(1, np.nan))
    m("inf_weight", lambda g: g.weight.__setitem__(1, np.inf))
    m("negative_olabel", lambda g: g.olabel.__setitem__(0, -3))
    m("start_out_of_range", lambda g: setattr(g, "start", 2))
    m("vocab_too_large", lambda g: setattr(g, "vocab", 65535))
    m("vocab_zero", lambda g: setattr(g, "vocab", 0))
    m("eps_id_out_of_range", lambda g: setattr(g, "epsilon_id", 3))
    return out


@pytest.mark.parametrize("name,g", _mutations(), ids=lambda x: x if isinstance(x, str) else "")
def test_corrupt_graph_rejected(lib, name, g):
    rc, msg = _upload_rc(g, lib)
    assert rc == WFST_ECORRUPT, (name, rc, msg)
    assert "corrupt graph" in msg


def test_superfinal_with_arcs_rejected(lib):
    spec = _good_spec()
    spec["states"].append([])
    spec["states"][2] = [[1, -1, 0, 0.0]]
    rc, msg = _upload_rc(graph_from_states(spec), lib)
    assert rc == WFST_ECORRUPT


def test_epsilon_order_enforced(lib):
    spec = {"start": 0, "vocab": 3, "epsilon_id": 0,
            "states": [[[1, 1, 0, -0.5], [1, 0, 0, -0.1], [2, -1, 0, 0.0]], [[2, -1, 0, 0.0]], []]}
    rc, msg = _upload_rc(graph_from_states(spec), lib)
    assert rc == WFST_ECORRUPT and "ordered" in msg


def test_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.wfst_graph_upload(None, 0, ctypes.byref(h)) in (WFST_EINVAL,)
    assert lib.wfst_decoder_create(None, None, ctypes.byref(h)) == WFST_EINVAL
    assert lib.wfst_decode(None, None, 1, 1, 1, None, None, None, 0, None, None, 0, None, None, None) == WFST_EINVAL
    assert lib.wfst_graph_release(None) == 0
    assert lib.wfst_decoder_destroy(None) == 0


def test_graph_from_arrays_validates_before_any_device_call(lib):
    """Graph.from_arrays marshals plain arrays into the same upload call: a
    corrupt graph (an arc into a state that does not exist) fails validation,
    which runs on the host before the device is touched."""
    rs = np.array([0, 2, 3, 3], np.int32)
    dest = np.array([1, 5, 2], np.int32)
    il = np.array([0, -1, -1], np.int32)
    ol = np.zeros(3, np.int32)
    w = np.array([-0.5, 0.0, 0.0], np.float32)
    with pytest.raises(wb.WfstError) as ei:
        wb.Graph.from_arrays(rs, dest, il, ol, w, start=0, vocab=2)
    assert ei.value.code == WFST_ECORRUPT
