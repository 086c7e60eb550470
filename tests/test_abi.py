"""The C-ABI library on the CPU: it loads, exports every symbol rkv.h
declares, and its pure host logic (sizes, status strings, the ring schedule,
argument validation that happens before any device call) behaves."""
import ctypes
import os
import re

import pytest

import position_split_kv_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    L = P.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(P.EXPORTS) == names


def test_status_strings():
    for code, name in [(0, "RKV_OK"), (-1, "RKV_E_INVAL"), (-2, "RKV_E_UNSUPPORTED"), (-3, "RKV_E_HIP"),
                       (-4, "RKV_E_NOMEM"), (-5, "RKV_E_STATE")]:
        assert P.lib().rkv_status_string(code).decode() == name


def test_row_bytes():
    assert P.row_bytes(P.RKV_F32, 128) == 512
    assert P.row_bytes(P.RKV_F16, 128) == 256
    assert P.row_bytes(P.RKV_Q8_0, 128) == 136
    assert P.row_bytes(P.RKV_Q4_0, 128) == 72
    assert P.row_bytes(P.RKV_Q8_0, 512) == 544
    assert P.row_bytes(P.RKV_Q8_0, 48) == 0
    assert P.row_bytes(P.RKV_TBQ3, 128) == 52
    assert P.row_bytes(P.RKV_TBQ3, 512) == 208
    assert P.row_bytes(P.RKV_TBQ3, 64) == 0
    assert P.row_bytes(7, 128) == 0


@pytest.mark.parametrize("B", [2, 3, 4])
def test_ring_schedule_exhaustive(B):
    """slot = j mod B; the copy of item j waits for the compute of item j - B;
    the order is layer-major, tile-minor, and empty layers contribute nothing."""
    import itertools
    for tiles in itertools.product(range(0, 4), repeat=3):
        sched = P.rkv_ring_schedule(list(tiles), B)
        assert len(sched) == sum(tiles)
        expect = [(l, t) for l, n in enumerate(tiles) for t in range(n)]
        assert [(a, b) for a, b, _, _ in sched] == expect
        for j, (_, _, slot, waits) in enumerate(sched):
            assert slot == j % B
            assert waits == (j - B if j >= B else -1)
            if waits >= 0:
                assert sched[waits][2] == slot  # the item it waits for used the same slot


def test_ring_schedule_rejects():
    with pytest.raises(P.RkvError) as e:
        P.rkv_ring_schedule([1, 2], 1)
    assert e.value.code == P.RKV_E_INVAL
    with pytest.raises(P.RkvError):
        P.rkv_ring_schedule([1, -2], 2)


def _ws(desc, view):
    return P.rkv_attend_workspace_bytes(desc, view)


def test_validation_before_any_device_call():
    v = P.make_view(0x1000, 0x2000, P.RKV_F16, P.RKV_F16, 100, 2048, 2048, 256, 256)
    cases = [
        (P.Desc(1, 8, 3, 128, 0.1), v, P.RKV_E_INVAL),                 # Hq % Hkv without a map
        (P.Desc(1, 8, 2, 96, 0.1), v, P.RKV_E_UNSUPPORTED),            # head_dim
        (P.Desc(0, 8, 2, 128, 0.1), v, P.RKV_E_INVAL),                 # n_seq
        (P.Desc(1, 8, 2, 128, 0.1, softcap=-1.0), v, P.RKV_E_INVAL),   # softcap
        (P.Desc(1, 4, 2, 128, 0.1, q_to_kv=[0, 1, 2, 0]), v, P.RKV_E_INVAL),  # map out of range
        (P.Desc(1, 8, 2, 128, 0.1), P.make_view(0x1000, 0x2000, 9, 1, 10, 2048, 2048, 256, 256), P.RKV_E_INVAL),
        (P.Desc(1, 8, 2, 128, 0.1), P.make_view(0x1004, 0x2000, 1, 1, 10, 2048, 2048, 256, 256), P.RKV_E_INVAL),
        (P.Desc(1, 8, 2, 128, 0.1), P.make_view(0x1000, 0x2000, 1, 1, 10, 2040, 2048, 256, 256), P.RKV_E_INVAL),
        (P.Desc(1, 8, 2, 128, 0.1), P.make_view(0x1000, 0x2000, 1, 1, -1, 2048, 2048, 256, 256), P.RKV_E_INVAL),
        (P.Desc(1, 8, 2, 128, 0.1), P.make_view(0, 0x2000, 1, 1, 10, 2048, 2048, 256, 256), P.RKV_E_INVAL),
        (P.Desc(2, 8, 2, 128, 0.1), P.make_view(0x1000, 0x2000, 1, 1, 10, 2048, 2048, 256, 256, 0, 4096),
         P.RKV_E_INVAL),                                                # K shared, V per sequence
        (P.Desc(1, 8, 2, 512, 0.1), P.make_view(0x1000, 0x2000, 1, 1, 100000, 2048, 2048, 1024, 1024), None),
    ]
    for desc, view, code in cases:
        if code is None:
            assert _ws(desc, view) > 0
            continue
        with pytest.raises(P.RkvError) as e:
            _ws(desc, view)
        assert e.value.code == code, (e.value, code)
        assert P.lib().rkv_last_error().decode()


def test_workspace_sizes():
    d = P.Desc(1, 40, 8, 128, 0.088)
    assert _ws(d, P.make_view(0x1000, 0x2000, 1, 1, 0, 2048, 2048, 256, 256)) == 0  # empty segment
    small = _ws(d, P.make_view(0x1000, 0x2000, 1, 1, 64, 2048, 2048, 256, 256))
    big = _ws(d, P.make_view(0x1000, 0x2000, 1, 1, 49152, 2048, 2048, 256, 256))
    assert 0 <= small < big  # a segment one workgroup per item covers needs no workspace
    # partials are a small fraction of the K/V bytes they summarise
    assert big < 0.05 * 49152 * 2048 * 2


def test_combine_and_dequant_host_checks():
    vp = ctypes.c_void_p
    arr = (vp * 1)(vp(0x1000))
    L = P.lib()
    assert L.rkv_lse_combine(0, arr, arr, 4, 128, 0x1000, 0x2000, None) == P.RKV_E_INVAL
    assert L.rkv_lse_combine(65, arr, arr, 4, 128, 0x1000, 0x2000, None) == P.RKV_E_INVAL
    assert L.rkv_dequant_q8_0(0x1000, 33, 0x2000, None) == P.RKV_E_INVAL
    assert L.rkv_dequant_q4_0(0x1000, -32, 0x2000, None) == P.RKV_E_INVAL
    assert L.rkv_dequant_q8_0(None, 0, None, None) == P.RKV_OK  # nothing to do


def test_ring_host_checks():
    h = ctypes.c_void_p(0)
    L = P.lib()
    assert L.rkv_ring_create(1, 1024, 1024, None, ctypes.byref(h)) == P.RKV_E_INVAL
    assert L.rkv_ring_create(17, 1024, 1024, None, ctypes.byref(h)) == P.RKV_E_INVAL
    assert L.rkv_ring_create(2, 0, 1024, None, ctypes.byref(h)) == P.RKV_E_INVAL
    assert L.rkv_ring_destroy(None) == P.RKV_OK
    assert L.rkv_ring_end_step(None) == P.RKV_E_INVAL


def test_library_fully_linked():
    """Every symbol the library references resolves (a kernel whose host stub
    was not emitted shows up here, not at the first launch)."""
    ctypes.CDLL(P.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
