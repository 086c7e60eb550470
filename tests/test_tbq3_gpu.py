"""GPU: the TBQ3 value tier through the C ABI against the binary64 oracle.

TBQ3 values are read in registers by the split kernel (rotated-space levels
times the block's norm, summed with the softmax weights) and the output gets
the inverse rotation once.  The oracle decodes every value row to the
original space in binary64 and runs plain softmax attention.  Caches are
drawn directly in the TBQ3 format (norms of normal draws, uniform indices and
signs), so every level and sign occurs.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import attend_views, check_host_shapes, compare, default_scale, note, oracle_views, pair

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, oracle.max_threads()))


def test_dequant_tbq3():
    """Standalone dequantisation: random blocks with norms of every binary16
    magnitude (zero, subnormal, the largest finite), against the oracle's
    binary64 values; the tolerance is a few binary32 roundings of the
    block's largest value (levels, the norm product, seven butterfly stages)."""
    note("dequant tbq3")
    nblk = 3001
    g = torch.Generator().manual_seed(321)
    raw = torch.randint(0, 256, (nblk, 52), generator=g, dtype=torch.uint8)
    e = torch.randint(0, 31, (nblk,), generator=g)
    m = torch.randint(0, 1024, (nblk,), generator=g)
    bits = (e << 10) | m
    bits[:4] = torch.tensor([0, 1, 0x03FF, 0x7BFF])  # 0, 2^-24, largest subnormal, 65504
    raw[:, 0] = (bits & 0xFF).to(torch.uint8)
    raw[:, 1] = (bits >> 8).to(torch.uint8)
    raw[:, 2:4] = 0
    n = nblk * 128
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    P.rkv_dequant_tbq3(raw.to(DEV).contiguous(), n, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(nblk, 128)
    want = oracle.dequant_tbq3(raw.contiguous().numpy().reshape(-1), n).astype(np.float64).reshape(nblk, 128)
    scale = np.maximum(np.max(np.abs(want), axis=1, keepdims=True), 1e-38)
    err = np.max(np.abs(got - want) / scale)
    note(f"  max error / block max = {err:.3e}")
    assert err <= 8 * 2.0 ** -23, err
    assert np.all(got[0] == 0.0)


# name, S, Hq, Hkv, D, K type, n, wc, scale, softcap, q_pos
CASES = [
    ("q8_t3_gqa5", 1, 40, 8, 128, synth.Q8_0, 3000, 1700, None, 0.0, None),       # block K: DMA path
    ("q4_t3_gqa4_ragged", 1, 8, 2, 128, synth.Q4_0, 1001, 333, None, 0.0, None),
    ("f16_t3_gqa4", 1, 8, 2, 128, synth.F16, 777, 400, None, 0.0, None),          # f16 K: staged values
    ("f32_t3", 1, 4, 2, 128, synth.F32, 300, 100, None, 0.0, None),               # f32 K: the VALU path
    ("q8_t3_d256_slices", 1, 16, 2, 256, synth.Q8_0, 500, 250, None, 0.0, None),  # 2 dim slices
    ("q8_t3_d512_cap", 1, 16, 2, 512, synth.Q8_0, 400, 129, None, 30.0, None),    # 4 dim slices, softcap
    ("f16_t3_d256", 1, 4, 2, 256, synth.F16, 260, 64, None, 0.0, None),           # VALU path, two blocks
    ("q8_t3_rows20", 1, 40, 2, 128, synth.Q8_0, 600, 300, None, 0.0, None),       # two row groups per head
    ("q8_t3_batch3", 3, 8, 2, 128, synth.Q8_0, 300, 100, None, 0.0, None),        # sequences with own keys
    ("q8_t3_masked", 4, 8, 2, 128, synth.Q8_0, 700, 300, None, 0.0, [299, 300, 500, 699]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tbq3_parity(case):
    name, S, Hq, Hkv, D, kt, n, wc, scale, cap, qpos = case
    scale = default_scale(D) if scale is None else scale
    note(f"tbq3 parity {name}: S={S} Hq={Hq} Hkv={Hkv} D={D} K={synth.TYPE_NAMES[kt]} n={n} wc={wc}")
    seed = zlib.crc32(name.encode()) % 100000
    own = S > 1 and qpos is None
    kc, vc = pair(S * n if own else n, Hkv, D, kt, synth.TBQ3, seed, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(seed, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, scale, cap, q_pos=qpos)
    check_host_shapes(desc, q, kc, vc)
    kss, vss = (n * kc.pos_stride, n * vc.pos_stride) if own else (0, 0)
    window = P.view_of_cache(kc, vc, 0, wc, kss, vss)
    tail = P.view_of_cache(kc, vc, wc, n, kss, vss)
    o_seg, l_seg = attend_views(desc, q, [window, tail])
    o_one, l_one = P.attend_split(desc, q, [window, tail])
    torch.cuda.synchronize()
    kh, vh = kc.to("cpu"), vc.to("cpu")
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), oracle_views(kh, vh, [0, n], (kss, vss)), Hkv, scale, cap,
                                 q_pos=qpos)
    compare(o_seg, l_seg, o_ref, l_ref, what="segment, segment, combine")
    compare(o_one, l_one, o_ref, l_ref, what="one call over both segments")


def test_tbq3_tile_edges_and_single_split():
    """Segments that end mid-tile, a single-key segment, and a call small
    enough for one split (the output written directly, then turned back)."""
    D, Hq, Hkv = 128, 8, 2
    kc, vc = pair(300, Hkv, D, synth.Q8_0, synth.TBQ3, 501, DEV)
    q = synth.make_query(1, Hq, D, 502, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.09)
    kh, vh = kc.to("cpu"), vc.to("cpu")
    for a, b in [(0, 1), (5, 68), (64, 129), (1, 300)]:
        note(f"tbq3 segment [{a}, {b})")
        o, l = P.attend(desc, q, P.view_of_cache(kc, vc, a, b))
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kh, vh, a, b)], Hkv, 0.09)
        compare(o, l, o_ref, l_ref, what=f"[{a},{b})")


def test_tbq3_limits():
    """TBQ3 keys, head_dim 64, a call mixing TBQ3 and other values, a streamed
    TBQ3 tail and an append to TBQ3 storage are refused before any launch."""
    note("tbq3 limits")
    D, Hq, Hkv = 128, 8, 2
    kc, vc = pair(200, Hkv, D, synth.Q8_0, synth.TBQ3, 601, DEV)
    k2, v2 = pair(200, Hkv, D, synth.Q8_0, synth.Q4_0, 602, DEV)
    q = synth.make_query(1, Hq, D, 603, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.1)
    with pytest.raises(P.RkvError) as e:
        P.attend(desc, q, P.view_of_cache(vc, vc))  # TBQ3 keys
    assert e.value.code == P.RKV_E_UNSUPPORTED
    with pytest.raises(P.RkvError) as e:
        P.attend_split(desc, q, [P.view_of_cache(kc, vc), P.view_of_cache(k2, v2)])
    assert e.value.code == P.RKV_E_UNSUPPORTED
    # an empty segment of another value type does not count
    o, l = P.attend_split(desc, q, [P.view_of_cache(kc, vc), P.view_of_cache(k2, v2, 0, 0)])
    k64, v64 = pair(10, Hkv, 64, synth.Q8_0, synth.Q8_0, 604, DEV)
    bad = P.view_of_cache(k64, v64)
    bad.v_type = P.RKV_TBQ3
    with pytest.raises(P.RkvError) as e:
        P.attend(P.Desc(1, Hq, Hkv, 64, 0.1), synth.make_query(1, Hq, 64, 605, DEV), bad)
    assert e.value.code == P.RKV_E_UNSUPPORTED
    ring = P.Ring(2, 64 * kc.pos_stride, 64 * vc.pos_stride)
    try:
        with pytest.raises(P.RkvError) as e:
            ring.rkv_ring_begin_step([P.view_of_cache(kc, vc, 100, 200)], 64)
        assert e.value.code == P.RKV_E_UNSUPPORTED
    finally:
        ring.close()
    x = synth.append_rows(1, Hkv, D, 606, DEV, large=False)
    with pytest.raises(P.RkvError) as e:
        P.rkv_append_kv(Hkv, D, 1, 5, 0, x, x, P.view_of_cache(kc, vc), None)
    assert e.value.code == P.RKV_E_UNSUPPORTED
    torch.cuda.synchronize()


def test_tbq3_full_size_sampled_rows():
    """The streamed-tail layer shape with TBQ3 values: 40/8 heads, head_dim
    128, q8_0 K, 65536 keys as window 49152 + tail 16384 in one call; one row
    of every KV head against the oracle."""
    S, Hq, Hkv, D, n, wc = 1, 40, 8, 128, 65536, 49152
    note(f"tbq3 full size: n={n} wc={wc} q8_0 K / tbq3 V")
    kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.TBQ3, 60001, DEV)
    q = synth.make_query(S, Hq, D, 60002, DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    o, l = P.attend_split(desc, q, [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)])
    torch.cuda.synchronize()
    rows = [0, 6, 12, 17, 22, 28, 33, 39]
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kc.to("cpu"), vc.to("cpu"))], Hkv,
                                 1.0 / math.sqrt(D), rows=rows)
    compare(o, l, o_ref, l_ref, rows=rows, what="full size, one call")


@pytest.mark.parametrize("n", [50, 3000])
def test_tbq3_phases_and_no_alloc(n):
    """The split kernel and the merge enqueued apart (rkv_attend_split_partials,
    then rkv_attend_split_merge), and the allocation-free entry point, give
    rkv_attend_split's bits over TBQ3 values: with one split (the output
    written directly, then turned back) and with many."""
    D, Hq, Hkv = 128, 40, 8
    note(f"tbq3 phases / no-alloc: n={n}")
    kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.TBQ3, 700 + n, DEV)
    q = synth.make_query(1, Hq, D, 701 + n, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    segs = [P.view_of_cache(kc, vc, 0, n // 2), P.view_of_cache(kc, vc, n // 2, n)]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs))
    o1, l1 = P.attend_split(desc, q, segs, ws=ws)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    P.rkv_attend_split_partials(desc, q, segs, o2, l2, ws)
    P.rkv_attend_split_merge(desc, segs, o2, l2, ws)
    o3, l3 = torch.empty_like(o1), torch.empty_like(l1)
    P.rkv_attend_split_noalloc(desc, q, segs, o3, l3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kc.to("cpu"), vc.to("cpu"))], Hkv,
                                 1.0 / math.sqrt(D))
    compare(o1, l1, o_ref, l_ref, what=f"n={n}")
