"""GPU: several query rows over the split cache with a causal mask.

The rows of a prefill chunk or of a verify step sit at absolute positions and
see the keys at positions up to their own ("F5 M7 -- Rolling KV", section
"2026-07-14 -- bug-2172 SHIPPED": the mask is indexed by absolute key
position, -inf for hidden keys; section "2026-07-12 -- #582-P2 SHIPPED",
bug-2161: the n_q > 1 path over window and tail).  They are passed as n_seq
query rows over shared (sequence stride 0) window and tail views, each view
carrying the absolute position of its first key.  Results must match the
oracle's masked unsplit attention within the method's tolerances; a row
that sees no key of a call gets O = 0, LSE = -inf.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import attend_views, check_host_shapes, compare, default_scale, note, pair

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, oracle.max_threads()))


def positions(kind, n, wc, nq):
    if kind == "verify":  # the last nq positions: draft tokens after the cache
        return list(range(n - nq, n))
    # a chunk spread over the cache: before anything, first keys, tile edges,
    # the window edge, inside the tail, the last key, past the end
    pos = [-1, 0, 1, 63, 64, 65, wc - 1, wc, wc + 1, (wc + n) // 2, n - 1, n + 100]
    return pos[:nq]


CASES = [
    # name, Hq, Hkv, D, K, V, n, wc, kind, n_q, softcap
    ("f16_verify8_gqa5", 40, 8, 128, synth.F16, synth.F16, 3000, 2000, "verify", 8, 0.0),
    ("f16_chunk12_gqa5", 40, 8, 128, synth.F16, synth.F16, 3000, 2000, "chunk", 12, 0.0),
    ("q8q4_verify16_gqa4", 32, 8, 128, synth.Q8_0, synth.Q4_0, 2500, 1700, "verify", 16, 0.0),
    ("q8q4_chunk12_gqa5", 40, 8, 128, synth.Q8_0, synth.Q4_0, 2500, 1700, "chunk", 12, 0.0),
    ("q8q8_d512_chunk9_cap", 16, 2, 512, synth.Q8_0, synth.Q8_0, 1500, 1000, "chunk", 9, 30.0),
    ("q4q8_d256_chunk12", 8, 2, 256, synth.Q4_0, synth.Q8_0, 900, 600, "chunk", 12, 0.0),
    ("f32_d64_chunk12", 8, 2, 64, synth.F32, synth.F32, 700, 450, "chunk", 12, 0.0),
    ("f16_d256_verify4", 8, 4, 256, synth.F16, synth.F16, 800, 500, "verify", 4, 5.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_masked_rows_parity(case):
    """One launch over window + tail, the unsplit cache, and the three-call
    form (window, tail, combine), all against the oracle."""
    name, Hq, Hkv, D, kt, vt, n, wc, kind, nq, cap = case
    pos = positions(kind, n, wc, nq)
    note(f"masked rows {name}: Hq={Hq} Hkv={Hkv} D={D} n={n} wc={wc} q_pos={pos}")
    seed = zlib.crc32(name.encode()) % 100000
    kc, vc = pair(n, Hkv, D, kt, vt, seed, DEV)
    q = synth.make_query(nq, Hq, D, synth.stream_seed(seed, 3), DEV)
    scale = default_scale(D)
    desc = P.Desc(nq, Hq, Hkv, D, scale, cap, q_pos=pos)
    check_host_shapes(desc, q, kc, vc)
    window, tail = P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)
    o_split, l_split = P.attend_split(desc, q, [window, tail])
    o_whole, l_whole = P.attend(desc, q, P.view_of_cache(kc, vc, 0, n))
    o_three, l_three = attend_views(desc, q, [window, tail])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kc.to("cpu"), vc.to("cpu"))], Hkv, scale, cap,
                                 q_pos=pos)
    compare(o_split, l_split, o_ref, l_ref, what="window+tail, one launch")
    compare(o_whole, l_whole, o_ref, l_ref, what="unsplit")
    compare(o_three, l_three, o_ref, l_ref, what="window, tail, combine")


def test_masked_single_split_empty_rows():
    """A short segment attended by one workgroup per head group (results
    written without the partial merge): rows before the segment get O = 0,
    LSE = -inf; rows inside it see a prefix of it."""
    Hq, Hkv, D, n, p0 = 8, 2, 128, 40, 1000
    kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.Q4_0, 5, DEV)
    pos = [p0 - 5, p0 - 1, p0, p0 + 7, p0 + n - 1, p0 + 500]
    q = synth.make_query(len(pos), Hq, D, 6, DEV)
    desc = P.Desc(len(pos), Hq, Hkv, D, 0.1, q_pos=pos)
    note(f"masked single split: n={n} pos0={p0} q_pos={pos}")
    o, lse = P.attend(desc, q, P.view_of_cache(kc, vc, 0, n, pos0=p0))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kc.to("cpu"), vc.to("cpu"))], Hkv, 0.1,
                                 q_pos=[p - p0 for p in pos])
    compare(o, lse, o_ref, l_ref, what="segment at pos0 1000")
    assert not torch.any(o[:2]) and torch.all(torch.isneginf(lse[:2]))


@pytest.mark.parametrize("kt,vt", [(synth.Q8_0, synth.Q4_0), (synth.F16, synth.F16)], ids=["q8q4", "f16"])
def test_masked_stream_tail(kt, vt):
    """A verify step of 6 rows (30 per KV head: the shared-decode kernel for
    q8_0 / q4_0, the staged-tile kernel for f16) with the tail in pinned host
    memory, streamed in tiles: equal bit for bit to the same ring step with the
    tail resident in device memory (attended in place, each tile at its
    absolute position), to the segment calls per tile + combine to rounding,
    and to the oracle."""
    Hq, Hkv, D, n, wc, tile, B = 40, 8, 128, 3000, 1200, 512, 3
    pos = [wc - 3, wc + 2, 2000, n - 3, n - 2, n - 1]
    note(f"masked stream tail {synth.TYPE_NAMES[kt]}/{synth.TYPE_NAMES[vt]}: n={n} wc={wc} tile={tile} q_pos={pos}")
    kc, vc = pair(n, Hkv, D, kt, vt, 9, DEV)
    q = synth.make_query(len(pos), Hq, D, 10, DEV)
    desc = P.Desc(len(pos), Hq, Hkv, D, default_scale(D), q_pos=pos)
    kh = torch.empty(kc.data[wc:].shape, dtype=kc.data.dtype, pin_memory=True)
    vh = torch.empty(vc.data[wc:].shape, dtype=vc.data.dtype, pin_memory=True)
    kh.copy_(kc.data[wc:])
    vh.copy_(vc.data[wc:])
    kt = synth.Cache(kh, kc.dtype, n - wc, Hkv, D)
    vt = synth.Cache(vh, vc.dtype, n - wc, Hkv, D)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def ring_step(tail):
        ring = P.Ring(B, tile * kc.pos_stride, tile * vc.pos_stride)
        try:
            ring.rkv_ring_begin_step([tail], tile)
            o_w, l_w = P.attend(desc, q, P.view_of_cache(kc, vc, 0, wc), stream)
            ws = P.workspace(ring.rkv_stream_tail_workspace_bytes(0, desc))
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
            ring.rkv_stream_tail(0, desc, q, o_w, l_w, o, lse, ws, stream)
            ring.rkv_ring_end_step()
            torch.cuda.synchronize()
        finally:
            ring.close()
        return o, lse

    o, lse = ring_step(P.view_of_cache(kt, vt, pos0=wc))
    o_res, l_res = ring_step(P.view_of_cache(kc, vc, wc, n))
    assert torch.equal(o, o_res) and torch.equal(lse, l_res)
    views = [P.view_of_cache(kc, vc, 0, wc)] + [P.view_of_cache(kc, vc, a, min(n, a + tile))
                                                 for a in range(wc, n, tile)]
    o_seg, l_seg = attend_views(desc, q, views)
    torch.cuda.synchronize()
    assert torch.allclose(o, o_seg, rtol=0, atol=1e-5) and torch.allclose(lse, l_seg, rtol=1e-6, atol=1e-6)
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kc.to("cpu"), vc.to("cpu"))], Hkv,
                                 default_scale(D), q_pos=pos)
    compare(o, lse, o_ref, l_ref, what="streamed")


def test_masked_limits():
    """Query positions for more than 64 rows, or a negative view position,
    are refused before anything is enqueued."""
    kc, vc = pair(100, 2, 128, synth.F16, synth.F16, 3, DEV)
    q = synth.make_query(65, 8, 128, 4, DEV)
    with pytest.raises(P.RkvError) as e:
        P.attend(P.Desc(65, 8, 2, 128, 0.1, q_pos=list(range(65))), q, P.view_of_cache(kc, vc))
    assert e.value.code == P.RKV_E_UNSUPPORTED
    with pytest.raises(P.RkvError) as e:
        P.attend(P.Desc(1, 8, 2, 128, 0.1, q_pos=[5]), q[:1].contiguous(), P.view_of_cache(kc, vc, pos0=-1))
    assert e.value.code == P.RKV_E_INVAL
