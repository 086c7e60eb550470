"""GPU: the pinned-host tail ring (rkv_ring_* / rkv_stream_tail).

A tail held in pinned host memory, cut into tiles and streamed through a
B-slot device ring, must give bit for bit what the same step gives with the
tails resident in device memory (the ring attends those in place: same tile
cut, same launches, same merge, no copies), whatever B is; it must agree
with the segment calls per tile + rkv_lse_combine to rounding, and match the
binary64 oracle over the whole unsplit cache.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import attend_views, compare, note, pair

pytestmark = pytest.mark.gpu

DEV = "cuda"


def pinned_copy(cache, start, stop):
    """The positions [start, stop) of a device cache, in pinned host memory."""
    host = torch.empty(cache.data[start:stop].shape, dtype=cache.data.dtype, pin_memory=True)
    host.copy_(cache.data[start:stop])
    return synth.Cache(host, cache.dtype, stop - start, cache.n_kv_heads, cache.head_dim)


def make_layers(L, n, wcs, Hq, Hkv, D, kt, vt, seed):
    layers = []
    for li in range(L):
        kc, vc = pair(n, Hkv, D, kt, vt, seed + 101 * li, DEV)
        q = synth.make_query(1, Hq, D, synth.stream_seed(seed, 3, li), DEV)
        wc = wcs[li]
        layers.append(dict(kc=kc, vc=vc, q=q, wc=wc, kh=pinned_copy(kc, wc, n), vh=pinned_copy(vc, wc, n)))
    torch.cuda.synchronize()
    return layers


def run_streamed(layers, desc, B, tile, n, inplace=False):
    """One ring step over the layers: tails streamed from pinned host memory,
    or (inplace) the same tails read where they are in device memory."""
    kc0, vc0 = layers[0]["kc"], layers[0]["vc"]
    ring = P.Ring(B, tile * kc0.pos_stride, tile * vc0.pos_stride)
    stream = torch.cuda.current_stream()
    outs = []
    if inplace:
        tails = [P.view_of_cache(L_["kc"], L_["vc"], L_["wc"], n, pos0=0) for L_ in layers]
    else:
        tails = [P.view_of_cache(L_["kh"], L_["vh"]) for L_ in layers]
    try:
        ring.rkv_ring_begin_step(tails, tile)
        for li, L_ in enumerate(layers):
            if L_["wc"] > 0:
                o_w, l_w = P.attend(desc, L_["q"], P.view_of_cache(L_["kc"], L_["vc"], 0, L_["wc"]), stream)
            else:
                o_w, l_w = None, None
            ws = P.workspace(ring.rkv_stream_tail_workspace_bytes(li, desc))
            o = torch.empty_like(L_["q"])
            lse = torch.empty(L_["q"].shape[:2], dtype=torch.float32, device=DEV)
            ring.rkv_stream_tail(li, desc, L_["q"], o_w, l_w, o, lse, ws, stream)
            outs.append((o, lse))
        ring.rkv_ring_end_step()
        torch.cuda.synchronize()
    finally:
        ring.close()
    return outs


def segments(L_, desc, tile, n):
    """The segment calls per tile + rkv_lse_combine (window, tile 0, tile 1, ...)."""
    views = []
    if L_["wc"] > 0:
        views.append(P.view_of_cache(L_["kc"], L_["vc"], 0, L_["wc"]))
    for a in range(L_["wc"], n, tile):
        views.append(P.view_of_cache(L_["kc"], L_["vc"], a, min(n, a + tile)))
    return attend_views(desc, L_["q"], views)


@pytest.mark.parametrize("B", [2, 3, 4])
def test_stream_tail_bit_identical_to_resident(B):
    """q8_0 K / q4_0 V, 40/8 heads, D 128; 3 layers whose tails (2000 keys) are
    cut into 512-key tiles (the last one partial)."""
    L, n, Hq, Hkv, D, tile = 3, 4000, 40, 8, 128, 512
    note(f"ring B={B}: {L} layers, n={n}, wc=2000, tile={tile}, q8_0 K / q4_0 V")
    layers = make_layers(L, n, [2000] * L, Hq, Hkv, D, synth.Q8_0, synth.Q4_0, 7000 + B)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    outs = run_streamed(layers, desc, B, tile, n)
    res = run_streamed(layers, desc, B, tile, n, inplace=True)
    for li, L_ in enumerate(layers):
        assert torch.equal(outs[li][0], res[li][0]), f"layer {li}: streamed O differs from the resident tails"
        assert torch.equal(outs[li][1], res[li][1]), f"layer {li}: streamed LSE differs from the resident tails"
        o_s, l_s = segments(L_, desc, tile, n)
        torch.cuda.synchronize()
        assert torch.allclose(outs[li][0], o_s, rtol=0, atol=1e-5) and torch.allclose(outs[li][1], l_s, rtol=1e-6, atol=1e-6)
    # and the oracle over the whole unsplit cache of layer 1
    L_ = layers[1]
    o_ref, l_ref = oracle.attend(L_["q"].cpu().numpy(), [oracle.view_of(L_["kc"].to("cpu"), L_["vc"].to("cpu"))],
                                 Hkv, 1.0 / math.sqrt(D))
    compare(outs[1][0], outs[1][1], o_ref, l_ref, what=f"ring B={B} vs oracle")


def test_stream_tail_dim_slices():
    """Tails of q8_0 K and V at head_dim 256 (each tile attended by the dim-sliced
    kernel) through a 2-slot ring: bit for bit the resident tiles, and the oracle."""
    L, n, Hq, Hkv, D, tile = 2, 900, 8, 2, 256, 256
    note(f"ring dim slices: {L} layers, n={n}, wc=400, tile={tile}, D={D}, q8_0 K / q8_0 V")
    layers = make_layers(L, n, [400] * L, Hq, Hkv, D, synth.Q8_0, synth.Q8_0, 8400)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    outs = run_streamed(layers, desc, 2, tile, n)
    res = run_streamed(layers, desc, 3, tile, n, inplace=True)
    for li, L_ in enumerate(layers):
        assert torch.equal(outs[li][0], res[li][0]) and torch.equal(outs[li][1], res[li][1]), f"layer {li}"
    L_ = layers[0]
    o_ref, l_ref = oracle.attend(L_["q"].cpu().numpy(), [oracle.view_of(L_["kc"].to("cpu"), L_["vc"].to("cpu"))],
                                 Hkv, 1.0 / math.sqrt(D))
    compare(outs[0][0], outs[0][1], o_ref, l_ref, what="ring D256 vs oracle")


def test_stream_tail_edge_layers():
    """A layer with no window (wc = 0), a layer with an empty tail (the window
    result comes back bit for bit), and a tail shorter than one tile."""
    n, Hq, Hkv, D, tile = 1500, 8, 2, 128, 1024
    wcs = [0, n, 1000]
    note(f"ring edge layers: wc = {wcs}, n={n}, tile={tile}, f16")
    layers = make_layers(3, n, wcs, Hq, Hkv, D, synth.F16, synth.F16, 8100)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    outs = run_streamed(layers, desc, 2, tile, n)
    res = run_streamed(layers, desc, 2, tile, n, inplace=True)
    for li, L_ in enumerate(layers):
        assert torch.equal(outs[li][0], res[li][0]) and torch.equal(outs[li][1], res[li][1]), f"layer {li}"
        if li == 1:  # an empty tail: the window result comes back bit for bit
            o_w, l_w = P.attend(desc, L_["q"], P.view_of_cache(L_["kc"], L_["vc"], 0, L_["wc"]))
            torch.cuda.synchronize()
            assert torch.equal(outs[li][0], o_w) and torch.equal(outs[li][1], l_w)
        o_ref, l_ref = oracle.attend(L_["q"].cpu().numpy(),
                                     [oracle.view_of(L_["kc"].to("cpu"), L_["vc"].to("cpu"))], Hkv,
                                     1.0 / math.sqrt(D))
        compare(outs[li][0], outs[li][1], o_ref, l_ref, what=f"edge layer {li} (wc={wcs[li]})")


def test_ring_state_errors():
    """Out-of-order layers, an early end of step, a second begin, and a tail in
    pageable host memory are refused with the documented status; every check
    happens on the host before the offending work is enqueued."""
    n, Hq, Hkv, D, tile = 1024, 8, 2, 128, 256
    note("ring state errors")
    layers = make_layers(2, n, [512, 512], Hq, Hkv, D, synth.F16, synth.F16, 8200)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    kc0, vc0 = layers[0]["kc"], layers[0]["vc"]
    ring = P.Ring(2, tile * kc0.pos_stride, tile * vc0.pos_stride)
    try:
        # a tail in pageable (not pinned) host memory
        kp, vp = kc0.to("cpu"), vc0.to("cpu")
        with pytest.raises(P.RkvError) as e:
            ring.rkv_ring_begin_step([P.view_of_cache(kp, vp, 512, n)], tile)
        assert e.value.code == P.RKV_E_INVAL
        ring.rkv_ring_begin_step([P.view_of_cache(L_["kh"], L_["vh"]) for L_ in layers], tile)
        with pytest.raises(P.RkvError) as e:
            ring.rkv_ring_begin_step([P.view_of_cache(L_["kh"], L_["vh"]) for L_ in layers], tile)
        assert e.value.code == P.RKV_E_STATE
        q = layers[1]["q"]
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
        ws = P.workspace(1 << 20)
        with pytest.raises(P.RkvError) as e:  # layer 1 before layer 0
            ring.rkv_stream_tail(1, desc, q, None, None, o, lse, ws)
        assert e.value.code == P.RKV_E_STATE
        ring.rkv_stream_tail(0, desc, layers[0]["q"], None, None, o, lse, ws)
        with pytest.raises(P.RkvError) as e:  # one layer left
            ring.rkv_ring_end_step()
        assert e.value.code == P.RKV_E_STATE
        torch.cuda.synchronize()
    finally:
        ring.close()


def test_ring_consecutive_steps():
    """One ring over three steps with different tails (a decode loop): the
    slots a step starts with are released by the previous step's last tiles,
    and every step still equals its tiles attended resident, bit for bit."""
    n, Hq, Hkv, D, tile, B = 3000, 16, 4, 128, 512, 3
    note(f"ring consecutive steps: n={n}, tile={tile}, B={B}, q8_0 K / q4_0 V")
    layers = make_layers(2, n, [1000, 1000], Hq, Hkv, D, synth.Q8_0, synth.Q4_0, 8300)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    kc0, vc0 = layers[0]["kc"], layers[0]["vc"]
    ring = P.Ring(B, tile * kc0.pos_stride, tile * vc0.pos_stride)
    stream = torch.cuda.current_stream()
    try:
        for step, tail_keys in enumerate([2000, 700, 1300]):
            note(f"  step {step}: tail {tail_keys} keys per layer")
            tails = [P.view_of_cache(L_["kh"], L_["vh"], 0, tail_keys) for L_ in layers]
            ring.rkv_ring_begin_step(tails, tile)
            outs = []
            for li, L_ in enumerate(layers):
                o_w, l_w = P.attend(desc, L_["q"], P.view_of_cache(L_["kc"], L_["vc"], 0, L_["wc"]), stream)
                ws = P.workspace(ring.rkv_stream_tail_workspace_bytes(li, desc))
                o = torch.empty_like(L_["q"])
                lse = torch.empty(L_["q"].shape[:2], dtype=torch.float32, device=DEV)
                ring.rkv_stream_tail(li, desc, L_["q"], o_w, l_w, o, lse, ws, stream)
                outs.append((o, lse))
            ring.rkv_ring_end_step()
            torch.cuda.synchronize()
            res = run_streamed(layers, desc, B, tile, L_["wc"] + tail_keys, inplace=True)
            for li, L_ in enumerate(layers):
                assert torch.equal(outs[li][0], res[li][0]) and torch.equal(outs[li][1], res[li][1]), \
                    f"step {step} layer {li}"
    finally:
        ring.close()


def test_stream_tail_tiny_f32():
    """The tiny f32 configuration's streamed variant: 8 query heads / 2 KV
    heads, head_dim 128, 4096 keys = window 3072 + a 1024-key tail in pinned
    host memory, 256-key tiles through 3 slots, 2 layers: bit for bit the
    resident-tail step, and the oracle over the whole unsplit cache."""
    L, n, wc, Hq, Hkv, D, tile, B = 2, 4096, 3072, 8, 2, 128, 256, 3
    note(f"ring tiny f32: {L} layers, n={n}, wc={wc}, tile={tile}, B={B}")
    layers = make_layers(L, n, [wc] * L, Hq, Hkv, D, synth.F32, synth.F32, 9100)
    desc = P.Desc(1, Hq, Hkv, D, 1.0 / math.sqrt(D))
    outs = run_streamed(layers, desc, B, tile, n)
    res = run_streamed(layers, desc, B, tile, n, inplace=True)
    for li, L_ in enumerate(layers):
        assert torch.equal(outs[li][0], res[li][0]) and torch.equal(outs[li][1], res[li][1]), f"layer {li}"
        o_ref, l_ref = oracle.attend(L_["q"].cpu().numpy(), [oracle.view_of(L_["kc"].to("cpu"), L_["vc"].to("cpu"))],
                                     Hkv, 1.0 / math.sqrt(D))
        compare(outs[li][0], outs[li][1], o_ref, l_ref, what=f"ring tiny f32 layer {li} vs oracle")
