"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times, on sampled query rows that the binary64
oracle computes one by one (every sampled row still attends every key).

  - Qwen2.5-14B-shaped f16 layer: 40/8 heads, D 128, 65536 keys (1 % outlier
    channels x8), window 49152 + tail 16384, one rkv_attend_split launch (the
    bench step) and the three-call form;
  - Gemma-style global layer: 16/2 heads, D 512, 262144 q8_0 keys, softcap 30,
    window 196608 + tail 65536; plus the scale-1.0 softcap stress variant;
  - streamed tail: q8_0 K / q4_0 V, 40/8 heads, 131072 keys, window 65536 on
    the device, tail 65536 in pinned host memory in 8192-key tiles through a
    3-slot ring (2 layers);
  - shared prefix: 15 sequences x 32/8 heads; a 32768-key q8_0 / q4_0 prefix
    stored once plus a private 2048-key f16 suffix per sequence, as one
    rkv_attend_split call (the shared-decode launch over the prefix, the
    suffix launch, one merge: the form the benchmark times) and as the
    three-call form;
  - verify step: 8 draft rows under the causal mask over the f16 layer above,
    one rkv_attend_split call (the staged-tile kernel).

Sampled rows cover every KV head.
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


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, oracle.max_threads()))


def host_views(kc, vc, cuts=None):
    kh, vh = kc.to("cpu"), vc.to("cpu")
    return [oracle.view_of(kh, vh)], (kh, vh)


def test_qwen14b_f16_layer_full():
    S, Hq, Hkv, D, n, wc = 1, 40, 8, 128, 65536, 49152
    note(f"full size f16: Hq={Hq} Hkv={Hkv} D={D} n={n} wc={wc}, 10 outlier channels")
    kc, vc = pair(n, Hkv, D, synth.F16, synth.F16, 20001, DEV, outliers=round(0.01 * Hkv * D))
    q = synth.make_query(S, Hq, D, synth.stream_seed(20001, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o1, l1 = P.attend_split(desc, q, segs)
    o3, l3 = attend_views(desc, q, segs)
    torch.cuda.synchronize()
    # at least one row of every KV head (query head h attends KV head h // 5)
    rows = [0, 4, 5, 13, 15, 19, 22, 26, 31, 39]
    assert sorted({r // (Hq // Hkv) for r in rows}) == list(range(Hkv))
    views, _ = host_views(kc, vc)
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, 1.0 / math.sqrt(D), rows=rows)
    compare(o1, l1, o_ref, l_ref, rows=rows, what="one launch (bench step)")
    compare(o3, l3, o_ref, l_ref, rows=rows, what="segment, segment, combine")


def test_verify_step_full():
    """The verify step the benchmark times: 8 draft rows at positions 65528 ..
    65535 over the 40/8-head, head_dim 128 f16 layer of 65536 keys (window 49152
    + tail 16384), causal mask, one rkv_attend_split call (40 rows per KV head:
    the staged-tile kernel)."""
    Hq, Hkv, D, n, wc, nq = 40, 8, 128, 65536, 49152, 8
    pos = list(range(n - nq, n))
    note(f"full size verify step: {nq} rows x Hq={Hq} Hkv={Hkv} D={D} n={n} wc={wc}, q_pos={pos[0]}..{pos[-1]}")
    kc, vc = pair(n, Hkv, D, synth.F16, synth.F16, 20011, DEV, outliers=round(0.01 * Hkv * D))
    q = synth.make_query(nq, Hq, D, synth.stream_seed(20011, 3), DEV)
    desc = P.Desc(nq, Hq, Hkv, D, 1.0 / math.sqrt(D), q_pos=pos)
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o1, l1 = P.attend_split(desc, q, segs)
    torch.cuda.synchronize()
    # rows b * Hq + h: every draft position and every KV head (h // 5)
    rows = [b * Hq + h for b, h in [(0, 0), (1, 6), (2, 12), (3, 17), (4, 23), (5, 27), (6, 33), (7, 39), (7, 5),
                                    (0, 38)]]
    assert sorted({(r % Hq) // (Hq // Hkv) for r in rows}) == list(range(Hkv))
    assert sorted({r // Hq for r in rows}) == list(range(nq))
    views, _ = host_views(kc, vc)
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, 1.0 / math.sqrt(D), rows=rows, q_pos=pos)
    compare(o1, l1, o_ref, l_ref, rows=rows, what="verify step, one call (bench form)")


@pytest.mark.parametrize("scale", [None, 1.0], ids=["scale_1_over_sqrt_d", "stress_scale_1"])
def test_gemma_q8_d512_softcap_full(scale):
    S, Hq, Hkv, D, n, wc, cap = 1, 16, 2, 512, 262144, 196608, 30.0
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    note(f"full size q8_0 D512 softcap {cap}: n={n} wc={wc} scale={sc:.5f}")
    kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.Q8_0, 30001, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(30001, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, sc, cap)
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o1, l1 = P.attend_split(desc, q, segs)
    torch.cuda.synchronize()
    rows = [0, 7, 8, 15]
    views, _ = host_views(kc, vc)
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, sc, softcap=cap, rows=rows)
    compare(o1, l1, o_ref, l_ref, rows=rows, what="q8_0 D512 softcap")
    if scale is not None:
        # the cap must matter at this scale: the uncapped result is far away
        o_nc, l_nc = oracle.attend(q.cpu().numpy(), views, Hkv, sc, softcap=0.0, rows=rows)
        assert np.max(np.abs(l_nc - l_ref)) > 1e-2


def test_streamed_tail_full():
    L, S, Hq, Hkv, D, n, wc, tile, B = 2, 1, 40, 8, 128, 131072, 65536, 8192, 3
    note(f"full size streamed tail: {L} layers, n={n} wc={wc} tile={tile} B={B}, q8_0 K / q4_0 V")
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    layers = []
    for li in range(L):
        kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.Q4_0, 40001 + li, DEV)
        q = synth.make_query(S, Hq, D, synth.stream_seed(40001, 3, li), DEV)
        kh = torch.empty(kc.data[wc:].shape, dtype=kc.data.dtype, pin_memory=True)
        vh = torch.empty(vc.data[wc:].shape, dtype=vc.data.dtype, pin_memory=True)
        kh.copy_(kc.data[wc:])
        vh.copy_(vc.data[wc:])
        layers.append((kc, vc, q, synth.Cache(kh, kc.dtype, n - wc, Hkv, D), synth.Cache(vh, vc.dtype, n - wc, Hkv, D)))
    torch.cuda.synchronize()

    def ring_step(tails):
        ring = P.Ring(B, tile * layers[0][0].pos_stride, tile * layers[0][1].pos_stride)
        outs = []
        try:
            ring.rkv_ring_begin_step(tails, tile)
            for li, (kc, vc, q, _, _) in enumerate(layers):
                o_w, l_w = P.attend(desc, q, P.view_of_cache(kc, vc, 0, wc))
                ws = P.workspace(ring.rkv_stream_tail_workspace_bytes(li, desc))
                o = torch.empty_like(q)
                lse = torch.empty(S, Hq, device=DEV)
                ring.rkv_stream_tail(li, desc, q, o_w, l_w, o, lse, ws)
                outs.append((o, lse))
            ring.rkv_ring_end_step()
            torch.cuda.synchronize()
        finally:
            ring.close()
        return outs

    outs = ring_step([P.view_of_cache(t[3], t[4], pos0=wc) for t in layers])
    res = ring_step([P.view_of_cache(t[0], t[1], wc, n) for t in layers])
    rows = [0, 9, 10, 17, 24, 25, 30, 39]  # one row of every KV head or more
    for li, (kc, vc, q, _, _) in enumerate(layers):
        assert torch.equal(outs[li][0], res[li][0]) and torch.equal(outs[li][1], res[li][1]), \
            f"layer {li}: streamed != resident"
        hv, _ = host_views(kc, vc)
        o_ref, l_ref = oracle.attend(q.cpu().numpy(), hv, Hkv, 1.0 / math.sqrt(D), rows=rows)
        compare(outs[li][0], outs[li][1], o_ref, l_ref, rows=rows, what=f"streamed layer {li}")


def test_shared_prefix_full():
    S, Hq, Hkv, D, npre, nsuf = 15, 32, 8, 128, 32768, 2048
    note(f"full size shared prefix: S={S} Hq={Hq} Hkv={Hkv} prefix={npre} q8_0/q4_0, suffix={nsuf} f16")
    pk, pv = pair(npre, Hkv, D, synth.Q8_0, synth.Q4_0, 50001, DEV)
    sk, sv = pair(S * nsuf, Hkv, D, synth.F16, synth.F16, 50002, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(50001, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    prefix = P.view_of_cache(pk, pv)
    suffix = P.view_of_cache(sk, sv, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)
    o1, l1 = P.attend_split(desc, q, [prefix, suffix])
    o3, l3 = attend_views(desc, q, [prefix, suffix])
    torch.cuda.synchronize()
    pkh, pvh, skh, svh = pk.to("cpu"), pv.to("cpu"), sk.to("cpu"), sv.to("cpu")
    views = [oracle.view_of(pkh, pvh), oracle.view_of(skh, svh, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)]
    # row b * Hq + h of sequence b attends KV head h // 4: one row of every KV head, spread over the
    # sequences, plus the first and last rows
    rows = [b * Hq + 4 * g + (g % 4) for g, b in zip(range(Hkv), (0, 3, 7, 11, 14, 1, 5, 9))] + [0, S * Hq - 1]
    assert sorted({(r % Hq) // (Hq // Hkv) for r in rows}) == list(range(Hkv))
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, 1.0 / math.sqrt(D), rows=rows)
    compare(o1, l1, o_ref, l_ref, rows=rows, what="one call (bench form): prefix + suffix")
    compare(o3, l3, o_ref, l_ref, rows=rows, what="segment, segment, combine")
