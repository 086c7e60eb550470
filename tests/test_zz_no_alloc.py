"""GPU: rkv_attend_split_noalloc (partials in the library's fixed scratch
array) against rkv_attend_split (partials in a caller's workspace) through
the C ABI.

The two run the same launches and arithmetic, so their outputs must agree
bit for bit; the sampled rows are also checked against the binary64 oracle
within the method's tolerances.  Two calls in a row, the second with a
smaller input (fewer keys, heads and a different type pair), show that the
array keeping the first call's contents does not leak into the second; a
call whose partials exceed the array is refused before anything is enqueued.
"""
import math

import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import compare, note, pair

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_both(desc, q, segs):
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs))
    o_ref = torch.full((desc.c.n_seq, desc.c.n_q_heads, desc.c.head_dim), float("nan"), device=DEV)
    l_ref = torch.full((desc.c.n_seq, desc.c.n_q_heads), float("nan"), device=DEV)
    P.rkv_attend_split(desc, q, segs, o_ref, l_ref, ws)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    P.rkv_attend_split_noalloc(desc, q, segs, o, lse)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_equals_workspace_form_two_calls():
    oracle.set_threads(min(16, oracle.max_threads()))
    # call 1: f16 K / V, 40 / 8 heads, window + tail over 20000 keys
    S, Hq, Hkv, D, n, wc = 1, 40, 8, 128, 20000, 14000
    note(f"noalloc call 1: f16 Hq={Hq} Hkv={Hkv} D={D} n={n} wc={wc}")
    kc, vc = pair(n, Hkv, D, synth.F16, synth.F16, 81001, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(81001, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    assert P.rkv_attend_split_workspace_bytes(desc, segs) <= P.RKV_NOALLOC_MAX_BYTES
    o, lse, o_ref, l_ref = _run_both(desc, q, segs)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "call 1: noalloc != workspace form"
    rows = [0, 7, 12, 19, 22, 27, 34, 39]
    kh, vh = kc.to("cpu"), vc.to("cpu")
    ro, rl = oracle.attend(q.cpu().numpy(), [oracle.view_of(kh, vh)], Hkv, 1.0 / math.sqrt(D), rows=rows)
    compare(o, lse, ro, rl, rows=rows, what="noalloc call 1 vs oracle")

    # call 2, smaller: q8_0 K / q4_0 V, 16 / 2 heads, 3000 keys, softcap
    S, Hq, Hkv, D, n, wc = 1, 16, 2, 128, 3000, 1000
    note(f"noalloc call 2: q8_0/q4_0 Hq={Hq} Hkv={Hkv} D={D} n={n} wc={wc} softcap 30")
    kc, vc = pair(n, Hkv, D, synth.Q8_0, synth.Q4_0, 81002, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(81002, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D), 30.0)
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o, lse, o_ref, l_ref = _run_both(desc, q, segs)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "call 2: noalloc != workspace form"
    kh, vh = kc.to("cpu"), vc.to("cpu")
    ro, rl = oracle.attend(q.cpu().numpy(), [oracle.view_of(kh, vh)], Hkv, 1.0 / math.sqrt(D), softcap=30.0)
    compare(o, lse, ro, rl, what="noalloc call 2 vs oracle")


def test_noalloc_empty_and_too_large():
    note("noalloc: all segments empty; a call whose partials exceed the array")
    S, Hq, Hkv, D = 2, 8, 2, 128
    kc, vc = pair(64, Hkv, D, synth.F16, synth.F16, 81003, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(81003, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    o = torch.full((S, Hq, D), float("nan"), device=DEV)
    lse = torch.zeros(S, Hq, device=DEV)
    P.rkv_attend_split_noalloc(desc, q, [P.view_of_cache(kc, vc, 0, 0)], o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # 64 sequences with their own keys x 128 query heads x head_dim 512 over four segments: at least one
    # split per segment, so the partials need at least 4 x 8192 rows x 512 x 4 bytes, past the array
    S, Hq, Hkv, D, n = 64, 128, 8, 512, 64
    desc = P.Desc(S, Hq, Hkv, D, 1.0 / math.sqrt(D))
    rb = P.row_bytes(P.RKV_F16, D)
    k = torch.zeros(S * n * Hkv * rb, dtype=torch.uint8, device=DEV)
    seg = [P.make_view(k, k, P.RKV_F16, P.RKV_F16, n, Hkv * rb, Hkv * rb, rb, rb, n * Hkv * rb, n * Hkv * rb)] * 4
    need = P.rkv_attend_split_workspace_bytes(desc, seg)
    assert need > P.RKV_NOALLOC_MAX_BYTES, need
    qq = torch.zeros(S, Hq, D, device=DEV)
    oo = torch.full((S, Hq, D), 7.0, device=DEV)
    ll = torch.full((S, Hq), 7.0, device=DEV)
    with pytest.raises(P.RkvError) as ei:
        P.rkv_attend_split_noalloc(desc, qq, seg, oo, ll)
    assert ei.value.code == P.RKV_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(oo == 7.0) and torch.all(ll == 7.0)  # nothing was enqueued
