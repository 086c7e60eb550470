"""GPU: the write path (rkv_append_kv) against the oracle.

Stored bytes must equal, bit for bit, what the oracle's encoder
(orc_encode_row) makes of the same binary32 rows, placed where the oracle's
router (orc_route) sends each position: window row p for p < wc, tail row
p - wc otherwise, per layer ("Rolling-KV: step/graph-level tail prefetch
(design)", "Staged plan", S0 / bug-1341; "F5 M7 -- Rolling KV", "2026-07-14 --
bug-2172 SHIPPED").  Rows the call does not write keep their bytes.
Attention over caches built by appends must match the oracle's attention over
the oracle-built caches within the method's tolerances, also when the tail is
in pinned host memory and streamed by the ring across decode steps.
"""
import numpy as np
import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import compare, default_scale, note

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0xA5


class Region:
    """A position-major byte region [cap][n_kv_heads] of rows of (k_type, v_type),
    with head and position strides padded by ``pad`` bytes, in device or
    pinned host memory, filled with a sentinel; plus its expected bytes."""

    def __init__(self, cap, hkv, d, kt, vt, pad=0, host=False, n_seq=1):
        self.cap, self.hkv, self.d, self.kt, self.vt, self.n_seq = cap, hkv, d, kt, vt, n_seq
        self.rbk, self.rbv = synth.row_bytes(kt, d), synth.row_bytes(vt, d)
        self.hk, self.hv = self.rbk + pad, self.rbv + pad
        self.pk, self.pv = hkv * self.hk + pad, hkv * self.hv + pad
        self.sk, self.sv = cap * self.pk, cap * self.pv
        kw = dict(dtype=torch.uint8, pin_memory=True) if host else dict(dtype=torch.uint8, device=DEV)
        self.k = torch.full((max(1, n_seq * self.sk),), SENTINEL, **kw)
        self.v = torch.full((max(1, n_seq * self.sv),), SENTINEL, **kw)
        self.ek = np.full(max(1, n_seq * self.sk), SENTINEL, dtype=np.uint8)
        self.ev = np.full(max(1, n_seq * self.sv), SENTINEL, dtype=np.uint8)

    def view(self, n_keys=None, start=0, seq=None):
        """View for the C ABI (n_keys = capacity by default); seq strides set
        unless a single sequence is selected."""
        n = self.cap if n_keys is None else n_keys
        k = self.k.data_ptr() + start * self.pk + (0 if seq is None else seq * self.sk)
        v = self.v.data_ptr() + start * self.pv + (0 if seq is None else seq * self.sv)
        ss = (self.sk, self.sv) if (seq is None and self.n_seq > 1) else (0, 0)
        return P.make_view(k, v, self.kt, self.vt, n, self.pk, self.pv, self.hk, self.hv, *ss)

    def expect(self, seq, row, xk, xv):
        """Place the oracle's encoding of one position's rows [hkv][d]."""
        bk = oracle.encode_rows(xk, self.kt)
        bv = oracle.encode_rows(xv, self.vt)
        for h in range(self.hkv):
            a = seq * self.sk + row * self.pk + h * self.hk
            self.ek[a:a + self.rbk] = bk[h]
            a = seq * self.sv + row * self.pv + h * self.hv
            self.ev[a:a + self.rbv] = bv[h]

    def check(self, what):
        gk = self.k.cpu().numpy()
        gv = self.v.cpu().numpy()
        for name, g, e in (("K", gk, self.ek), ("V", gv, self.ev)):
            bad = np.nonzero(g != e)[0]
            assert bad.size == 0, f"{what} {name}: {bad.size} bytes differ, first at {bad[:8]}"

    def oracle_view(self, start, stop, seq=0):
        """Oracle view over the expected (oracle-made) bytes of rows [start, stop)."""
        return oracle.View(self.ek.ctypes.data + seq * self.sk + start * self.pk,
                           self.ev.ctypes.data + seq * self.sv + start * self.pv,
                           self.kt, self.vt, stop - start, self.pk, self.pv, self.hk, self.hv, keep=(self,))


def oracle_append(window, tail, fresh, pos0, seq, k_new, v_new):
    """Expected effect of one append, by the oracle's router and encoder."""
    wc = window.cap if window else 0
    tc = tail.cap if tail else 0
    kn, vn = k_new.cpu().numpy(), v_new.cpu().numpy()
    j = 0
    for t in range(kn.shape[0]):
        region, row = oracle.route(pos0 + t, wc, tc)
        (window if region == "window" else tail).expect(seq, row, kn[t], vn[t])
        if region == "tail" and fresh is not None:
            fresh.expect(0, j, kn[t], vn[t])
            j += 1


def append(window, tail, fresh, pos0, seq, k_new, v_new, ring=None, layer=0, stream=None):
    n, hkv, d = k_new.shape
    assert k_new.shape == v_new.shape and k_new.dtype == torch.float32 and k_new.is_contiguous()
    assert v_new.is_contiguous() and k_new.device.type == "cuda"
    P.rkv_append_kv(hkv, d, n, pos0, seq, k_new, v_new, None if window is None else window.view(seq=seq),
                    None if tail is None else tail.view(seq=seq), None if fresh is None else fresh.view(),
                    ring, layer, stream)


T = synth
BIT_CASES = [
    # (D, window K, window V, tail K, tail V, tail in host memory, pad bytes)
    (128, T.Q8_0, T.Q4_0, T.Q8_0, T.Q4_0, True, 0),
    (128, T.F16, T.F16, T.Q8_0, T.Q4_0, False, 4),
    (64, T.F32, T.Q8_0, T.Q4_0, T.F16, True, 2),
    (256, T.Q4_0, T.Q8_0, T.F32, T.Q8_0, False, 2),
    (512, T.Q8_0, T.Q8_0, T.Q4_0, T.Q4_0, True, 6),
    (512, T.F16, T.F32, T.F16, T.F32, False, 0),
]


@pytest.mark.parametrize("case", BIT_CASES, ids=lambda c: f"D{c[0]}-w{c[1]}{c[2]}-t{c[3]}{c[4]}-{'host' if c[5] else 'dev'}-pad{c[6]}")
def test_append_bytes_bit_exact(case):
    """Three appends into sequence 1 of two: a chunk that crosses from the
    window into the tail, one token into the tail, and a chunk inside the
    window; every byte of window, tail and the device copy of the tail rows
    equals the oracle's, untouched rows keep the sentinel."""
    D, wk, wv, tk, tv, host, pad = case
    hkv, wc, tc = 3, 20, 40
    note(f"append bytes: D={D} window=({wk},{wv}) tail=({tk},{tv}) host={host} pad={pad}")
    win = Region(wc, hkv, D, wk, wv, pad, n_seq=2)
    tail = Region(tc, hkv, D, tk, tv, pad, host=host, n_seq=2)
    fresh = Region(64, hkv, D, tk, tv, pad)
    calls = [(5, 37), (42, 1), (0, 4)]
    for i, (pos0, n) in enumerate(calls):
        kx = synth.append_rows(n, hkv, D, synth.stream_seed(D, 11, i)).to(DEV)
        vx = synth.append_rows(n, hkv, D, synth.stream_seed(D, 12, i)).to(DEV)
        fr = fresh if i < 2 else None
        if fr is not None:  # the copy holds only this call's tail rows
            fr.ek[:] = SENTINEL
            fr.k.fill_(SENTINEL)
            fr.v.fill_(SENTINEL)
            fr.ev[:] = SENTINEL
        append(win, tail, fr, pos0, 1, kx, vx)
        oracle_append(win, tail, fr, pos0, 1, kx, vx)
        torch.cuda.synchronize()
        if fr is not None:
            fr.check(f"fresh after call {i}")
    win.check("window")
    tail.check("tail")


def test_append_layer_without_tail():
    """A layer whose window holds every position (no tail) writes every row to
    its window ("Staged plan", S0 / bug-1341: routing by the layer's own
    window size); a position past its capacity is an error and writes
    nothing."""
    hkv, D, wc = 2, 128, 48
    win = Region(wc, hkv, D, T.Q8_0, T.Q4_0)
    kx = synth.append_rows(wc, hkv, D, 21).to(DEV)
    vx = synth.append_rows(wc, hkv, D, 22).to(DEV)
    append(win, None, None, 0, 0, kx, vx)
    oracle_append(win, None, None, 0, 0, kx, vx)
    torch.cuda.synchronize()
    win.check("window")
    with pytest.raises(P.RkvError) as e:
        append(win, None, None, wc, 0, kx[:1], vx[:1])
    assert e.value.code == P.RKV_E_INVAL
    torch.cuda.synchronize()
    win.check("window after the rejected call")


def test_append_errors():
    hkv, D = 2, 128
    win = Region(8, hkv, D, T.Q8_0, T.Q8_0)
    host_win = Region(8, hkv, D, T.Q8_0, T.Q8_0, host=True)
    tail = Region(8, hkv, D, T.Q8_0, T.Q8_0)
    small = Region(1, hkv, D, T.Q8_0, T.Q8_0)
    kx = synth.append_rows(4, hkv, D, 31).to(DEV)
    with pytest.raises(P.RkvError) as e:  # window must be device memory
        append(host_win, tail, None, 0, 0, kx, kx)
    assert e.value.code == P.RKV_E_INVAL
    with pytest.raises(P.RkvError) as e:  # fresh copy too small for the tail rows
        append(win, tail, small, 6, 0, kx, kx)
    assert e.value.code == P.RKV_E_INVAL
    with pytest.raises(P.RkvError) as e:  # head_dim not supported
        P.rkv_append_kv(hkv, 96, 1, 0, 0, kx, kx, win.view(), tail.view())
    assert e.value.code == P.RKV_E_UNSUPPORTED
    torch.cuda.synchronize()
    win.check("window")  # nothing written by the rejected calls
    tail.check("tail")


@pytest.mark.parametrize("kt,vt", [(T.Q8_0, T.Q4_0), (T.F16, T.F16), (T.Q8_0, T.Q8_0)])
def test_append_then_attend(kt, vt):
    """A prefill chunk that crosses into the tail, then decode steps of one
    token: after each, attention over window + device tail matches the
    oracle's attention over the oracle-built cache.  (Rows at N(0,1) scale:
    with the 2^10-scaled blocks of the encoder tests, scores reach ~10^3 and
    binary32 scoring alone moves O by ~0.1, beyond an absolute tolerance.)"""
    hkv, hq, D, wc, tc = 4, 16, 128, 96, 160
    note(f"append then attend: K={kt} V={vt}")
    win = Region(wc, hkv, D, kt, vt)
    tail = Region(tc, hkv, D, kt, vt)
    desc = P.Desc(1, hq, hkv, D, default_scale(D))
    n = 0
    for step, chunk in enumerate([130, 1, 1, 1, 7, 1]):
        kx = synth.append_rows(chunk, hkv, D, synth.stream_seed(5, 1, step), large=False).to(DEV)
        vx = synth.append_rows(chunk, hkv, D, synth.stream_seed(5, 2, step), large=False).to(DEV)
        append(win, tail, None, n, 0, kx, vx)
        oracle_append(win, tail, None, n, 0, kx, vx)
        n += chunk
        q = synth.make_query(1, hq, D, synth.stream_seed(5, 3, step), DEV)
        segs = [win.view(min(n, wc))] + ([tail.view(n - wc)] if n > wc else [])
        o, lse = P.attend_split(desc, q, segs)
        torch.cuda.synchronize()
        views = [win.oracle_view(0, min(n, wc))] + ([tail.oracle_view(0, n - wc)] if n > wc else [])
        o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, hkv, default_scale(D))
        compare(o, lse, o_ref, l_ref, what=f"n_kv={n}")
    win.check("window")
    tail.check("tail")


@pytest.mark.parametrize("L,B,tile", [(3, 2, 32), (1, 4, 32)])
def test_append_ring_decode(L, B, tile):
    """Decode steps with the tail in pinned host memory, streamed by the ring:
    each layer appends its new token (window full, so it goes to the tail and
    to a device copy), attends window + the copy in one launch, then streams
    the tail rows of earlier steps.  Nothing on the host waits for the GPU
    inside the loop and a large matrix product runs before every append, so
    the GPU trails the host: a step's prefetch copies of rows appended one
    step earlier are correct only if they wait for that append.  Every step's
    result matches the oracle over the cache as it was at that step (rows are
    only appended); the host tails end equal to the oracle's bytes."""
    hkv, hq, D, wc, tc, kt, vt = 2, 8, 128, 64, 256, T.Q8_0, T.Q4_0
    steps, n0 = 6, 100
    note(f"append + ring decode: L={L} B={B} tile={tile}")
    desc = P.Desc(1, hq, hkv, D, default_scale(D))
    wins = [Region(wc, hkv, D, kt, vt) for _ in range(L)]
    tails = [Region(tc, hkv, D, kt, vt, host=True) for _ in range(L)]
    fresh = [Region(1, hkv, D, kt, vt) for _ in range(L)]
    ring = P.Ring(B, tile * tails[0].pk, tile * tails[0].pv)
    stream = torch.cuda.current_stream()
    rows = lambda n, seed: synth.append_rows(n, hkv, D, seed, large=False).to(DEV)
    pre = [(rows(n0, synth.stream_seed(7, 1, li)), rows(n0, synth.stream_seed(7, 2, li))) for li in range(L)]
    new = {(s_, li): (rows(1, synth.stream_seed(8, 1, 100 * s_ + li)), rows(1, synth.stream_seed(8, 2, 100 * s_ + li)),
                      synth.make_query(1, hq, D, synth.stream_seed(8, 3, 100 * s_ + li), DEV))
           for s_ in range(steps) for li in range(L)}
    lag = torch.randn(3072, 3072, device=DEV)
    results = []
    torch.cuda.synchronize()
    try:
        n = n0
        for li in range(L):  # prefill: 64 window rows + 36 tail rows per layer
            append(wins[li], tails[li], None, 0, 0, *pre[li], ring, li, stream)
        for step in range(steps):
            ring.rkv_ring_begin_step([t.view(n - wc) for t in tails], tile)
            for li in range(L):
                for _ in range(3):
                    lag = lag @ lag
                    lag /= lag.abs().max()
                kx, vx, q = new[(step, li)]
                append(wins[li], tails[li], fresh[li], n, 0, kx, vx, ring, li, stream)
                o_w, l_w = P.attend_split(desc, q, [wins[li].view(wc), fresh[li].view(1)], stream)
                ws = P.workspace(ring.rkv_stream_tail_workspace_bytes(li, desc))
                o = torch.empty_like(q)
                lse = torch.empty(1, hq, dtype=torch.float32, device=DEV)
                ring.rkv_stream_tail(li, desc, q, o_w, l_w, o, lse, ws, stream)
                results.append((step, li, n + 1, q, o, lse))
            ring.rkv_ring_end_step()
            n += 1
        torch.cuda.synchronize()
    finally:
        ring.close()
    for li in range(L):
        oracle_append(wins[li], tails[li], None, 0, 0, *pre[li])
    for step in range(steps):
        for li in range(L):
            kx, vx, _ = new[(step, li)]
            oracle_append(wins[li], tails[li], None, n0 + step, 0, kx, vx)
    for step, li, n_kv, q, o, lse in results:
        views = [wins[li].oracle_view(0, wc), tails[li].oracle_view(0, n_kv - wc)]
        o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, hkv, default_scale(D))
        compare(o, lse, o_ref, l_ref, what=f"step {step} layer {li} n_kv={n_kv}")
    for li in range(L):
        wins[li].check(f"window {li}")
        tails[li].check(f"tail {li}")


def test_binding_stream_is_torch_current_stream():
    """The binding's default stream (no stream argument) is torch's current
    stream, also inside a stream context and after leaving it."""
    s = torch.cuda.Stream()
    assert P._stream(None) == torch.cuda.current_stream().cuda_stream
    with torch.cuda.stream(s):
        assert P._stream(None) == s.cuda_stream
    assert P._stream(None) == torch.cuda.current_stream().cuda_stream
    assert P._stream(s) == s.cuda_stream and P._stream(s.cuda_stream) == s.cuda_stream
