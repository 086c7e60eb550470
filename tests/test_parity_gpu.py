"""GPU parity: the HIP path through the C ABI against the binary64 oracle.

Every test prints the case it runs before touching the GPU.  Inputs are
seeded synthetic caches made on the GPU and copied to the host for the
oracle (the same bytes feed both sides).
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


# ----------------------------------------------------------------------------- dequant

@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_dequant_bit_exact(kind):
    note(f"dequant {kind} bit-exact")
    nblk = 4099
    bsz = 34 if kind == "q8_0" else 18
    g = torch.Generator().manual_seed(123)
    raw = torch.randint(0, 256, (nblk, bsz), generator=g, dtype=torch.uint8)
    # finite scales of every magnitude, including subnormals and zero
    e = torch.randint(0, 31, (nblk,), generator=g)
    m = torch.randint(0, 1024, (nblk,), generator=g)
    sgn = torch.randint(0, 2, (nblk,), generator=g)
    bits = (sgn << 15) | (e << 10) | m
    raw[:, 0] = (bits & 0xFF).to(torch.uint8)
    raw[:, 1] = (bits >> 8).to(torch.uint8)
    raw[:3, 0:2] = torch.tensor([[0, 0], [1, 0], [0, 0x80]], dtype=torch.uint8)  # +0, 2^-24, -0
    n = nblk * 32
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    dev = raw.to(DEV).contiguous()
    (P.rkv_dequant_q8_0 if kind == "q8_0" else P.rkv_dequant_q4_0)(dev, n, out)
    torch.cuda.synchronize()
    ref = (oracle.dequant_q8_0 if kind == "q8_0" else oracle.dequant_q4_0)(raw.contiguous().numpy().reshape(-1), n)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------- the split path at small sizes

CASES = [
    # name, S, Hq, Hkv, D, K, V, n, wc, scale, softcap, q_to_kv
    ("tiny_f32_gqa4", 1, 8, 2, 128, synth.F32, synth.F32, 4096, 3072, None, 0.0, None),
    ("f16_gqa5_ragged", 1, 40, 8, 128, synth.F16, synth.F16, 1000, 700, None, 0.0, None),
    ("q8q8_d512_cap", 1, 16, 2, 512, synth.Q8_0, synth.Q8_0, 777, 500, None, 30.0, None),
    ("q8q8_d512_cap_stress", 1, 16, 2, 512, synth.Q8_0, synth.Q8_0, 777, 500, 1.0, 30.0, None),
    ("q8q4_gqa5", 1, 40, 8, 128, synth.Q8_0, synth.Q4_0, 1100, 512, None, 0.0, None),
    # binary32 / binary16 K beside q4_0 V rows at 128 dims (their 22-dword LDS stride), ragged tails
    ("f32q4_gqa5_d128", 1, 40, 8, 128, synth.F32, synth.Q4_0, 701, 300, None, 0.0, None),
    ("f16q4_gqa4_d128", 2, 16, 4, 128, synth.F16, synth.Q4_0, 517, 203, None, 0.0, None),
    ("q8q4_d512_wall", 1, 8, 1, 512, synth.Q8_0, synth.Q4_0, 300, 129, None, 0.0, None),
    ("q4q8_d64", 2, 6, 3, 64, synth.Q4_0, synth.Q8_0, 333, 65, None, 0.0, None),
    ("f16q4_d256_mha", 2, 4, 4, 256, synth.F16, synth.Q4_0, 257, 63, None, 0.0, None),
    ("f32f16_d64_g3", 1, 9, 3, 64, synth.F32, synth.F16, 190, 64, 0.3, 0.0, None),
    ("f16f32_d256", 1, 4, 2, 256, synth.F16, synth.F32, 130, 1, None, 5.0, None),
    ("q4q4_map", 1, 6, 2, 128, synth.Q4_0, synth.Q4_0, 500, 250, None, 0.0, [1, 0, 0, 1, 1, 0]),
    ("f16_g20_rowgroups", 1, 40, 2, 128, synth.F16, synth.F16, 400, 200, None, 0.0, None),
    ("f16_batch3_own_keys", 3, 8, 2, 128, synth.F16, synth.F16, 300, 100, None, 0.0, None),
    ("q8q8_d256_g8", 1, 16, 2, 256, synth.Q8_0, synth.Q8_0, 200, 64, None, 0.0, None),
    ("f16_d512", 1, 4, 1, 512, synth.F16, synth.F16, 150, 70, None, 0.0, None),
    # block-type K and V at head_dim 256 / 512 run as dim slices of 128 (one wave each, partial scores summed
    # across the slices of a head): MHA with a second workgroup of head slots half empty; 16 rows per slice
    # (4-wave workgroups) with a cap; sequences with their own keys; and a head map whose second row group is
    # empty for one head (its slice waves hold no rows and still walk every tile)
    ("q4q4_d512_mha3", 1, 3, 3, 512, synth.Q4_0, synth.Q4_0, 600, 300, None, 0.0, None),
    ("q8q8_d512_g16_cap", 1, 32, 2, 512, synth.Q8_0, synth.Q8_0, 300, 100, None, 10.0, None),
    ("q4q8_d256_batch2", 2, 8, 2, 256, synth.Q4_0, synth.Q8_0, 260, 130, None, 0.0, None),
    ("q8q4_d256_g2", 1, 4, 2, 256, synth.Q8_0, synth.Q4_0, 333, 200, None, 0.0, None),
    ("q8q8_d512_map_rowgroups", 1, 20, 2, 512, synth.Q8_0, synth.Q8_0, 257, 128, None, 0.0, [0] * 18 + [1] * 2),
    # more than 16 rows per KV head over block K and q4_0 V at head_dim 128: the shared-decode kernel (two KV heads
    # x four 16-row groups per workgroup): an odd KV-head count (an empty head slot) with 20 rows per head (two
    # empty row groups), one KV head of 40 rows with a cap, and 120 rows per head (two blocks of row groups)
    ("q4q4_shd_odd_heads", 1, 60, 3, 128, synth.Q4_0, synth.Q4_0, 777, 333, None, 0.0, None),
    ("q8q4_shd_rows40_cap", 1, 40, 1, 128, synth.Q8_0, synth.Q4_0, 500, 200, None, 20.0, None),
    ("q8q4_shd_rows120", 1, 240, 2, 128, synth.Q8_0, synth.Q4_0, 420, 70, None, 0.0, None),
    # more than 16 rows per KV head over f16 K and V at head_dim 128: the staged-tile kernel (one KV head x four
    # 16-row groups per workgroup, each tile staged once in LDS): 20 rows per head over an odd head count (two
    # row groups without rows), 40 rows with a cap, 120 rows (two blocks of row groups, default cache policy),
    # sequences with their own keys (32 rows per sequence and head), 64 rows over ragged tiles, a head map with
    # 18 and 2 rows, and segments of one short tile (a single split: o and lse written directly)
    ("f16_rgs_odd_heads", 1, 60, 3, 128, synth.F16, synth.F16, 777, 333, None, 0.0, None),
    ("f16_rgs_rows40_cap", 1, 40, 1, 128, synth.F16, synth.F16, 500, 200, None, 20.0, None),
    ("f16_rgs_rows120", 1, 240, 2, 128, synth.F16, synth.F16, 420, 70, None, 0.0, None),
    ("f16_rgs_batch2_own_keys", 2, 64, 2, 128, synth.F16, synth.F16, 300, 130, None, 0.0, None),
    ("f16_rgs_rows64_ragged", 1, 64, 1, 128, synth.F16, synth.F16, 129, 64, None, 0.0, None),
    ("f16_rgs_map_18_2", 1, 20, 2, 128, synth.F16, synth.F16, 257, 128, None, 0.0, [0] * 18 + [1] * 2),
    ("f16_rgs_one_tile", 1, 40, 2, 128, synth.F16, synth.F16, 50, 20, None, 0.0, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_parity(case):
    name, S, Hq, Hkv, D, kt, vt, n, wc, scale, cap, qmap = case
    scale = default_scale(D) if scale is None else scale
    note(f"split parity {name}: S={S} Hq={Hq} Hkv={Hkv} D={D} K={synth.TYPE_NAMES[kt]} V={synth.TYPE_NAMES[vt]} "
         f"n={n} wc={wc}")
    seed = zlib.crc32(name.encode()) % 100000
    # per-sequence keys for S > 1: one cache of S*n positions, sequence stride n*pos_stride
    kc, vc = pair(S * n, Hkv, D, kt, vt, seed, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(seed, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, scale, cap, qmap)
    check_host_shapes(desc, q, kc, vc)
    kss, vss = (n * kc.pos_stride, n * vc.pos_stride) if S > 1 else (0, 0)
    window = P.view_of_cache(kc, vc, 0, wc, kss, vss)
    tail = P.view_of_cache(kc, vc, wc, n, kss, vss)
    whole = P.view_of_cache(kc, vc, 0, n, kss, vss)
    o_split, l_split = attend_views(desc, q, [window, tail])
    o_whole, l_whole = attend_views(desc, q, [whole])
    torch.cuda.synchronize()
    kh, vh = kc.to("cpu"), vc.to("cpu")
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), oracle_views(kh, vh, [0, n], (kss, vss)), Hkv, scale, cap, qmap)
    compare(o_split, l_split, o_ref, l_ref, what="window+tail")
    compare(o_whole, l_whole, o_ref, l_ref, what="unsplit")


def test_tile_boundaries():
    """Segments of 1, 63, 64, 65, 127, 128, 129 keys and key ranges that end
    mid-tile."""
    D, Hq, Hkv = 128, 8, 2
    kc, vc = pair(700, Hkv, D, synth.Q8_0, synth.F16, 77, DEV)
    q = synth.make_query(1, Hq, D, 78, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.09)
    kh, vh = kc.to("cpu"), vc.to("cpu")
    for a, b in [(0, 1), (5, 68), (0, 64), (64, 129), (3, 130), (100, 227), (1, 700)]:
        note(f"tile boundary segment [{a}, {b})")
        o, l = P.attend(desc, q, P.view_of_cache(kc, vc, a, b))
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kh, vh, a, b)], Hkv, 0.09)
        compare(o, l, o_ref, l_ref, what=f"[{a},{b})")


def test_empty_and_degenerate_splits():
    """wc = 0 and wc = n: the empty side gives O = 0, LSE = -inf, and the
    combine returns the other side bit for bit."""
    D, Hq, Hkv, n = 128, 8, 2, 500
    kc, vc = pair(n, Hkv, D, synth.F16, synth.Q4_0, 88, DEV)
    q = synth.make_query(1, Hq, D, 89, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.1)
    note("empty segment")
    oe, le = P.attend(desc, q, P.view_of_cache(kc, vc, 7, 7))
    whole = P.attend(desc, q, P.view_of_cache(kc, vc))
    torch.cuda.synchronize()
    assert torch.all(oe == 0) and torch.all(torch.isneginf(le))
    for wc in (0, n):
        note(f"degenerate split wc={wc}")
        o, l = attend_views(desc, q, [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)])
        torch.cuda.synchronize()
        assert torch.equal(o, whole[0]) and torch.equal(l, whole[1])
    note("all parts empty")
    o = torch.empty_like(oe)
    l = torch.empty_like(le)
    P.rkv_lse_combine([oe, oe, oe], [le, le, le], o, l, D)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_combine_aliasing_and_single_part():
    D, rows = 128, 37
    g = torch.Generator(device=DEV).manual_seed(5)
    o1 = torch.randn(rows, D, device=DEV, generator=g)
    o2 = torch.randn(rows, D, device=DEV, generator=g)
    l1 = torch.randn(rows, device=DEV, generator=g) * 5
    l2 = torch.randn(rows, device=DEV, generator=g) * 5
    note("combine single part / aliasing")
    o = torch.empty_like(o1)
    l = torch.empty_like(l1)
    P.rkv_lse_combine([o1], [l1], o, l, D)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(l, l1)
    ref_o, ref_l = oracle.lse_combine([o1.double().cpu().numpy(), o2.double().cpu().numpy()],
                                      [l1.double().cpu().numpy(), l2.double().cpu().numpy()])
    a, b = o1.clone(), l1.clone()
    P.rkv_lse_combine([a, o2], [b, l2], a, b, D)  # in place on part 0
    torch.cuda.synchronize()
    assert np.max(np.abs(a.double().cpu().numpy() - ref_o)) < 1e-5
    assert np.max(np.abs(b.double().cpu().numpy() - ref_l)) < 1e-5


def test_deterministic():
    D, Hq, Hkv, n = 128, 40, 8, 20000
    kc, vc = pair(n, Hkv, D, synth.F16, synth.F16, 99, DEV)
    q = synth.make_query(1, Hq, D, 98, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.088)
    note("run-to-run determinism")
    a = P.attend(desc, q, P.view_of_cache(kc, vc))
    b = P.attend(desc, q, P.view_of_cache(kc, vc))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_shared_prefix_batch():
    """15 sequences share one q8_0/q4_0 prefix (sequence stride 0) and each has
    its own f16 suffix; two segments merged by the LSE combine."""
    S, Hq, Hkv, D, npre, nsuf = 15, 32, 8, 128, 2000, 300
    note(f"shared prefix: S={S} prefix={npre} suffix={nsuf}")
    pk, pv = pair(npre, Hkv, D, synth.Q8_0, synth.Q4_0, 111, DEV)
    sk, sv = pair(S * nsuf, Hkv, D, synth.F16, synth.F16, 112, DEV)
    q = synth.make_query(S, Hq, D, 113, DEV)
    desc = P.Desc(S, Hq, Hkv, D, default_scale(D))
    prefix = P.view_of_cache(pk, pv)
    suffix = P.view_of_cache(sk, sv, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)
    o, l = attend_views(desc, q, [prefix, suffix])
    o1, l1 = P.attend_split(desc, q, [prefix, suffix])  # one call: two launches, one merge
    torch.cuda.synchronize()
    pkh, pvh, skh, svh = pk.to("cpu"), pv.to("cpu"), sk.to("cpu"), sv.to("cpu")
    views = [oracle.view_of(pkh, pvh), oracle.view_of(skh, svh, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)]
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, default_scale(D))
    compare(o, l, o_ref, l_ref, what="prefix+suffix")
    compare(o1, l1, o_ref, l_ref, what="prefix+suffix, one call")


@pytest.mark.parametrize("D", [256, 512])
def test_shared_prefix_dim_slices(D):
    """A shared q8_0 / q4_0 prefix at head_dim 256 / 512 (dim slices, several
    sequences reading one copy of the keys) plus per-sequence f16 suffixes,
    merged by the LSE combine."""
    S, Hq, Hkv, npre, nsuf = 3, 8, 2, 300, 100
    note(f"shared prefix with dim slices: D={D} S={S} prefix={npre} suffix={nsuf}")
    pk, pv = pair(npre, Hkv, D, synth.Q8_0, synth.Q4_0, 121 + D, DEV)
    sk, sv = pair(S * nsuf, Hkv, D, synth.F16, synth.F16, 122 + D, DEV)
    q = synth.make_query(S, Hq, D, 123 + D, DEV)
    desc = P.Desc(S, Hq, Hkv, D, default_scale(D))
    prefix = P.view_of_cache(pk, pv)
    suffix = P.view_of_cache(sk, sv, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)
    o, l = attend_views(desc, q, [prefix, suffix])
    o1, l1 = P.attend_split(desc, q, [prefix, suffix])
    torch.cuda.synchronize()
    pkh, pvh, skh, svh = pk.to("cpu"), pv.to("cpu"), sk.to("cpu"), sv.to("cpu")
    views = [oracle.view_of(pkh, pvh), oracle.view_of(skh, svh, 0, nsuf, nsuf * sk.pos_stride, nsuf * sv.pos_stride)]
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, default_scale(D))
    compare(o, l, o_ref, l_ref, what=f"prefix+suffix D={D}")
    compare(o1, l1, o_ref, l_ref, what=f"prefix+suffix D={D}, one call")


def test_errors_on_device():
    D, Hq, Hkv, n = 128, 8, 2, 20000  # long enough to need a workspace
    kc, vc = pair(n, Hkv, D, synth.F16, synth.F16, 5, DEV)
    q = synth.make_query(1, Hq, D, 6, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.1)
    view = P.view_of_cache(kc, vc)
    ws = P.workspace(P.rkv_attend_workspace_bytes(desc, view))
    o = torch.empty(1, Hq, D, device=DEV)
    l = torch.empty(1, Hq, device=DEV)
    note("error paths")
    with pytest.raises(P.RkvError) as e:  # host query
        P.rkv_attend_segment(desc, q.cpu(), view, o, l, ws)
    assert e.value.code == P.RKV_E_INVAL
    with pytest.raises(P.RkvError) as e:  # workspace too small
        P.rkv_attend_segment(desc, q, view, o, l, ws[:16])
    assert e.value.code == P.RKV_E_INVAL
    kh = kc.to("cpu")
    with pytest.raises(P.RkvError) as e:  # host K
        P.rkv_attend_segment(desc, q, P.view_of_cache(kh, vc), o, l, ws)
    assert e.value.code == P.RKV_E_INVAL
    # nothing was enqueued by the failing calls; a good call still works
    assert ws.numel() > 16
    P.rkv_attend_segment(desc, q, view, o, l, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()


# ----------------------------------------------------------------------------- several segments in one launch

SPLIT_CASES = [
    # name, S, Hq, Hkv, D, K, V, n, cuts, softcap
    ("f16_window_tail", 1, 40, 8, 128, synth.F16, synth.F16, 6000, [0, 4500, 6000], 0.0),
    ("q8q4_window_tiles", 1, 40, 8, 128, synth.Q8_0, synth.Q4_0, 5000, [0, 2000, 3000, 4000, 5000], 0.0),
    ("q8_d512_cap", 1, 16, 2, 512, synth.Q8_0, synth.Q8_0, 3000, [0, 2250, 3000], 30.0),
    ("f16_empty_segment", 1, 8, 2, 128, synth.F16, synth.F16, 1000, [0, 0, 700, 1000], 0.0),
    ("f16_batch_own_keys", 3, 8, 2, 128, synth.F16, synth.F16, 900, [0, 300, 900], 0.0),
    ("f32_tiny", 1, 8, 2, 128, synth.F32, synth.F32, 4096, [0, 3072, 4096], 0.0),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_attend_split_parity(case):
    name, S, Hq, Hkv, D, kt, vt, n, cuts, cap = case
    note(f"attend_split {name}: segments {list(zip(cuts, cuts[1:]))}")
    seed = zlib.crc32(name.encode()) % 100000
    kc, vc = pair(S * n, Hkv, D, kt, vt, seed, DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(seed, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, default_scale(D), cap)
    kss, vss = (n * kc.pos_stride, n * vc.pos_stride) if S > 1 else (0, 0)
    segs = [P.view_of_cache(kc, vc, a, b, kss, vss) for a, b in zip(cuts, cuts[1:])]
    o, l = P.attend_split(desc, q, segs)
    torch.cuda.synchronize()
    kh, vh = kc.to("cpu"), vc.to("cpu")
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), oracle_views(kh, vh, [0, n], (kss, vss)), Hkv, default_scale(D), cap)
    compare(o, l, o_ref, l_ref, what="one launch")


def test_workspace_reuse():
    """A workspace is reused by consecutive calls without clearing; results
    stay correct and deterministic."""
    D, Hq, Hkv = 128, 40, 8
    kc, vc = pair(30000, Hkv, D, synth.F16, synth.F16, 606, DEV)
    q1 = synth.make_query(1, Hq, D, 607, DEV)
    q2 = synth.make_query(1, Hq, D, 608, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.088)
    segs = [P.view_of_cache(kc, vc, 0, 22000), P.view_of_cache(kc, vc, 22000, 30000)]
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs))
    note("workspace reuse")
    outs = []
    for qq in (q1, q2, q1, q2, q1):
        o, l = P.attend_split(desc, qq, segs, ws=ws)
        outs.append((o, l))
    torch.cuda.synchronize()
    for a, b in ((0, 2), (2, 4), (1, 3)):
        assert torch.equal(outs[a][0], outs[b][0]) and torch.equal(outs[a][1], outs[b][1])
    kh, vh = kc.to("cpu"), vc.to("cpu")
    o_ref, l_ref = oracle.attend(q2.cpu().numpy(), [oracle.view_of(kh, vh)], Hkv, 0.088)
    compare(outs[3][0], outs[3][1], o_ref, l_ref, what="reused workspace")


def test_attend_split_unsupported_group_rejected():
    """Segments of different types are accepted (one launch each), but a group
    with no kernel -- f32 rows of 512 values -- is refused before anything is
    enqueued."""
    D, Hq, Hkv = 512, 8, 2
    a, b = pair(200, Hkv, D, synth.Q8_0, synth.Q8_0, 1, DEV)
    c, d = pair(200, Hkv, D, synth.F32, synth.F32, 2, DEV)
    desc = P.Desc(1, Hq, Hkv, D, 0.1)
    q = synth.make_query(1, Hq, D, 3, DEV)
    note("a group without a kernel in a mixed call")
    with pytest.raises(P.RkvError) as e:
        P.attend_split(desc, q, [P.view_of_cache(a, b), P.view_of_cache(c, d)], ws=P.workspace(1 << 22))
    assert e.value.code == P.RKV_E_UNSUPPORTED


@pytest.mark.parametrize("kt,vt,n,wc,D,Hq,Hkv", [
    (synth.F16, synth.F16, 20000, 15000, 128, 40, 8),   # many splits: partials then the merge
    (synth.Q8_0, synth.Q4_0, 3000, 0, 128, 40, 8),      # an empty window
    (synth.Q8_0, synth.Q8_0, 5000, 3000, 512, 16, 2),   # dim slices
    (synth.F16, synth.F16, 40, 20, 128, 8, 2),          # one split: o / lse written by the first phase
])
def test_split_phases_equal_one_call(kt, vt, n, wc, D, Hq, Hkv):
    """rkv_attend_split_partials then rkv_attend_split_merge give the bits of
    rkv_attend_split."""
    note(f"split phases: K={kt} V={vt} n={n} wc={wc} D={D} Hq={Hq} Hkv={Hkv}")
    kc, vc = pair(n, Hkv, D, kt, vt, 61, DEV)
    q = synth.make_query(1, Hq, D, 62, DEV)
    desc = P.Desc(1, Hq, Hkv, D, default_scale(D))
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o1, l1 = P.attend_split(desc, q, segs)
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs))
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    P.rkv_attend_split_partials(desc, q, segs, o2, l2, ws)
    P.rkv_attend_split_merge(desc, segs, o2, l2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


MIXED = [
    # name, Hq, Hkv, D, [(K, V, keys), ...] segments in position order, softcap, masked rows
    ("f16_window_q8q4_tail", 40, 8, 128, [(synth.F16, synth.F16, 1500), (synth.Q8_0, synth.Q4_0, 700)], 0.0, 0),
    ("q8q8_window_q4q4_tail_d512_cap", 16, 2, 512, [(synth.Q8_0, synth.Q8_0, 600), (synth.Q4_0, synth.Q4_0, 330)],
     30.0, 0),
    ("three_groups", 8, 2, 128, [(synth.F16, synth.F16, 257), (synth.Q8_0, synth.Q8_0, 300),
                                 (synth.Q4_0, synth.Q4_0, 99)], 0.0, 0),
    ("f16_window_q8q4_tail_masked", 40, 8, 128, [(synth.F16, synth.F16, 1500), (synth.Q8_0, synth.Q4_0, 700)], 0.0, 6),
    ("same_types_split_apart", 8, 2, 64, [(synth.F32, synth.F16, 200), (synth.Q8_0, synth.Q4_0, 64),
                                         (synth.F32, synth.F16, 130)], 5.0, 0),
]


@pytest.mark.parametrize("case", MIXED, ids=[c[0] for c in MIXED])
def test_mixed_segments_one_call(case):
    """Segments stored at different types in one rkv_attend_split call (the
    pages' window and tail each at its own type): one launch per type group,
    one merge; against the oracle over the concatenated keys, and the two
    phases give the bits of the one call."""
    name, Hq, Hkv, D, parts, cap, nq = case
    note(f"mixed segments {name}: Hq={Hq} Hkv={Hkv} D={D} parts={[(k, v, n) for k, v, n in parts]} rows={nq}")
    seed = zlib.crc32(name.encode()) % 100000
    caches = [pair(n, Hkv, D, kt, vt, seed + 7 * i, DEV) for i, (kt, vt, n) in enumerate(parts)]
    n_all = sum(n for _, _, n in parts)
    pos = None
    if nq:
        pos = [-1, 3, 1499, 1500, 1800, n_all + 5][:nq]
    S = nq or 1
    q = synth.make_query(S, Hq, D, synth.stream_seed(seed, 3), DEV)
    desc = P.Desc(S, Hq, Hkv, D, default_scale(D), cap, q_pos=pos)
    segs, p0 = [], 0
    for (kc, vc), (_, _, n) in zip(caches, parts):
        segs.append(P.view_of_cache(kc, vc, pos0=p0))
        p0 += n
    o, l = P.attend_split(desc, q, segs)
    ws = P.workspace(P.rkv_attend_split_workspace_bytes(desc, segs))
    o2, l2 = torch.full_like(o, float("nan")), torch.full_like(l, float("nan"))
    P.rkv_attend_split_partials(desc, q, segs, o2, l2, ws)
    P.rkv_attend_split_merge(desc, segs, o2, l2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l, l2)
    views = [oracle.view_of(kc.to("cpu"), vc.to("cpu")) for kc, vc in caches]
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), views, Hkv, default_scale(D), cap, q_pos=pos)
    compare(o, l, o_ref, l_ref, what=name)
