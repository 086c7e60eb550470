"""GPU parity over the whole legal range of the inputs, not just unit-sized
draws.

The matrix-core paths carry binary32 values as binary16 operands: the query
(times scale and log2 e) as a high and a low part, f16 K and V as they are,
block codes as exact small integers, and for block-type V the products
d * code split into high and low parts.  Legal inputs reach past binary16's
range on both sides:

  - q8_0 / q4_0 block scales d are any finite binary16 value ("F5 M6 --
    PolyKV", "S0 -- Bootstrap": a block is a binary16 scale and its codes),
    so d * code leaves binary16 once |d| >= 512 (q8_0, codes down to -128) or
    |d| >= 8192 (q4_0), and d may be subnormal;
  - q8_0 codes include -128, which the quantiser never makes;
  - a query of any binary32 size: q * scale * log2 e above 65504 overflows a
    binary16 operand, and a tiny one falls into binary16's subnormal range.

Caches come from synth.make_cache_wide (per-block power-of-two factors from
binary16-subnormal to past those limits, planted -128 codes; some runs of 64
keys hold only ordinary blocks, so both the fast and the exact path of the
V product run) and queries from synth.make_query_scaled.  The softmax scale
of each case keeps the scores of order one, so that the softmax is not a
bare argmax.

Tolerance: O is compared element by element against the binary64 oracle with
|dO| <= 2e-3 + 1e-4 * A, where A = the attention output of |V| (the same
weights over the magnitudes of the values; A is the size of the sum that O
is, so the bound scales with the data the way rounding does, and reduces to
the method's 2e-3 for unit-sized values).  LSE: |dLSE| <= 1e-3 max(1, |LSE|).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import position_split_kv_amd as P
import synth
from gpu_util import note

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, oracle.max_threads()))


def _abs_f32(c: synth.Cache) -> synth.Cache:
    """|values| of a host cache as an f32 cache (exact dequantisation by the oracle)."""
    n = c.n_keys * c.n_kv_heads * c.head_dim
    if c.dtype == synth.F32:
        x = c.data.numpy().reshape(-1)
    elif c.dtype == synth.F16:
        x = c.data.float().numpy().reshape(-1)
    elif c.dtype == synth.Q8_0:
        x = oracle.dequant_q8_0(c.data.contiguous().numpy().reshape(-1), n)
    else:
        x = oracle.dequant_q4_0(c.data.contiguous().numpy().reshape(-1), n)
    a = torch.from_numpy(np.abs(x).astype(np.float32)).view(c.n_keys, c.n_kv_heads, c.head_dim).contiguous()
    return synth.Cache(a, synth.F32, c.n_keys, c.n_kv_heads, c.head_dim)


def check(o, lse, q, views_host, views_abs, hkv, scale, softcap=0.0, what=""):
    qn = q.cpu().numpy()
    o_ref, l_ref = oracle.attend(qn, views_host, hkv, scale, softcap=softcap)
    a_ref, _ = oracle.attend(qn, views_abs, hkv, scale, softcap=softcap)
    og = o.reshape(-1, o.shape[-1]).double().cpu().numpy()
    lg = lse.reshape(-1).double().cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all(), what
    tol = 2e-3 + 1e-4 * a_ref
    worst = float(np.max(np.abs(og - o_ref) / tol))
    err_l = float(np.max(np.abs(lg - l_ref) / np.maximum(1.0, np.abs(l_ref))))
    note(f"  {what}: max |dO| / tol = {worst:.3e} (max A = {a_ref.max():.3e}), max rel dLSE = {err_l:.3e}")
    assert worst <= 1.0, (what, worst)
    assert err_l <= 1e-3, (what, err_l)


# name, S, Hq, Hkv, D, K type, K wide, V type, V wide, n, wc, scale, softcap, query row log2 factors
CASES = [
    # block-type V scales past binary16's d * code range (general kernel, MFMA P.V with the exact VALU
    # path for the tiles that need it), f16 and q8_0 keys
    ("v_q8_wide", 1, 40, 8, 128, synth.F16, False, synth.Q8_0, True, 700, 300, None, 0.0, [0]),
    ("v_q4_wide", 1, 40, 8, 128, synth.F16, False, synth.Q4_0, True, 650, 200, None, 0.0, [0]),
    # block-type K scales wide as well (codes -128 included); the softmax scale brings the large blocks'
    # scores to order one
    ("kv_q8_wide", 1, 16, 2, 128, synth.Q8_0, True, synth.Q8_0, True, 520, 260, 2.0 ** -16 / math.sqrt(128), 0.0,
     [0]),
    ("kv_q8q4_wide_16rows", 1, 32, 2, 128, synth.Q8_0, True, synth.Q4_0, True, 400, 129,
     2.0 ** -16 / math.sqrt(128), 0.0, [0]),
    # head_dim 512 as dim slices (each slice scales its own query rows before the partial scores are summed)
    ("kv_q8_wide_d512_cap", 1, 16, 2, 512, synth.Q8_0, True, synth.Q8_0, True, 333, 100,
     2.0 ** -16 / math.sqrt(512), 30.0, [0, 3, -2]),
    ("v_q4_wide_d256", 1, 8, 2, 256, synth.Q8_0, False, synth.Q4_0, True, 300, 64, None, 0.0, [0]),
    # queries whose scaled values overflow binary16 (keys in f16's subnormal range keep the scores of order
    # one) and queries in binary16's subnormal range (large keys, large softmax scale)
    ("q_big_f16", 1, 40, 8, 128, synth.F16, "tiny", synth.F16, False, 600, 250, None, 0.0, [19, 0, 18, -3, 19]),
    ("q_tiny_f16", 1, 40, 8, 128, synth.F16, "big", synth.F16, False, 600, 250, 2.0 ** 14 / math.sqrt(128), 0.0,
     [-26, -26, -25, -26, -27]),
    ("q_big_q8q4", 1, 16, 2, 128, synth.Q8_0, "tiny", synth.Q4_0, False, 500, 200, None, 0.0, [19, 18, 0, 19]),
    # the same query ranges with 40 rows per KV head over f16 K and V (the staged-tile kernel)
    ("q_big_f16_rows40", 1, 40, 1, 128, synth.F16, "tiny", synth.F16, False, 600, 250, None, 0.0, [19, 0, 18, -3, 19]),
    ("q_tiny_f16_rows40", 2, 40, 2, 128, synth.F16, "big", synth.F16, False, 600, 250, 2.0 ** 14 / math.sqrt(128),
     0.0, [-26, -26, -25, -26, -27]),
]


def _cache(n, hkv, d, t, wide, seed):
    if wide is True:
        return synth.make_cache_wide(n, hkv, d, t, seed, DEV)
    c = synth.make_cache(n, hkv, d, t if wide is False else synth.F32, seed, "cpu")
    if wide is False:
        return c.to(DEV)
    # keys of one power-of-two size: "tiny" 2^-19 (binary16 subnormal for f16), "big" 2^12
    x = c.data * (2.0 ** -19 if wide == "tiny" else 2.0 ** 12)
    return synth.Cache(synth.encode(x, t).to(DEV), t, n, hkv, d)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_wide_range(case):
    name, S, Hq, Hkv, D, kt, kw, vt, vw, n, wc, scale, cap, rl = case
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    note(f"wide range {name}: S={S} Hq={Hq} Hkv={Hkv} D={D} K={synth.TYPE_NAMES[kt]} ({kw}) "
         f"V={synth.TYPE_NAMES[vt]} ({vw}) n={n} wc={wc} scale={sc:.3e} cap={cap}")
    seed = 70000 + sum(map(ord, name))
    kc = _cache(n, Hkv, D, kt, kw, synth.stream_seed(seed, 1))
    vc = _cache(n, Hkv, D, vt, vw, synth.stream_seed(seed, 2))
    q = synth.make_query_scaled(S, Hq, D, synth.stream_seed(seed, 3), rl, DEV)
    desc = P.Desc(S, Hq, Hkv, D, sc, cap)
    segs = [P.view_of_cache(kc, vc, 0, wc), P.view_of_cache(kc, vc, wc, n)]
    o, lse = P.attend_split(desc, q, segs)
    torch.cuda.synchronize()
    kh, vh = kc.to("cpu"), vc.to("cpu")
    va = _abs_f32(vh)
    check(o, lse, q, [oracle.view_of(kh, vh)], [oracle.view_of(kh, va)], Hkv, sc, cap, what=name)


def test_wide_range_shared_decode():
    """Many rows per KV head over a shared q8_0 / q4_0 prefix (the shared-decode
    kernel): wide V scales, -128 K codes, and queries past binary16's range."""
    S, Hq, Hkv, D, n = 5, 32, 8, 128, 700
    note(f"wide range shared decode: S={S} Hq={Hq} Hkv={Hkv} D={D} prefix {n} q8_0 (wide) / q4_0 (wide)")
    seed = 71001
    kc = synth.make_cache_wide(n, Hkv, D, synth.Q8_0, synth.stream_seed(seed, 1), DEV)
    vc = synth.make_cache_wide(n, Hkv, D, synth.Q4_0, synth.stream_seed(seed, 2), DEV)
    sc = 2.0 ** -16 / math.sqrt(D)
    q = synth.make_query_scaled(S, Hq, D, synth.stream_seed(seed, 3), [0, 5, -7, 0], DEV)
    desc = P.Desc(S, Hq, Hkv, D, sc)
    o, lse = P.attend_split(desc, q, [P.view_of_cache(kc, vc)])
    torch.cuda.synchronize()
    kh, vh = kc.to("cpu"), vc.to("cpu")
    check(o, lse, q, [oracle.view_of(kh, vh)], [oracle.view_of(kh, _abs_f32(vh))], Hkv, sc, what="shared decode")
