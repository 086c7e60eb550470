"""Pins of the binary64 oracle to things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and asserts; ``test_oracle_pins``
runs them on the real oracle and ``test_oracle_mutants`` runs them on
deliberately broken copies of oracle.c to show that a plausible mistake
(a dropped term, a wrong sign, index or operand) fails at least one of them.

What pins what:
  - binary16 decoding: all 65536 bit patterns against numpy's float16.
  - block formats: hand-built q8_0 / q4_0 blocks with known values, and the
    byte sizes the pages print ("F5 M6 -- PolyKV", tier-family table and S0).
  - attention: torch's scaled_dot_product_attention and logsumexp in float64
    (library routines), closed forms of softmax, symmetry / linearity
    invariants, and brute force in pure Python on tiny inputs.
  - the split/merge: the pages' statement that the LSE-weighted combine of
    window and tail is exact online softmax ("F5 M7 -- Rolling KV",
    "Implementation decomposition, refined", S2), and that a single tile /
    an all-resident cache degenerates to plain attention.
  - the write path: binary16 encoding against hand-worked patterns, every
    binary16 value and every midpoint between neighbours (ties to even), and
    numpy's float16 cast; block quantisation against hand-worked blocks
    (tests/golden/quant_blocks.json), against optimality of each code given
    the scale (brute force over all codes), and against the round-trip error
    bound through the separately pinned dequantiser; routing against a
    hand-worked table.
  - the causal mask of several query rows: bit-equality with the unmasked
    attention over the truncated key set, torch SDPA with a boolean mask,
    closed forms and pure-Python brute force, and the masked split merge.
  - the TBQ3 tier: the codebook against the two Lloyd-Max optimality
    conditions (conditional means by numerical quadrature, midpoint
    thresholds) and Max's published 8-level table for N(0,1); splitmix64
    against its author's published first outputs; the rotation against
    scipy's Sylvester Hadamard matrix on hand-built blocks, orthogonality
    (Parseval); the encoder against brute force over the 8 levels and the
    codebook's distortion on Gaussian data; attention over TBQ3 values
    against torch SDPA on values decoded here.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- helpers

def host_pair(n, hkv, d, kt, vt, seed):
    kc = synth.make_cache(n, hkv, d, kt, synth.stream_seed(seed, 1), "cpu")
    vc = synth.make_cache(n, hkv, d, vt, synth.stream_seed(seed, 2), "cpu")
    return kc, vc


def values_f64(orc, cache) -> np.ndarray:
    """[n][hkv][d] float64 values of a host cache (float types via numpy,
    block types via the oracle's block reader, pinned separately)."""
    t = cache.data
    if cache.dtype == synth.F32:
        return t.numpy().astype(np.float64)
    if cache.dtype == synth.F16:
        return t.numpy().astype(np.float64)
    nval = cache.n_keys * cache.n_kv_heads * cache.head_dim
    raw = np.ascontiguousarray(t.numpy().reshape(-1))
    if cache.dtype == synth.TBQ3:
        return tbq3_values_f64(orc, raw).reshape(cache.n_keys, cache.n_kv_heads, cache.head_dim)
    f = orc.dequant_q8_0 if cache.dtype == synth.Q8_0 else orc.dequant_q4_0
    return f(raw, nval).astype(np.float64).reshape(cache.n_keys, cache.n_kv_heads, cache.head_dim)


def sdpa_ref(q, k, v, scale, q_to_kv):
    """torch SDPA (float64, CPU) + torch.logsumexp for the LSE.

    q [S][Hq][D], k/v [n][Hkv][D] float64 numpy -> o [S*Hq][D], lse [S*Hq]."""
    qs = torch.from_numpy(q)
    kk = torch.from_numpy(k)
    vv = torch.from_numpy(v)
    idx = torch.tensor(q_to_kv, dtype=torch.long)
    ke = kk[:, idx, :].permute(1, 0, 2).contiguous()  # [Hq][n][D]
    ve = vv[:, idx, :].permute(1, 0, 2).contiguous()
    S, Hq, D = q.shape
    outs, lses = [], []
    for b in range(S):
        qb = qs[b][:, None, :]  # [Hq][1][D]
        o = torch.nn.functional.scaled_dot_product_attention(qb[None], ke[None], ve[None], scale=scale)[0]
        scores = torch.matmul(qb, ke.transpose(1, 2)) * scale  # [Hq][1][n]
        outs.append(o[:, 0, :])
        lses.append(torch.logsumexp(scores[:, 0, :], dim=-1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def default_map(hq, hkv):
    return [h // (hq // hkv) for h in range(hq)]


def close(a, b, rtol=1e-12, atol=1e-12):
    return np.allclose(a, b, rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------- binary16 and blocks

def pin_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero preserved
    assert math.copysign(1.0, orc.f16_to_f64(0x8000)) == -1.0


def _q8_block(d_bits, qs):
    b = np.zeros(34, dtype=np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2:] = np.asarray(qs, dtype=np.int8).view(np.uint8)
    return b


def _q4_block(d_bits, nib_bytes):
    b = np.zeros(18, dtype=np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2:] = np.asarray(nib_bytes, dtype=np.uint8)
    return b


def pin_q8_0_hand_blocks(orc):
    ints = np.arange(-127, 129)  # 256 values -> 8 blocks; 128 wraps to -128 as int8
    ints[-1] = -128
    blocks = np.concatenate([_q8_block(0x3C00, ints[32 * i:32 * i + 32]) for i in range(8)])  # d = 1
    got = orc.dequant_q8_0(blocks, 256)
    assert np.array_equal(got, ints.astype(np.float32))
    # d = 2^-24 (smallest binary16 subnormal): exact products
    qs = np.arange(-16, 16)
    got = orc.dequant_q8_0(_q8_block(0x0001, qs), 32)
    assert np.array_equal(got.astype(np.float64), qs * 2.0 ** -24)
    # d = -0.5
    got = orc.dequant_q8_0(_q8_block(0xB800, qs), 32)
    assert np.array_equal(got.astype(np.float64), qs * -0.5)
    # d = 0 -> zeros
    assert not np.any(orc.dequant_q8_0(_q8_block(0x0000, qs), 32))
    # blocks are independent: a second block reads its own scale
    two = np.concatenate([_q8_block(0x3C00, qs), _q8_block(0x4000, qs)])  # d = 1, 2
    got = orc.dequant_q8_0(two, 64)
    assert np.array_equal(got[:32], qs.astype(np.float32)) and np.array_equal(got[32:], 2 * qs.astype(np.float32))


def pin_q4_0_hand_blocks(orc):
    # byte 0 = 0x1F: element 0 = low nibble 0xF -> (15-8) d; element 16 = high nibble 1 -> (1-8) d
    nb = np.full(16, 0x88, dtype=np.uint8)
    nb[0] = 0x1F
    got = orc.dequant_q4_0(_q4_block(0x4000, nb), 32)  # d = 2
    exp = np.zeros(32)
    exp[0] = 14.0
    exp[16] = -14.0
    assert np.array_equal(got.astype(np.float64), exp)
    # nibble order over the whole block: byte i = i | (15 - i) << 4
    nb = np.array([i | ((15 - i) << 4) for i in range(16)], dtype=np.uint8)
    got = orc.dequant_q4_0(_q4_block(0x3C00, nb), 32)
    exp = np.array([i - 8 for i in range(16)] + [7 - i for i in range(16)], dtype=np.float64)
    assert np.array_equal(got.astype(np.float64), exp)
    # code 8 -> 0
    assert not np.any(orc.dequant_q4_0(_q4_block(0x3C00, np.full(16, 0x88, np.uint8)), 32))


def pin_block_sizes_match_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "kv_type_sizes.json")))
    tier = g["tier_table"]
    f16_mib = tier["f16"]["kv_mib"]
    bpv = {t: orc.row_bytes(code, 32) / 32 for t, code in (("f16", synth.F16), ("q8_0", synth.Q8_0), ("q4_0", synth.Q4_0))}
    for t in ("f16", "q8_0", "q4_0"):
        assert f"{bpv[t]:.3f}" == f"{tier[t]['bpv']:.3f}", (t, bpv[t])
        assert f"{bpv[t] / bpv['f16']:.2f}x" == tier[t]["vs_f16"]
        assert f"{f16_mib * bpv[t] / 2.0:.1f}" == f"{tier[t]['kv_mib']:.1f}"
    asym = f16_mib * (bpv["q8_0"] + bpv["q4_0"]) / 2.0 / 2.0
    assert f"{asym:.1f}" == f"{g['asymmetric_kv_mib']['q8_0_k_q4_0_v']:.1f}"
    # stock scale overhead: one binary16 per 32 values = 2/32
    assert (orc.row_bytes(synth.Q8_0, 32) - 32) / 32 == 0.0625
    # rows of several blocks: blocks never straddle a row
    for d in (64, 128, 512):
        assert orc.row_bytes(synth.Q8_0, d) == 34 * d // 32
        assert orc.row_bytes(synth.Q4_0, d) == 18 * d // 32
    assert orc.row_bytes(synth.Q8_0, 48) == 0  # D % 32 != 0 is not a block row


# ----------------------------------------------------------------------------- write path

def _quant_golden():
    return json.load(open(os.path.join(GOLDEN, "quant_blocks.json")))


def pin_f16_encode_hand(orc):
    for x, bits, _why in _quant_golden()["f16"]["cases"]:
        v = float(x) if x in ("inf", "-inf") else float.fromhex(x)
        assert orc.f32_to_f16(v) == int(bits, 16), (x, bits, hex(orc.f32_to_f16(v)))


def pin_f16_encode_exhaustive(orc):
    # every finite binary16 value encodes to itself; every midpoint between
    # two neighbours (exact in binary32) goes to the one with the even
    # fraction, and the binary32 values just beside the midpoint go to the
    # nearer neighbour
    enc = np.frompyfunc(lambda v: orc.f32_to_f16(float(v)), 1, 1)
    pos = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = pos.view(np.float16).astype(np.float32)
    got = enc(vals).astype(np.int64)
    assert np.array_equal(got, pos.astype(np.int64))
    got = enc(-vals).astype(np.int64)
    assert np.array_equal(got, pos.astype(np.int64) | 0x8000)
    lo = pos[:-1].view(np.float16).astype(np.float64)
    hi = pos[1:].view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:]).astype(np.int64)
    assert np.array_equal(enc(mid).astype(np.int64), even)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(enc(below).astype(np.int64), pos[:-1].astype(np.int64))
    assert np.array_equal(enc(above).astype(np.int64), pos[1:].astype(np.int64))


def pin_f16_encode_library(orc):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000), rng.standard_normal(2000) * 1e-5,
                        rng.standard_normal(2000) * 3e4, rng.standard_normal(500) * 1e-7]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16).astype(np.int64)
    got = np.array([orc.f32_to_f16(float(v)) for v in x], dtype=np.int64)
    assert np.array_equal(got, ref)


def pin_quant_hand_blocks(orc):
    for b in _quant_golden()["blocks"]:
        x = np.array([float.fromhex(v) for v in b["x"]], dtype=np.float32)
        got = orc.encode_rows(x, b["type"]).tobytes().hex()
        assert got == b["expected"], (b["name"], got)


def _random_blocks(seed, n):
    """N(0,1) blocks at several magnitudes, some with planted ties of the
    largest magnitude (same and opposite sign) and exact half-way values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= np.float32(10.0) ** rng.integers(-6, 4, size=(n, 1)).astype(np.float32)
    for i in range(0, n, 3):
        j, k = rng.choice(32, 2, replace=False)
        x[i, k] = -x[i, j] if i % 2 else x[i, j]
        x[i, j] = x[i, k] if abs(x[i, k]) >= np.abs(x[i]).max() else x[i, j]
    x[::7] = np.round(x[::7] * 4) / 4  # quarter grid: many exact halves after scaling
    return x


def _decode_scale(orc, blk):
    return orc.f16_to_f64(int(blk[0]) | (int(blk[1]) << 8))


def _nearest_f16(orc, d32, bits):
    """bits is a binary16 value nearest to d32 (checked against both neighbours)."""
    h = orc.f16_to_f64(bits)
    for nb in (bits - 1, bits + 1):
        if (nb & 0x7FFF) <= 0x7BFF and (nb & 0x7FFF) != 0x7FFF:
            assert abs(h - d32) <= abs(orc.f16_to_f64(nb & 0xFFFF) - d32), (d32, bits)


def pin_quant_brute_force(orc):
    # Each code is the best one for the binary32 scale, over all codes the
    # format can hold; the stored scale is a nearest binary16 of it.
    x = _random_blocks(11, 96)
    q8 = orc.encode_rows(x, synth.Q8_0)
    q4 = orc.encode_rows(x, synth.Q4_0)
    cand8 = np.arange(-128, 128, dtype=np.float64)
    cand4 = np.arange(0, 16, dtype=np.float64)
    for b in range(x.shape[0]):
        xb = x[b]
        amax = float(np.abs(xb).max())
        # --- q8_0
        d = float(np.float32(amax / 127.0))  # binary64 quotient rounded once: the binary32 quotient
        inv = np.float32(1.0 / d) if d else np.float32(0.0)
        bits = int(q8[b, 0]) | (int(q8[b, 1]) << 8)
        _nearest_f16(orc, d, bits)
        codes = q8[b, 2:].view(np.int8).astype(np.float64)
        v = (xb * inv).astype(np.float64)  # the binary32 scaled values
        for i in range(32):
            err = np.abs(v[i] - cand8)
            best = cand8[err == err.min()]
            want = best[np.argmax(np.abs(best))]  # a tie goes away from zero
            assert codes[i] == want, ("q8_0", b, i, v[i], codes[i])
        # --- q4_0
        m = 0.0
        for t in range(32):  # first value of largest magnitude
            if abs(float(xb[t])) > abs(m):
                m = float(xb[t])
        d4 = m / -8.0
        assert d4 == float(np.float32(d4))
        bits = int(q4[b, 0]) | (int(q4[b, 1]) << 8)
        _nearest_f16(orc, d4, bits)
        if m == 0.0:
            assert bits == 0x8000 and np.all(q4[b, 2:] == 0x88)
            continue
        inv4 = np.float32(1.0 / d4)
        nib = q4[b, 2:]
        n = np.concatenate([nib & 15, nib >> 4]).astype(np.float64)
        v4 = (xb * inv4).astype(np.float64)
        for i in range(32):
            # n - 8 is the nearest code to v (within the rounding of one
            # binary32 add), clamped to the 16 codes; the value -m alone
            # (v = +8) needs the clamp
            err = np.abs(v4[i] - (cand4 - 8))
            assert err[int(n[i])] <= err.min() + 2.0 ** -19 * 16, ("q4_0", b, i, v4[i], n[i])
            if abs(v4[i] - round(v4[i])) > 2.0 ** -18 and abs(abs(v4[i] - np.floor(v4[i])) - 0.5) > 2.0 ** -18:
                assert n[i] - 8 == min(7, int(np.floor(v4[i] + 0.5))), ("q4_0", b, i, v4[i], n[i])
        # exact halves go up: v = k + 1/2 -> code k + 1
        for i in range(32):
            if v4[i] - np.floor(v4[i]) == 0.5 and v4[i] < 7:
                assert n[i] - 8 == np.floor(v4[i]) + 1


def pin_quant_round_trip(orc):
    # Through the separately pinned dequantiser: each value is within half a
    # step of the binary32 scale, plus what storing the scale as binary16
    # moves the grid.  q4_0's 16 codes cover -8..7 steps on the side of -m
    # ... +m: a value beyond 7.5 steps (on the side opposite m) is clamped to
    # 7 steps and may be up to a whole step away.
    x = _random_blocks(12, 200)
    for t in (synth.Q8_0, synth.Q4_0):
        blocks = orc.encode_rows(x, t)
        deq = (orc.dequant_q8_0 if t == synth.Q8_0 else orc.dequant_q4_0)(blocks.reshape(-1), x.size).reshape(x.shape)
        bb = blocks.reshape(x.shape[0], -1)
        for b in range(x.shape[0]):
            xb = x[b].astype(np.float64)
            d16 = _decode_scale(orc, bb[b])
            if t == synth.Q8_0:
                d32 = float(np.abs(xb).max()) / 127.0
                allowed = 0.5 * d32 * (1 + 2.0 ** -18) + 127 * abs(abs(d16) - d32)
            else:
                m = xb[np.argmax(np.abs(xb))]
                d32 = m / -8.0
                steps = xb / d32 if d32 else np.zeros(32)
                allowed = np.maximum(0.5, steps - 7) * abs(d32) * (1 + 2.0 ** -18) + 8 * abs(d16 - d32)
            err = np.abs(xb - deq[b].astype(np.float64))
            assert np.all(err <= allowed + 1e-30), (t, b, float(err.max()))
    # float storage types: binary32 unchanged, binary16 as numpy rounds it
    assert np.array_equal(orc.encode_rows(x, synth.F32).view(np.float32).reshape(x.shape), x)
    assert np.array_equal(orc.encode_rows(x, synth.F16).view(np.float16).reshape(x.shape), x.astype(np.float16))


def pin_route(orc):
    for pos, wc, tc, region, row in _quant_golden()["route"]["cases"]:
        if region is None:
            try:
                orc.route(pos, wc, tc)
            except ValueError:
                continue
            raise AssertionError(f"position {pos} routed with window {wc}, tail {tc}")
        assert orc.route(pos, wc, tc) == (region, row), (pos, wc, tc)


# ----------------------------------------------------------------------------- attention against library routines

def _sdpa_case(orc, n, hq, hkv, d, kt, vt, seed, q_to_kv=None, scale=None, n_seq=2):
    kc, vc = host_pair(n, hkv, d, kt, vt, seed)
    q = synth.make_query(n_seq, hq, d, synth.stream_seed(seed, 3)).numpy()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qmap = default_map(hq, hkv) if q_to_kv is None else q_to_kv
    o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, scale, 0.0, q_to_kv=q_to_kv)
    ro, rl = sdpa_ref(q.astype(np.float64), values_f64(orc, kc), values_f64(orc, vc), scale, qmap)
    assert close(o, ro, 1e-10, 1e-12), np.abs(o - ro).max()
    assert close(lse, rl, 1e-12, 1e-12), np.abs(lse - rl).max()


def pin_sdpa_float_types(orc):
    _sdpa_case(orc, 37, 8, 2, 16, synth.F32, synth.F32, 11)
    _sdpa_case(orc, 50, 6, 3, 8, synth.F16, synth.F32, 12)
    _sdpa_case(orc, 19, 4, 4, 24, synth.F32, synth.F16, 13, scale=0.37)


def pin_sdpa_block_types(orc):
    _sdpa_case(orc, 33, 4, 2, 64, synth.Q8_0, synth.Q4_0, 14)
    _sdpa_case(orc, 21, 8, 2, 32, synth.Q4_0, synth.Q8_0, 15)
    _sdpa_case(orc, 9, 2, 1, 96, synth.Q8_0, synth.Q8_0, 16)


def pin_sdpa_explicit_map(orc):
    # non-contiguous map: rows of KV head 1 are query heads 0, 3, 4
    _sdpa_case(orc, 29, 6, 2, 16, synth.F32, synth.F32, 17, q_to_kv=[1, 0, 0, 1, 1, 0])


# ----------------------------------------------------------------------------- softmax closed forms

def _const_pair(n, hkv, d, k_row, v_rows):
    k = np.broadcast_to(np.asarray(k_row, np.float32), (n, hkv, d)).copy()
    v = np.asarray(v_rows, np.float32).reshape(n, hkv, d).copy()
    kc = synth.Cache(torch.from_numpy(k), synth.F32, n, hkv, d)
    vc = synth.Cache(torch.from_numpy(v), synth.F32, n, hkv, d)
    return kc, vc


def pin_closed_forms(orc):
    n, hkv, d = 13, 1, 4
    rng = np.random.default_rng(5)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    q = np.array([[[0.5, -1.0, 2.0, 0.25]]], dtype=np.float32)
    # (i) all key rows equal -> O = mean(V), LSE = s0 + ln n with s0 = scale q.k
    k_row = np.array([1.0, 2.0, 0.5, -4.0], np.float32)
    kc, vc = _const_pair(n, hkv, d, k_row, v)
    s0 = 0.5 * float(np.dot(q[0, 0].astype(np.float64), k_row.astype(np.float64)))
    o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.5)
    assert close(o[0], v[:, 0, :].astype(np.float64).mean(0))
    assert close(lse[0], s0 + math.log(n))
    # (ii) K = 0 -> LSE = ln n
    kc, vc = _const_pair(n, hkv, d, np.zeros(d), v)
    o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.5)
    assert close(lse[0], math.log(n)) and close(o[0], v[:, 0, :].astype(np.float64).mean(0))
    # (iii) n = 1 -> O = v0, LSE = s0 (q = a e0, k0 = b e0 -> s0 = scale a b)
    q1 = np.array([[[3.0, 0, 0, 0]]], np.float32)
    kc, vc = _const_pair(1, 1, d, [0.75, 0, 0, 0], v[:1])
    o, lse = orc.attend(q1, [oracle.view_of(kc, vc)], 1, 0.5)
    assert np.array_equal(o[0], v[0, 0].astype(np.float64)) and lse[0] == 0.5 * 3.0 * 0.75
    # (iv) two keys: softmax is the logistic function of the score gap
    k2 = np.array([[[1.0, 0, 0, 0]], [[-0.5, 0, 0, 0]]], np.float32)
    v2 = np.array([[[1.0, 0, 0, 0]], [[0, 1.0, 0, 0]]], np.float32)
    kc = synth.Cache(torch.from_numpy(k2), synth.F32, 2, 1, d)
    vc = synth.Cache(torch.from_numpy(v2), synth.F32, 2, 1, d)
    o, lse = orc.attend(q1, [oracle.view_of(kc, vc)], 1, 1.0)
    gap = 3.0 * 1.0 - 3.0 * -0.5
    w0 = 1.0 / (1.0 + math.exp(-gap))
    assert close(o[0], [w0, 1 - w0, 0, 0])
    assert close(lse[0], 3.0 + math.log1p(math.exp(-gap)))
    # (v) one dominant key -> O is its value row
    kd = np.zeros((n, 1, d), np.float32)
    kd[7, 0, 0] = 100.0
    kc = synth.Cache(torch.from_numpy(kd), synth.F32, n, 1, d)
    vc = synth.Cache(torch.from_numpy(v[:, :1, :].copy()), synth.F32, n, 1, d)
    o, lse = orc.attend(q1, [oracle.view_of(kc, vc)], 1, 1.0)
    assert close(o[0], v[7, 0].astype(np.float64), 0.0, 1e-12)


def pin_empty_and_rows(orc):
    kc, vc = host_pair(16, 2, 32, synth.F16, synth.F16, 21)
    q = synth.make_query(2, 4, 32, 22).numpy()
    empty = oracle.view_of(kc, vc, 5, 5)
    o, lse = orc.attend(q, [empty], 2, 0.1)
    assert not np.any(o) and np.all(np.isneginf(lse))
    full_o, full_l = orc.attend(q, [oracle.view_of(kc, vc)], 2, 0.1)
    # an empty view contributes nothing
    o2, l2 = orc.attend(q, [empty, oracle.view_of(kc, vc), empty], 2, 0.1)
    assert np.array_equal(o2, full_o) and np.array_equal(l2, full_l)
    # a row subset equals the same rows of the full result
    rows = [7, 0, 5]
    o3, l3 = orc.attend(q, [oracle.view_of(kc, vc)], 2, 0.1, rows=rows)
    assert np.array_equal(o3, full_o[rows]) and np.array_equal(l3, full_l[rows])


# ----------------------------------------------------------------------------- softcap

def pin_softcap(orc):
    kc, vc = host_pair(40, 2, 16, synth.F32, synth.F32, 31)
    q = synth.make_query(1, 4, 16, 32).numpy()
    view = [oracle.view_of(kc, vc)]
    plain = orc.attend(q, view, 2, 1.0, 0.0)
    huge = orc.attend(q, view, 2, 1.0, 1e30)
    assert close(plain[0], huge[0]) and close(plain[1], huge[1])
    # capped scores lie in (-c, c): LSE in (ln n - c, ln n + c)
    c = 0.5
    o, lse = orc.attend(q, view, 2, 1.0, c)
    assert np.all(lse < math.log(40) + c) and np.all(lse > math.log(40) - c)
    # the cap changes the answer when scores exceed it
    assert not close(o, plain[0], 1e-3, 1e-3)
    # n = 1 with s0 = scale a b: LSE = c tanh(s0 / c)
    d = 4
    q1 = np.array([[[3.0, 0, 0, 0]]], np.float32)
    kc1, vc1 = _const_pair(1, 1, d, [2.0, 0, 0, 0], np.ones((1, 1, d)))
    for cc in (1.0, 7.5, 30.0):
        _, l1 = orc.attend(q1, [oracle.view_of(kc1, vc1)], 1, 1.0, cc)
        assert close(l1[0], cc * math.tanh(6.0 / cc))
    # two keys: logistic of the gap of capped scores
    k2 = np.array([[[1.0, 0, 0, 0]], [[-0.5, 0, 0, 0]]], np.float32)
    v2 = np.array([[[1.0, 0, 0, 0]], [[0, 1.0, 0, 0]]], np.float32)
    kc2 = synth.Cache(torch.from_numpy(k2), synth.F32, 2, 1, d)
    vc2 = synth.Cache(torch.from_numpy(v2), synth.F32, 2, 1, d)
    cc = 2.0
    o, _ = orc.attend(q1, [oracle.view_of(kc2, vc2)], 1, 1.0, cc)
    gap = cc * math.tanh(3.0 / cc) - cc * math.tanh(-1.5 / cc)
    w0 = 1.0 / (1.0 + math.exp(-gap))
    assert close(o[0], [w0, 1 - w0, 0, 0])


# ----------------------------------------------------------------------------- invariants

def pin_permutation_and_linearity(orc):
    n, hkv, d = 45, 2, 16
    kc, vc = host_pair(n, hkv, d, synth.F32, synth.F32, 41)
    q = synth.make_query(1, 4, d, 42).numpy()
    o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.3)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(n))
    kp = synth.Cache(kc.data[perm].contiguous(), synth.F32, n, hkv, d)
    vp = synth.Cache(vc.data[perm].contiguous(), synth.F32, n, hkv, d)
    op, lp = orc.attend(q, [oracle.view_of(kp, vp)], hkv, 0.3)
    assert close(o, op) and close(lse, lp)
    # O is linear in V for fixed K: O(2 V1 - 3 V2) = 2 O(V1) - 3 O(V2); LSE depends on K only
    # (values on a 2^-10 grid so that the mixture is exact in binary32)
    grid = lambda t: torch.round(t * 1024) / 1024
    v1 = synth.Cache(grid(vc.data).contiguous(), synth.F32, n, hkv, d)
    v2 = synth.Cache(grid(synth.make_cache(n, hkv, d, synth.F32, 43).data).contiguous(), synth.F32, n, hkv, d)
    vmix = synth.Cache((2 * v1.data - 3 * v2.data).contiguous(), synth.F32, n, hkv, d)
    o, lse = orc.attend(q, [oracle.view_of(kc, v1)], hkv, 0.3)
    o2, l2 = orc.attend(q, [oracle.view_of(kc, v2)], hkv, 0.3)
    om, lm = orc.attend(q, [oracle.view_of(kc, vmix)], hkv, 0.3)
    assert close(om, 2 * o - 3 * o2, 1e-9, 1e-9) and np.array_equal(lm, lse)


def pin_gqa(orc):
    n, d = 30, 8
    kc, vc = host_pair(n, 2, d, synth.F32, synth.F32, 51)
    q = synth.make_query(1, 2, d, 52).numpy()
    # GQA 3:1 with identical query rows inside a group gives identical outputs,
    # equal to MHA with one query per KV head
    q3 = np.repeat(q, 3, axis=1)
    o3, l3 = orc.attend(q3, [oracle.view_of(kc, vc)], 2, 0.25)
    o1, l1 = orc.attend(q, [oracle.view_of(kc, vc)], 2, 0.25)
    assert np.array_equal(o3, np.repeat(o1, 3, axis=0)) and np.array_equal(l3, np.repeat(l1, 3))
    # the head map selects the KV head: swapping the map swaps the KV heads
    kswap = synth.Cache(kc.data[:, [1, 0]].contiguous(), synth.F32, n, 2, d)
    vswap = synth.Cache(vc.data[:, [1, 0]].contiguous(), synth.F32, n, 2, d)
    os_, ls_ = orc.attend(q, [oracle.view_of(kswap, vswap)], 2, 0.25, q_to_kv=[1, 0])
    assert np.array_equal(os_, o1) and np.array_equal(ls_, l1)


def pin_strides(orc):
    """A head-major copy read through its own strides gives the same result."""
    n, hkv, d = 23, 3, 32
    kc, vc = host_pair(n, hkv, d, synth.Q8_0, synth.F16, 61)
    q = synth.make_query(1, 6, d, 62).numpy()
    o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.2)
    kh = kc.data.permute(1, 0, 2).contiguous()  # [hkv][n][row]
    vh = vc.data.permute(1, 0, 2).contiguous()
    krb, vrb = kc.row_bytes, vc.row_bytes
    view = oracle.View(kh.data_ptr(), vh.data_ptr(), synth.Q8_0, synth.F16, n, krb, vrb, n * krb, n * vrb, keep=(kh, vh))
    o2, l2 = orc.attend(q, [view], hkv, 0.2)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def pin_shared_prefix(orc):
    """A view with sequence stride 0 is shared; each sequence adds its own suffix."""
    S, hq, hkv, d, npre, nsuf = 3, 4, 2, 32, 20, 7
    pk, pv = host_pair(npre, hkv, d, synth.Q8_0, synth.Q4_0, 71)
    suf = [host_pair(nsuf, hkv, d, synth.F16, synth.F16, 72 + b) for b in range(S)]
    q = synth.make_query(S, hq, d, 79).numpy()
    sk = torch.stack([s[0].data for s in suf]).contiguous()  # [S][n][hkv][d]
    sv = torch.stack([s[1].data for s in suf]).contiguous()
    kst, vst = sk[0].numel() * 2, sv[0].numel() * 2
    views = [oracle.view_of(pk, pv),
             oracle.View(sk.data_ptr(), sv.data_ptr(), synth.F16, synth.F16, nsuf,
                         hkv * d * 2, hkv * d * 2, d * 2, d * 2, kst, vst, keep=(sk, sv))]
    o, lse = orc.attend(q, views, hkv, 0.125)
    for b in range(S):
        kcat = torch.cat([torch.from_numpy(values_f64(orc, pk)), torch.from_numpy(values_f64(orc, suf[b][0]))]).numpy()
        vcat = torch.cat([torch.from_numpy(values_f64(orc, pv)), torch.from_numpy(values_f64(orc, suf[b][1]))]).numpy()
        ro, rl = sdpa_ref(q[b:b + 1].astype(np.float64), kcat, vcat, 0.125, default_map(hq, hkv))
        assert close(o[b * hq:(b + 1) * hq], ro, 1e-10, 1e-12) and close(lse[b * hq:(b + 1) * hq], rl)


def pin_brute_force_tiny(orc):
    """Pure-Python brute force (no max shift, math.fsum) on tiny inputs."""
    rng = np.random.default_rng(8)
    for trial in range(6):
        n = int(rng.integers(1, 12))
        hkv = int(rng.integers(1, 3))
        g = int(rng.integers(1, 3))
        d = int(rng.integers(1, 7))
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        q = rng.standard_normal((1, hkv * g, d)).astype(np.float32)
        scale = float(rng.uniform(0.1, 1.5))
        kc = synth.Cache(torch.from_numpy(k), synth.F32, n, hkv, d)
        vc = synth.Cache(torch.from_numpy(v), synth.F32, n, hkv, d)
        o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, scale)
        for h in range(hkv * g):
            kv = h // g
            e = [math.exp(scale * math.fsum(float(q[0, h, i]) * float(k[j, kv, i]) for i in range(d))) for j in range(n)]
            z = math.fsum(e)
            assert abs(lse[h] - math.log(z)) <= 1e-12 * max(1.0, abs(math.log(z)))
            for i in range(d):
                ref = math.fsum(e[j] * float(v[j, kv, i]) for j in range(n)) / z
                assert abs(o[h, i] - ref) <= 1e-12 * max(1.0, abs(ref))


# ----------------------------------------------------------------------------- split / merge

def pin_split_merge_exact(orc):
    n, hkv, hq, d = 96, 2, 8, 32
    kc, vc = host_pair(n, hkv, d, synth.Q8_0, synth.Q4_0, 81)
    q = synth.make_query(2, hq, d, 82).numpy()
    full_o, full_l = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.18)
    # window + tail at several wc
    for wc in (1, 17, 64, 95):
        w = orc.attend(q, [oracle.view_of(kc, vc, 0, wc)], hkv, 0.18)
        t = orc.attend(q, [oracle.view_of(kc, vc, wc, n)], hkv, 0.18)
        o, l = orc.lse_combine([w[0], t[0]], [w[1], t[1]])
        assert close(o, full_o) and close(l, full_l)
    # the tail cut into T tiles (the last one partial)
    for T in (1, 2, 4, 8):
        wc = 40
        edges = [wc + (n - wc) * i // T for i in range(T + 1)]
        parts = [orc.attend(q, [oracle.view_of(kc, vc, 0, wc)], hkv, 0.18)]
        parts += [orc.attend(q, [oracle.view_of(kc, vc, a, b)], hkv, 0.18) for a, b in zip(edges, edges[1:])]
        o, l = orc.lse_combine([p[0] for p in parts], [p[1] for p in parts])
        assert close(o, full_o) and close(l, full_l)


def pin_split_degenerate(orc):
    n, hkv, hq, d = 50, 2, 4, 32
    kc, vc = host_pair(n, hkv, d, synth.F16, synth.Q8_0, 91)
    q = synth.make_query(1, hq, d, 92).numpy()
    full = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.2)
    for wc in (0, n):  # one side empty: weights exactly 0 and 1
        w = orc.attend(q, [oracle.view_of(kc, vc, 0, wc)], hkv, 0.2)
        t = orc.attend(q, [oracle.view_of(kc, vc, wc, n)], hkv, 0.2)
        o, l = orc.lse_combine([w[0], t[0]], [w[1], t[1]])
        assert np.array_equal(o, full[0]) and np.array_equal(l, full[1])
    # a single part is the identity; all parts empty -> O = 0, LSE = -inf
    o, l = orc.lse_combine([full[0]], [full[1]])
    assert np.array_equal(o, full[0]) and np.array_equal(l, full[1])
    e = orc.attend(q, [oracle.view_of(kc, vc, 3, 3)], hkv, 0.2)
    o, l = orc.lse_combine([e[0], e[0]], [e[1], e[1]])
    assert not np.any(o) and np.all(np.isneginf(l))


# ----------------------------------------------------------------------------- causal mask (several query rows)
#
# Rows of a prefill chunk or a verify step sit at absolute positions; a row at
# position p sees the keys at positions 0 .. p and no later one ("F5 M7 --
# Rolling KV", section "2026-07-14 -- bug-2172 SHIPPED": the mask is indexed by
# absolute key position, hidden keys at -inf; section "2026-07-12 -- #582-P2
# SHIPPED", bug-2161: the n_q > 1 path over window and tail).  Key t of the
# concatenated views sits at position t.

def _mask_case(seed, n=70, wc=40, hq=8, hkv=2, d=32, kt=synth.Q8_0, vt=synth.F16):
    kc, vc = host_pair(n, hkv, d, kt, vt, seed)
    pos = [-1, 0, 5, wc - 1, wc, wc + 1, n - 2, n - 1, n + 30]
    q = synth.make_query(len(pos), hq, d, synth.stream_seed(seed, 3)).numpy()
    return kc, vc, q, pos


def pin_mask_is_truncation(orc):
    """A row at position p equals, bit for bit, the unmasked row over keys
    [0, p] (the seen keys are the same and summed in the same order); p < 0
    sees nothing (O = 0, LSE = -inf); p >= n sees everything."""
    n, wc, hq, hkv = 70, 40, 8, 2
    kc, vc, q, pos = _mask_case(101)
    views = [oracle.view_of(kc, vc, 0, wc), oracle.view_of(kc, vc, wc, n)]
    o, lse = orc.attend(q, views, hkv, 0.2, q_pos=pos)
    for b, p in enumerate(pos):
        rows = slice(b * hq, (b + 1) * hq)
        if p < 0:
            assert not np.any(o[rows]) and np.all(np.isneginf(lse[rows]))
            continue
        top = min(p + 1, n)
        ro, rl = orc.attend(q[b:b + 1], [oracle.view_of(kc, vc, 0, top)], hkv, 0.2)
        assert np.array_equal(o[rows], ro) and np.array_equal(lse[rows], rl), p


def pin_mask_sdpa(orc):
    """torch SDPA (float64) with a boolean mask of keys t <= p per row."""
    n, wc, hq, hkv, d = 70, 40, 8, 2, 32
    kc, vc, q, pos = _mask_case(102, kt=synth.F16, vt=synth.Q4_0)
    o, lse = orc.attend(q, [oracle.view_of(kc, vc, 0, wc), oracle.view_of(kc, vc, wc, n)], hkv, 0.3, q_pos=pos)
    kk = torch.from_numpy(values_f64(orc, kc))
    vv = torch.from_numpy(values_f64(orc, vc))
    idx = torch.tensor(default_map(hq, hkv))
    ke = kk[:, idx, :].permute(1, 0, 2).contiguous()
    ve = vv[:, idx, :].permute(1, 0, 2).contiguous()
    for b, p in enumerate(pos):
        if p < 0:
            continue
        qb = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        mask = (torch.arange(n) <= p)[None, None, :].expand(hq, 1, n)
        ro = torch.nn.functional.scaled_dot_product_attention(qb, ke, ve, attn_mask=mask, scale=0.3)[:, 0, :]
        sc = (torch.matmul(qb, ke.transpose(1, 2)) * 0.3)[:, 0, :].masked_fill(~mask[:, 0, :], -math.inf)
        rl = torch.logsumexp(sc, dim=-1)
        rows = slice(b * hq, (b + 1) * hq)
        assert close(o[rows], ro.numpy(), 1e-10, 1e-12) and close(lse[rows], rl.numpy()), p


def pin_mask_closed_form_and_brute_force(orc):
    """p = 0: O = v_0 and LSE = s_0 exactly; tiny random cases against a
    pure-Python sum (no max shift, math.fsum) over the keys t <= p."""
    rng = np.random.default_rng(12)
    for trial in range(6):
        n = int(rng.integers(2, 12))
        hkv, g, d = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 7))
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        pos = [0] + [int(rng.integers(0, n)) for _ in range(3)]
        q = rng.standard_normal((len(pos), hkv * g, d)).astype(np.float32)
        scale = float(rng.uniform(0.1, 1.5))
        kc = synth.Cache(torch.from_numpy(k), synth.F32, n, hkv, d)
        vc = synth.Cache(torch.from_numpy(v), synth.F32, n, hkv, d)
        o, lse = orc.attend(q, [oracle.view_of(kc, vc)], hkv, scale, q_pos=pos)
        for b, p in enumerate(pos):
            for h in range(hkv * g):
                r, kv = b * hkv * g + h, h // g
                s = [scale * math.fsum(float(q[b, h, i]) * float(k[j, kv, i]) for i in range(d)) for j in range(p + 1)]
                if p == 0:
                    assert np.array_equal(o[r], v[0, kv].astype(np.float64))
                    assert abs(lse[r] - s[0]) <= 1e-15 * max(1.0, abs(s[0]))
                e = [math.exp(x) for x in s]
                z = math.fsum(e)
                assert abs(lse[r] - math.log(z)) <= 1e-12 * max(1.0, abs(math.log(z)))
                for i in range(d):
                    ref = math.fsum(e[j] * float(v[j, kv, i]) for j in range(p + 1)) / z
                    assert abs(o[r, i] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_mask_split_merge(orc):
    """Masked window and tail attended apart (the tail's keys start at
    position wc, so its rows see t <= p - wc) and merged equal the masked
    unsplit attention; a row before the tail gets a hidden tail (weight 0)
    and the window's result exactly."""
    n, wc, hq, hkv = 70, 40, 8, 2
    kc, vc, q, pos = _mask_case(103)
    full = orc.attend(q, [oracle.view_of(kc, vc)], hkv, 0.2, q_pos=pos)
    w = orc.attend(q, [oracle.view_of(kc, vc, 0, wc)], hkv, 0.2, q_pos=pos)
    t = orc.attend(q, [oracle.view_of(kc, vc, wc, n)], hkv, 0.2, q_pos=[p - wc for p in pos])
    o, l = orc.lse_combine([w[0], t[0]], [w[1], t[1]])
    assert close(o, full[0]) and close(l, full[1])
    for b, p in enumerate(pos):
        rows = slice(b * hq, (b + 1) * hq)
        if p < wc:
            assert np.all(np.isneginf(t[1][rows])) and np.array_equal(o[rows], w[0][rows])


# ----------------------------------------------------------------------------- TBQ3

# Max (1960), "Quantizing for minimum distortion", table for 8 output levels
# of a unit Gaussian: the positive output levels and the mean squared error.
MAX_1960_LEVELS = (0.2451, 0.7560, 1.3440, 2.1520)
MAX_1960_MSE = 0.03455


def _hadamard128():
    import scipy.linalg
    return scipy.linalg.hadamard(128).astype(np.float64)


def tbq3_rotation(orc):
    """R = S2 H S1 / sqrt(128) from the oracle's signs and scipy's Hadamard matrix."""
    s1, s2 = orc.tbq3_signs()
    return (s2[:, None] * _hadamard128() * s1[None, :]) / math.sqrt(128.0)


def tbq3_values_f64(orc, raw) -> np.ndarray:
    """Original-space binary64 values of TBQ3 blocks (bytes), decoded here:
    y = +-c_m n / sqrt(128), x = R^T y."""
    blk = np.asarray(raw, dtype=np.uint8).reshape(-1, 52)
    lv = orc.tbq3_levels()
    n = blk[:, 0:2].copy().view(np.float16).astype(np.float64)[:, 0]
    i = np.arange(128)
    m = (blk[:, 4 + i // 4] >> (2 * (i % 4))) & 3
    neg = (blk[:, 36 + i // 8] >> (i % 8)) & 1
    y = np.where(neg == 1, -1.0, 1.0) * lv[m] * n[:, None] / math.sqrt(128.0)
    return (y @ tbq3_rotation(orc)).reshape(-1)  # row-vector form of R^T y


def pin_tbq3_lloyd_max(orc):
    from scipy import integrate, stats
    c = orc.tbq3_levels()
    assert np.all(np.diff(c) > 0) and c[0] > 0
    t = [0.0] + [(c[j - 1] + c[j]) / 2 for j in range(1, 4)] + [np.inf]
    mse = 0.0
    for j in range(4):
        mass = stats.norm.sf(t[j]) - stats.norm.sf(t[j + 1])
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), t[j], t[j + 1], epsabs=1e-14, epsrel=1e-13)[0] / mass
        assert abs(mean - c[j]) < 1e-9, (j, mean, c[j])
        mse += 2 * integrate.quad(lambda x: (x - c[j]) ** 2 * stats.norm.pdf(x), t[j], t[j + 1], epsabs=1e-14)[0]
    assert np.max(np.abs(c - np.array(MAX_1960_LEVELS))) < 1.5e-4, c
    assert abs(mse - MAX_1960_MSE) < 1e-5, mse


def pin_splitmix64_published(orc):
    # the first outputs of splitmix64 seeded with 1234567, as its author publishes them
    assert orc.splitmix64(1234567, 5) == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                                          4593380528125082431, 16408922859458223821]


def pin_tbq3_signs_from_seed(orc):
    w = orc.splitmix64(42, 4)
    s1, s2 = orc.tbq3_signs()
    bits = lambda a, b: np.array([((a if i < 64 else b) >> (i % 64)) & 1 for i in range(128)])
    assert np.array_equal(s1, np.where(bits(w[0], w[1]) == 1, -1, 1))
    assert np.array_equal(s2, np.where(bits(w[2], w[3]) == 1, -1, 1))
    assert not np.array_equal(s1, s2)


def _tbq3_block(norm_bits, mags, negs):
    b = np.zeros(52, dtype=np.uint8)
    b[0], b[1] = norm_bits & 0xFF, norm_bits >> 8
    for i in range(128):
        b[4 + i // 4] |= (mags[i] & 3) << (2 * (i % 4))
        b[36 + i // 8] |= (negs[i] & 1) << (i % 8)
    return b


def pin_tbq3_hand_blocks(orc):
    lv = orc.tbq3_levels()
    R = tbq3_rotation(orc)
    rng = np.random.default_rng(5)
    cases = [(0x3C00, [1] * 128, [0] * 128),                      # n = 1, every value +c_1
             (0x4900, [i % 4 for i in range(128)], [(i // 4) % 2 for i in range(128)]),
             (0x0001, [3] * 128, [1] * 128),                      # subnormal norm
             (0x0000, list(rng.integers(0, 4, 128)), list(rng.integers(0, 2, 128)))]
    for nb, mags, negs in cases:
        blk = _tbq3_block(nb, mags, negs)
        n = float(np.array([nb], dtype=np.uint16).view(np.float16)[0])
        y = np.array([(-1.0 if negs[i] else 1.0) * lv[mags[i]] * n / math.sqrt(128.0) for i in range(128)])
        want = R.T @ y
        got = orc.dequant_tbq3(blk, 128).astype(np.float64)
        assert np.allclose(got, want, rtol=2e-7, atol=1e-30 + 1e-7 * np.max(np.abs(want))), (hex(nb),)
        assert np.allclose(np.linalg.norm(got), np.linalg.norm(y), rtol=1e-6, atol=1e-30)
    # a single index: value 0 at level 0, everything else at level 0 with the other sign pattern
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-12)


def pin_tbq3_encoder(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((600, 128)).astype(np.float32)
    x[0] = 0.0
    x[1] *= 1e-3
    enc = orc.encode_rows(x, synth.TBQ3)
    lv = orc.tbq3_levels()
    R = tbq3_rotation(orc)
    levels = np.concatenate([lv, -lv])
    for r in range(x.shape[0]):
        blk = enc[r]
        n = np.linalg.norm(x[r].astype(np.float64))
        assert blk[:2].copy().view(np.float16)[0] == np.float16(n), r
        assert blk[2] == 0 and blk[3] == 0
        if n == 0:
            assert not blk[4:].any()
            continue
        z = (R @ x[r].astype(np.float64)) * math.sqrt(128.0) / n
        i = np.arange(128)
        m = (blk[4 + i // 4] >> (2 * (i % 4))) & 3
        neg = (blk[36 + i // 8] >> (i % 8)) & 1
        best = np.argmin(np.abs(z[:, None] - levels[None, :]), axis=1)
        assert np.array_equal(m, best % 4) and np.array_equal(neg, (best >= 4).astype(neg.dtype)), r
    xd = orc.dequant_tbq3(np.ascontiguousarray(enc[2:].reshape(-1)), 598 * 128).reshape(598, 128).astype(np.float64)
    x2 = x[2:].astype(np.float64)
    rel = np.sum((xd - x2) ** 2) / np.sum(x2 ** 2)
    assert abs(rel - MAX_1960_MSE) < 3e-3, rel


def pin_sdpa_tbq3(orc):
    _sdpa_case(orc, 150, 8, 2, 128, synth.Q8_0, synth.TBQ3, 71)
    _sdpa_case(orc, 60, 4, 1, 256, synth.F16, synth.TBQ3, 72)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
