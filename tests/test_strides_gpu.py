"""GPU: block-type K and V stored at padded position strides (each position's
rows followed by unused bytes), against the binary64 oracle.

The caches the other tests build pack their rows (position stride = KV heads x
row bytes), so with one KV head the position stride is a single row and only
the clamped tile copy runs.  Here the rows are laid out again at the smallest
strides the whole-tile copies take (4 x the padded LDS row, rounded up to the
row type's alignment: q8_0 rows at head_dim 128, 136 bytes, at 144; q4_0, 72
bytes, at 80) and at wider ones, so that the whole-tile copies run with a small
wrap increment and with large ones, in the general kernel, with dim slices and
in the shared-decode kernel.
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


class Strided:
    """A position-major cache re-laid at a given position stride (heads packed
    inside a position); the same attributes the views of both sides read."""

    def __init__(self, cache, pos_stride, data=None):
        rb, H = cache.row_bytes, cache.n_kv_heads
        assert pos_stride >= H * rb and pos_stride % 2 == 0
        self.dtype, self.n_keys, self.n_kv_heads, self.head_dim = cache.dtype, cache.n_keys, H, cache.head_dim
        self.row_bytes, self.head_stride, self.pos_stride = rb, rb, pos_stride
        if data is None:
            src = cache.data.contiguous().view(torch.uint8).reshape(cache.n_keys, H * rb)
            data = torch.zeros(cache.n_keys * pos_stride, dtype=torch.uint8, device=src.device)
            data.view(cache.n_keys, pos_stride)[:, : H * rb] = src
        self.data = data

    def to(self, device):
        return Strided(self, self.pos_stride, self.data.to(device))


def pad_to_lds_row(rb):
    """4 x the padded LDS row of a block-type row of rb bytes, rounded up to
    the alignment the boundary asks of that row's pointers and strides."""
    dw = rb // 4 + 4 if rb % 16 == 0 else (rb // 4 if (rb // 4) % 2 else rb // 4 + 1)
    align = 16 if rb % 16 == 0 else 8 if rb % 8 == 0 else 4
    return -(-4 * dw // align) * align


CASES = [
    # name, K type, V type, D, Hq, Hkv, n_seq (shared caches), n keys, wc, extra bytes per position
    ("q8q4_one_head_min", synth.Q8_0, synth.Q4_0, 128, 5, 1, 1, 700, 300, 0),
    ("q8q4_one_head_wide", synth.Q8_0, synth.Q4_0, 128, 5, 1, 1, 700, 300, 64),
    ("q8q8_d512_slices", synth.Q8_0, synth.Q8_0, 512, 16, 2, 1, 600, 250, 96),
    ("q8q4_shared_decode", synth.Q8_0, synth.Q4_0, 128, 40, 8, 8, 650, 200, 32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_padded_position_strides(case):
    name, kt, vt, D, Hq, Hkv, S, n, wc, extra = case
    note(f"strides {name}: K {synth.TYPE_NAMES[kt]} V {synth.TYPE_NAMES[vt]} D={D} {Hq}/{Hkv} heads, S={S}, n={n}")
    kc0, vc0 = pair(n, Hkv, D, kt, vt, 8300 + D + Hkv, "cpu")
    kh = Strided(kc0, Hkv * pad_to_lds_row(kc0.row_bytes) + extra)
    vh = Strided(vc0, Hkv * pad_to_lds_row(vc0.row_bytes) + extra)
    kd, vd = kh.to(DEV), vh.to(DEV)
    q = synth.make_query(S, Hq, D, synth.stream_seed(8300, 3, D), DEV)
    scale = 1.0 / math.sqrt(D)
    desc = P.Desc(S, Hq, Hkv, D, scale)
    o, lse = P.attend_split(desc, q, [P.view_of_cache(kd, vd, 0, wc), P.view_of_cache(kd, vd, wc, n)])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend(q.cpu().numpy(), [oracle.view_of(kh, vh)], Hkv, scale)
    compare(o, lse, o_ref, l_ref, what=f"padded strides {name}")
