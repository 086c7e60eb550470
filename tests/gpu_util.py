"""Helpers for the GPU parity tests: build the same seeded inputs for the HIP
path and the oracle, run segments through the C ABI, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import position_split_kv_amd as P
import synth

# Tolerances of the method's statement: O max-abs 2e-3, LSE relative 1e-3
# (taken as |dLSE| <= 1e-3 * max(1, |LSE|) since LSE can be near 0).
O_TOL = 2e-3
LSE_TOL = 1e-3


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def pair(n, hkv, d, kt, vt, seed, device="cuda", outliers=0):
    kc = synth.make_cache(n, hkv, d, kt, synth.stream_seed(seed, 1), device, outlier_channels=outliers,
                          channels_seed=synth.stream_seed(seed, 7))
    vc = synth.make_cache(n, hkv, d, vt, synth.stream_seed(seed, 2), device, outlier_channels=outliers,
                          channels_seed=synth.stream_seed(seed, 7))
    return kc, vc


def check_host_shapes(desc: P.Desc, q: torch.Tensor, kc, vc):
    """Shapes the kernels assume, checked on the host before any launch."""
    S, Hq, D = desc.c.n_seq, desc.c.n_q_heads, desc.c.head_dim
    assert q.shape == (S, Hq, D) and q.dtype == torch.float32 and q.is_contiguous()
    assert kc.head_dim == D and vc.head_dim == D
    assert kc.n_kv_heads == desc.c.n_kv_heads and vc.n_kv_heads == desc.c.n_kv_heads
    assert kc.data.is_contiguous() and vc.data.is_contiguous()


def attend_views(desc, q, views):
    """rkv_attend_segment on each view, then rkv_lse_combine in view order."""
    parts = [P.attend(desc, q, v) for v in views]
    if len(parts) == 1:
        return parts[0]
    o = torch.empty_like(parts[0][0])
    lse = torch.empty_like(parts[0][1])
    P.rkv_lse_combine([p[0] for p in parts], [p[1] for p in parts], o, lse, desc.c.head_dim)
    return o, lse


def oracle_views(kc_h, vc_h, cuts, seq_strides=(0, 0)):
    return [oracle.view_of(kc_h, vc_h, a, b, *seq_strides) for a, b in zip(cuts, cuts[1:])]


def compare(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, what=""):
    og = o_gpu.reshape(-1, o_gpu.shape[-1]).double().cpu().numpy()
    lg = lse_gpu.reshape(-1).double().cpu().numpy()
    if rows is not None:
        og, lg = og[rows], lg[rows]
    err_o = float(np.max(np.abs(og - o_ref))) if og.size else 0.0
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), what
    err_l = float(np.max(np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin])))) if fin.any() else 0.0
    note(f"  {what}: max|dO| = {err_o:.3e}, max rel dLSE = {err_l:.3e}")
    assert err_o <= O_TOL, (what, err_o)
    assert err_l <= LSE_TOL, (what, err_l)
    return err_o, err_l


def default_scale(d):
    return 1.0 / math.sqrt(d)
