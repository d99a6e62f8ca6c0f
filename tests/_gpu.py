"""Helpers shared by the GPU parity tests: host <-> device transfers of
boundary arrays, error metrics and the tolerances the tests enforce.

Tolerances (written here, used by every attention test):
  * attention: max |gpu - oracle| <= 2e-2 and ||gpu - oracle||_2 / ||oracle||_2
    <= 5e-3 per output tensor (detail and global separately);
  * RoPE, bf16: the output bit pattern is RNE(oracle) or one of its two bf16
    neighbours (<= 1 ulp), except where the rotation cancels to a value far
    below its inputs: fp32 arithmetic carries an absolute error floor of a few
    2^-24 of the pair's norm, so there the bound is |gpu - oracle| <= 2^-20 *
    |(x0, x1)| (the pair norm, which the rotation preserves); fp32:
    |gpu - oracle| <= 1e-5 * max|x|;
  * reorder / unorder: bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
ROPE_F32_REL = 1e-5
ROPE_ABS_FLOOR = 2.0 ** -20


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev(a):
    """numpy boundary array (uint16 = bf16 bits, float32) -> GPU tensor."""
    if a is None:
        return None
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).to("cuda").view(t.bfloat16)
    return t.from_numpy(a).to("cuda")


def host(x):
    """GPU tensor -> numpy boundary array (bf16 as uint16 bits)."""
    if x is None:
        return None
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def host_rows(x, rows):
    """Selected token rows of a GPU tensor, as a numpy boundary array."""
    t = torch()
    idx = t.as_tensor(np.asarray(rows, dtype=np.int64), device=x.device)
    return host(x.index_select(0, idx))


def attn_errors(gpu, ref):
    g = oracle.to_f64(gpu) if gpu.dtype != np.float64 else gpu
    err = g - ref
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def assert_attn_close(gpu, ref, what):
    max_abs, rel = attn_errors(gpu, ref)
    say(f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(oracle.to_f64(gpu))), f"{what}: non-finite output"
    assert max_abs <= ATTN_MAX_ABS, f"{what}: max abs {max_abs} > {ATTN_MAX_ABS}"
    assert rel <= ATTN_REL_L2, f"{what}: rel L2 {rel} > {ATTN_REL_L2}"


def _ordered(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_rope_close(gpu, ref_f64, what):
    """gpu: boundary array after the GPU RoPE; ref_f64: oracle rotation (fp64)."""
    if gpu.dtype == np.uint16:
        want = oracle.round_bf16(ref_f64)
        ulps = np.abs(_ordered(gpu) - _ordered(want))
        pair = np.sqrt(ref_f64[..., 0::2] ** 2 + ref_f64[..., 1::2] ** 2)
        pair = np.repeat(pair, 2, axis=-1)
        abs_err = np.abs(oracle.to_f64(gpu) - ref_f64)
        far = ulps > 1
        floor_ok = abs_err <= ROPE_ABS_FLOOR * pair
        n_exact = int(np.sum(ulps == 0))
        # the largest error beyond 1 ulp as a multiple of its floor (< 1 passes)
        worst = float(np.max(abs_err[far] / (ROPE_ABS_FLOOR * pair[far]))) if far.any() else 0.0
        say(f"{what}: max ulp={int(ulps.max()) if ulps.size else 0} exact={n_exact}/{ulps.size} "
            f">1ulp={int(far.sum())} (all within the cancellation floor: {bool(floor_ok[far].all())}; "
            f"largest such error = {worst:.3f} x the floor)")
        bad = far & ~floor_ok
        assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 1 ulp and the floor"
    else:
        err = np.abs(gpu.astype(np.float64) - ref_f64).max()
        bound = ROPE_F32_REL * np.abs(ref_f64).max()
        say(f"{what}: max err={err:.3e} bound={bound:.3e}")
        assert err <= bound
