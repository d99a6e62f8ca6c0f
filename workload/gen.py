"""Seeded, block-wise, reproducible input generation.

Recipe (the same for the tests, the smoke check and the bench):
  * tensor ids: q_d=0, k_d=1, v_d=2, q_g=3, k_g=4, v_g=5; detail tensors are
    [N, heads, D] in RASTER order, global tensors [G, heads, D] in raster
    order over the proxy grid;
  * fp32 workloads: one ``numpy.random.default_rng(seed)`` stream drawing
    ``standard_normal`` float32 for q_d, k_d, v_d, q_g, k_g, v_g in that order;
  * bf16 workloads: token block b (4096 tokens) of tensor id draws
    ``standard_normal`` float32 from
    ``default_rng(SeedSequence(seed, spawn_key=(id, b)))``, then rounds to
    bf16 (nearest, ties to even) by integer arithmetic on the bit patterns;
  * outlier workloads: token row r of q_d, k_d, q_g, k_g is multiplied by 8
    (exact) when ``splitmix64(seed ^ (id << 40) ^ r) % 100 == 0``; v is never
    scaled.
bf16 tensors are returned as uint16 arrays of raw bit patterns.
"""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"q_d": 0, "k_d": 1, "v_d": 2, "q_g": 3, "k_g": 4, "v_g": 5,
              "do_d": 6, "do_g": 7}
OUTLIER_IDS = (0, 1, 3, 4)
BLOCK_TOKENS = 4096
_M64 = (1 << 64) - 1


def splitmix64(x):
    """SplitMix64 output function (Steele, Lea, Flood 2014), vectorised."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def outlier_rows(seed: int, tensor_id: int, n_rows: int) -> np.ndarray:
    """Boolean mask of the token rows scaled by 8 (about 1%)."""
    key = np.uint64((seed ^ (tensor_id << 40)) & _M64)
    r = np.arange(n_rows, dtype=np.uint64)
    return (splitmix64(key ^ r) % np.uint64(100)) == 0


def bf16_bits_from_f32(x: np.ndarray, out: np.ndarray | None = None,
                       scratch: np.ndarray | None = None) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs).

    Textbook integer rounding on the fp32 pattern: add 0x7FFF plus the lowest
    kept bit, keep the high 16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).reshape(-1)
    t = np.empty_like(u) if scratch is None else scratch.reshape(-1)[: u.size]
    np.right_shift(u, np.uint32(16), out=t)
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(t, u, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    if out is None:
        out = np.empty(x.shape, dtype=np.uint16)
    np.copyto(out.reshape(-1), t, casting="unsafe")
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_tls = threading.local()


def _scratch(n: int) -> np.ndarray:
    """Per-thread uint32 buffer reused across blocks (avoids fresh page faults)."""
    buf = getattr(_tls, "buf", None)
    if buf is None or buf.size < n:
        buf = np.empty(n, dtype=np.uint32)
        _tls.buf = buf
    return buf[:n]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen_tensor(cfg, name: str, n_tokens: int | None = None) -> np.ndarray:
    """One bf16 input tensor of a bf16 workload, [n_tokens, heads, D] uint16."""
    if cfg.dtype != "bf16":
        raise ValueError("gen_tensor is the block scheme of bf16 workloads")
    tid = TENSOR_IDS[name]
    if n_tokens is None:
        n_tokens = cfg.N if name.endswith("_d") else cfg.G
    row = cfg.heads * cfg.head_dim
    out = np.empty((n_tokens, cfg.heads, cfg.head_dim), dtype=np.uint16)
    flat = out.reshape(n_tokens, row)
    nblk = (n_tokens + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    scale_rows = outlier_rows(cfg.seed, tid, n_tokens) if (cfg.outliers and tid in OUTLIER_IDS) else None

    def work(b):
        t0 = b * BLOCK_TOKENS
        t1 = min(n_tokens, t0 + BLOCK_TOKENS)
        rng = np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=(tid, b)))
        x = rng.standard_normal((t1 - t0) * row, dtype=np.float32).reshape(t1 - t0, row)
        if scale_rows is not None:
            m = scale_rows[t0:t1]
            if m.any():
                x[m] *= np.float32(8.0)
        bf16_bits_from_f32(x, out=flat[t0:t1], scratch=_scratch(x.size))

    if nblk <= 1:
        for b in range(nblk):
            work(b)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def gen_inputs(cfg) -> dict:
    """All six inputs of a workload: dict name -> array (None for G = 0)."""
    N, G, h, D = cfg.N, cfg.G, cfg.heads, cfg.head_dim
    names = ("q_d", "k_d", "v_d", "q_g", "k_g", "v_g")
    if cfg.dtype == "f32":
        rng = np.random.default_rng(cfg.seed)
        out = {}
        for nm in names:
            n = N if nm.endswith("_d") else G
            if n == 0:
                out[nm] = None
                continue
            x = rng.standard_normal(n * h * D, dtype=np.float32).reshape(n, h, D)
            if cfg.outliers and nm in ("q_d", "k_d", "q_g", "k_g"):
                x[outlier_rows(cfg.seed, TENSOR_IDS[nm], n)] *= np.float32(8.0)
            out[nm] = x
        return out
    out = {}
    for nm in names:
        n = N if nm.endswith("_d") else G
        out[nm] = gen_tensor(cfg, nm, n) if n else None
    return out


def gen_grad_outputs(cfg) -> dict:
    """Upstream gradients of the attention outputs: do_d [N, heads, D] and
    do_g [G, heads, D] (None for G = 0), standard normal, never scaled."""
    N, G, h, D = cfg.N, cfg.G, cfg.heads, cfg.head_dim
    out = {}
    for nm in ("do_d", "do_g"):
        n = N if nm.endswith("_d") else G
        if n == 0:
            out[nm] = None
        elif cfg.dtype == "f32":
            rng = np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=(TENSOR_IDS[nm],)))
            out[nm] = rng.standard_normal(n * h * D, dtype=np.float32).reshape(n, h, D)
        else:
            out[nm] = gen_tensor(cfg, nm, n)
    return out
