"""bench.py's host-side helpers, checked on the CPU: the HBM traffic figure is
taken from a counter summary only while that summary's kernel source hash
matches the source, and the CPU-baseline sample holds the row sets its
docstring lists, with the useful-FLOP count of exactly those rows."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workload import by_name, custom, outlier_rows  # noqa: E402


def _setup(tmp_path, monkeypatch, src_text, sha):
    src = tmp_path / "hier_attn.hip"
    src.write_text(src_text)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hier_attn_4k-latent_pmc.json").write_text(json.dumps(
        {"kernel_source_sha256": sha, "hbm_bytes_per_launch": 1.25e11}))
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    return src


def test_traffic_read_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    import hashlib
    text = "// kernel source\n"
    sha = hashlib.sha256(text.encode()).hexdigest()
    src = _setup(tmp_path, monkeypatch, text, sha)
    assert bench.pmc_traffic("4k-latent") == 1.25e11
    assert bench.pmc_traffic("720p-latent") is None          # no summary for that workload
    src.write_text(text + "// edited\n")                     # the kernel changed since
    assert bench.pmc_traffic("4k-latent") is None


def test_traffic_of_an_unreadable_summary_is_none(tmp_path, monkeypatch):
    _setup(tmp_path, monkeypatch, "x", "0" * 64)
    (tmp_path / "profiles" / "hier_attn_4k-latent_pmc.json").write_text("{not json")
    assert bench.pmc_traffic("4k-latent") is None


def test_committed_summaries_name_their_source():
    for w in ("4k-latent", "8k-latent"):
        with open(os.path.join(ROOT, "profiles", f"hier_attn_{w}_pmc.json")) as f:
            d = json.load(f)
        assert len(d["kernel_source_sha256"]) == 64
        assert d["kernel_source"].endswith("hier_attn.hip")
        assert d["hbm_bytes_per_launch"] > d["algorithmic_bytes_per_launch"] > 0


def _check_sample(cfg, seed):
    rng = np.random.default_rng(seed)
    (rows, heads, glob), flops = bench.oracle_sample(cfg, rng)
    N, V, G, H = cfg.N, cfg.V, cfg.G, cfg.heads
    det = glob == 0
    assert rows.shape == heads.shape == glob.shape
    assert np.all((rows[det] >= 0) & (rows[det] < N)) and np.all((rows[~det] >= 0) & (rows[~det] < G))
    assert np.all((heads >= 0) & (heads < H))
    assert int((~det).sum()) == min(1024, G)
    # every row of the first and the last window, in head 0 and in head H - 1
    for h in (0, H - 1):
        for c in (0, cfg.C - 1):
            want = np.arange(c * V, (c + 1) * V)
            got = rows[det & (heads == h)]
            assert np.isin(want, got).all()
    n_d = int(det.sum())
    assert flops == 4.0 * cfg.head_dim * (n_d * (V + G) + int((~det).sum()) * G)
    return rows[det], heads[det]


def test_cpu_sample_row_sets():
    cfg = custom("s", (6, 34, 48), (3, 17, 24), (3, 15, 26), heads=6, head_dim=128)
    for seed in range(4):
        rows, _ = _check_sample(cfg, seed)
        # up to 4 windows x 4 heads of whole windows (first and last of each,
        # two random picks that may repeat them), then 4,096 random rows
        k, r = divmod(rows.size - 4096, cfg.V)
        assert r == 0 and 4 <= k <= 16


def test_cpu_sample_takes_the_outlier_queries():
    cfg = by_name("4k-latent")
    assert cfg.outliers
    rows, heads = _check_sample(cfg, 1)
    orows = np.nonzero(outlier_rows(cfg.seed, 0, cfg.N))[0]
    assert orows.size > 1024
    # 1,024 outlier query rows are added on top of the window and random rows
    k, r = divmod(rows.size - 4096 - 1024, cfg.V)
    assert r == 0 and 4 <= k <= 16
    assert np.isin(rows[-1024:], orows).all()
