"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the graph
length divisor, the visible-key count per query row, and the parity summary
of timed outputs against the oracle."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import NAMED, make_batch  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("steps,cap", [(1, 100), (7, 100), (100, 100), (500, 100), (2000, 100), (50, 20), (97, 100)])
def test_graph_length_divides_the_steps(steps, cap):
    g = bench._graph_len(steps, cap)
    assert 1 <= g <= min(steps, cap) and steps % g == 0
    assert all(steps % d for d in range(g + 1, min(steps, cap) + 1))


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 5)])
def test_visible_keys_match_a_brute_force_mask(causal, window):
    """visible_keys (used for the CPU sample's FLOPs and the error bands)
    against the causal bottom-right mask written out key by key (a window
    needs the causal mask)."""
    b = make_batch(11, [1, 4, 9, 1], [7, 4, 20, 33], Hq=2, Hkv=1, D=64, dtype="fp32", causal=causal,
                   window=window, name="vis")
    rows = np.arange(b.T)
    got = bench.visible_keys(b, rows)
    for r in rows:
        s = int(np.searchsorted(b.cu_seqlens_q, r, side="right") - 1)
        i = r - int(b.cu_seqlens_q[s])
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        pos = lk - lq + i   # the row's position among the keys (decode rows: lk - 1)
        n = 0
        for j in range(lk):
            vis = j <= pos if causal else True
            if window:
                vis = vis and j > pos - window
            n += vis
        assert got[r] == n, (r, got[r], n)


def test_parity_summary():
    b = NAMED["tiny_varlen_fp32"]()
    rows = np.arange(b.T)
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((b.T, b.Hq, b.D))
    lse = rng.standard_normal((b.T, b.Hq))
    ok = bench._parity(rows, ref, lse, ref + 1e-6, lse, 1e-5, b)
    assert ok["ok"] and ok["rows"] == b.T
    assert ok["cosine_out"] == pytest.approx(1.0, abs=1e-9)
    assert ok["rel_l2_out"] == pytest.approx(1e-6 * np.sqrt(ref.size) / np.linalg.norm(ref), rel=1e-6)
    assert max(ok["max_abs_out_by_visible_keys"].values()) == pytest.approx(ok["max_abs_out"])
    bad = ref.copy()
    bad[3, 1, 5] += 0.5
    r = bench._parity(rows, ref, lse, bad, lse, 1e-5, b)
    assert not r["ok"] and r["max_abs_out"] == pytest.approx(0.5)
    nan = ref.copy()
    nan[0, 0, 0] = np.nan
    assert not bench._parity(rows, ref, lse, nan, lse, 1e-5)["ok"]


def test_commit_read_from_git_files(tmp_path, monkeypatch):
    """_git_head reads the checked-out commit from .git (loose ref, packed ref,
    detached head) without starting git, and gives None without a .git."""
    sha = "0123456789abcdef0123456789abcdef01234567"
    g = tmp_path / ".git"
    (g / "refs" / "heads").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (g / "HEAD").write_text("ref: refs/heads/main\n")
    (g / "refs" / "heads" / "main").write_text(sha + "\n")
    assert bench._git_head() == sha[:7]
    (g / "refs" / "heads" / "main").unlink()
    (g / "packed-refs").write_text("# pack-refs with: peeled\n" + sha + " refs/heads/main\n")
    assert bench._git_head() == sha[:7]
    (g / "HEAD").write_text(sha + "\n")
    assert bench._git_head() == sha[:7]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "none"))
    assert bench._git_head() is None


def test_dpm_clocks_never_raise():
    """The clock levels come from sysfs files (None where there are none)."""
    c = bench._dpm_clocks()
    assert c is None or (isinstance(c, dict) and all(isinstance(v, dict) for v in c.values()))
