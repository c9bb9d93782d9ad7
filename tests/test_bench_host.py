"""Host logic of bench.py, on the CPU: the one-GPU guard, and the rule that a
profile summary's HBM traffic is reported only while the kernel source it was
taken from is unchanged (its SHA-256 prefix matches)."""
import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _fake_tree(tmp_path, src_text, recorded_sha, nbytes="1.234500e+08"):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(src_text)
    (tmp_path / "profiles" / "s.md").write_text(
        f"# summary\n\nhbm_bytes_per_launch: {nbytes}\nsource_sha256_16: {recorded_sha}\n")


def test_traffic_reported_while_source_unchanged(tmp_path, monkeypatch):
    src = "kernel source v1\n"
    sha = hashlib.sha256(src.encode()).hexdigest()[:16]
    _fake_tree(tmp_path, src, sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic("s.md", "k.hip") == 1.2345e8


def test_traffic_null_once_source_changes(tmp_path, monkeypatch):
    old = hashlib.sha256(b"kernel source v1\n").hexdigest()[:16]
    _fake_tree(tmp_path, "kernel source v2\n", old)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic("s.md", "k.hip") is None
    assert bench._traffic("missing.md", "k.hip") is None


def test_committed_summaries_name_their_kernel_source():
    """Every committed PMC summary the bench reads records a source hash."""
    for summary in ("fa_fwd_trading_day_bf16_pmc.md", "fa_decode_gqa_bf16_pmc.md"):
        txt = open(os.path.join(ROOT, "profiles", summary)).read()
        assert "source_sha256_16:" in txt and "hbm_bytes_per_launch:" in txt


def test_ceiling_library_builds_and_exports_its_launchers():
    """The bench's attainable-ceiling kernels (bench_ceilings.hip) build for
    gfx950 and export the launchers bench.py binds (no launch here)."""
    import ctypes

    import __graft_entry__
    path = __graft_entry__.build_ceilings()
    lib = ctypes.CDLL(path)
    for name in ("ceil_read_chunks_launch", "ceil_read_stride_launch", "ceil_mfma_launch",
                 "ceil_mfma_mix_launch", "ceil_mfma_mix_variant_launch"):
        assert hasattr(lib, name), name
