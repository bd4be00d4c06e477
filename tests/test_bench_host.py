"""Host-side pieces of bench.py that need no GPU: the byte counts the
throughput figures divide by, and the reading of the committed rocprofv3
traffic summary (reported only while it matches the kernel source)."""
import bench


def test_kv_bytes_count_every_attended_byte_once():
    # fp16 K and V: 4 D bytes per position and kv head; int8 V: 2D + D + 2 D/32
    assert bench.kv_bytes([10, 0, 3], 0, 2, 64, False) == 13 * 2 * 256
    assert bench.kv_bytes([10], 4, 2, 64, False) == 4 * 2 * 256
    assert bench.kv_bytes([32768] * 8, 0, 8, 256, True) == 1644167168
    # codebook: 2D + D + 4 bytes per min(D, 256)-dim block
    assert bench.cb_kv_bytes([100], 0, 1, 512, ) == 100 * (1024 + 512 + 8)
    assert bench.cb_kv_bytes([100], 0, 1, 128) == 100 * (256 + 128 + 4)


def test_traffic_summary_is_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY_DIR", str(tmp_path))
    digest = bench.kernel_source_digest()
    body = "# comment line\nkernel_source_sha256_16: {}\nfetch_factor: 2.0\nhbm_bytes_per_launch: 1234567\n"
    (tmp_path / "traffic_wl_w0.txt").write_text(body.format(digest))
    assert bench.read_traffic("wl", 0) == 1234567
    (tmp_path / "traffic_wl_w0.txt").write_text(body.format("0" * 16))
    assert bench.read_traffic("wl", 0) is None
    assert bench.read_traffic("missing", 0) is None


def test_every_committed_profile_is_of_the_current_kernel_source():
    """Each rocprofv3 summary under profiles/ names the digest of the kernel headers it was
    taken on; a summary of other kernels describes code that is no longer built."""
    import glob
    import os
    digest = bench.kernel_source_digest()
    files = sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(bench.__file__)), "profiles", "*")))
    assert files, "no profiles committed"
    stale = [os.path.basename(f) for f in files if digest not in open(f).read()]
    assert not stale, f"profiles taken on other kernel sources (current {digest}): {stale}"


def test_more_than_one_gpu_is_refused_before_any_gpu_work(capsys):
    for n in (2, 8):
        assert bench.main(["--gpus", str(n)]) == 2
        assert f"--gpus {n} is not supported" in capsys.readouterr().err
