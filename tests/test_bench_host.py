"""Host-side tests of bench.py's bookkeeping (no GPU): the digest that ties a counter
summary under profiles/ to the kernel sources it was taken on (code only, so that an
edited comment does not void the summary, while any code change does), the traffic
read-back that follows it, the roofline arithmetic, and the one-GPU contract."""
import bench


def _digest_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.source_digest([str(p)])


def test_digest_ignores_comments_and_whitespace(tmp_path):
    code = "__global__ void k(int *p) {\n    p[0] = 1;  // store\n}\n"
    base = _digest_of(tmp_path, code)
    assert _digest_of(tmp_path, "// a header comment\n" + code) == base
    assert _digest_of(tmp_path, code.replace("// store", "// the only store")) == base
    assert _digest_of(tmp_path, code.replace("    p[0]", "p[0]")) == base
    assert _digest_of(tmp_path, "/* block\n comment */" + code) == base


def test_digest_follows_code(tmp_path):
    code = "__global__ void k(int *p) {\n    p[0] = 1;\n}\n"
    base = _digest_of(tmp_path, code)
    assert _digest_of(tmp_path, code.replace("p[0] = 1", "p[0] = 2")) != base
    assert _digest_of(tmp_path, code.replace("p[0]", "p[1]")) != base


def test_roofline_of_two_regimes():
    # k at M = 16: bytes-bound (1024*2560/2 packed + 1024*20*4 scale/bias + 2*16*2560 A
    # + 2*16*1024 C = 1,507,328 bytes: 0.188 us at 8 TB/s); q at M = 2048: flop-bound
    # (2*2048*4096*2560 = 4.29e10 flop: 17.18 us at 2.5 PFLOP/s)
    assert bench.algorithmic_bytes(16, 1024, 2560) == 1310720 + 81920 + 81920 + 32768
    r = bench.roofline(16, 1024, 2560, 1.884e-6)
    assert r["bound"] == "hbm" and abs(r["t_roof_us"] - 0.188416) < 1e-6 and abs(r["frac"] - 0.1) < 1e-3
    r = bench.roofline(2048, 4096, 2560, 34.36e-6)
    assert r["bound"] == "mfma" and abs(r["t_roof_us"] - 17.179869) < 1e-5 and abs(r["frac"] - 0.5) < 1e-3
    # another format's own bytes: 8-bit codes, groups of 32
    assert bench.algorithmic_bytes(1, 64, 256, bits=8, group=32) == 64 * 256 + 64 * 8 * 4 + 2 * 256 + 2 * 64


def test_traffic_read_back_follows_the_digest(tmp_path, monkeypatch):
    # the committed summary's figure when its digest matches the sources, else None
    good = tmp_path / "traffic.txt"
    good.write_text("# summary\nkernel source digest: %s\nhbm bytes per launch (scaled): 1.5e+08\n"
                    % bench.source_digest())
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(good))
    t, note = bench.read_traffic(5e7)
    assert t == 1.5e8 and "3.00x" in note
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel source digest: 0000000000000000\nhbm bytes per launch (scaled): 1.5e+08\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(stale))
    assert bench.read_traffic(5e7)[0] is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.read_traffic(5e7)[0] is None


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
