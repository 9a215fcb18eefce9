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


def test_decode_traffic_summary(tmp_path, capsys):
    """The decode counter summary pairs each shape's second-round launches (plan, then
    matrix-vector) with its counters and trace, scales the bytes by the copy kernel and
    states the weight-read fraction: a synthetic run with known values."""
    import qmm_synth as syn
    shapes = syn.decode_sweep()
    names = []
    for _ in range(2):
        for _ in shapes:
            names += ["w4a16_skinny_kernel<4, 1, 1, 3, 16, 4>", "gemv_kernel<1, 2, 2, 2, 5>", "reduce_vec8"]
    names.append("calib_copy_kernel")
    kib = 1000.0  # every matmul launch: 1000 KiB fetched, 10 KiB written; the copy: half its bytes fetched
    for d, counter, vals in (("f", "FETCH_SIZE", (kib, bench.COPY_BYTES / 2048.0)),
                             ("w", "WRITE_SIZE", (10.0, bench.COPY_BYTES / 1024.0))):
        (tmp_path / d).mkdir()
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        for i, k in enumerate(names):
            rows.append('%d,"%s",%s,%r' % (i + 1, k, counter, vals[1] if "calib_copy" in k else vals[0]))
        (tmp_path / d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    (tmp_path / "t").mkdir()
    rows = ["Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    for i, k in enumerate(names):
        rows.append('%d,"%s",%d,%d' % (i + 1, k, 1000 * i, 1000 * i + 5000))  # 5 us each
    (tmp_path / "t" / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_decode_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t"), ["cmd"])
    out = capsys.readouterr().out.splitlines()
    assert "fetch scale: 2.0000" in out and "write scale: 1.0000" in out
    body = [l.split() for l in out if l.split() and l.split()[0] in ("down", "gate")]
    assert len(body) == 2 * len(shapes)
    for (name, M, N, K, _), plan, mv in zip(shapes, body[0::2], body[1::2]):
        assert plan[4] == "plan" and mv[4] == "matvec" and plan[:4] == [name, str(M), str(N), str(K)]
        b = 2 * kib * 1024 + 10 * 1024
        assert abs(float(plan[5]) - 2 * kib * 1024) / b < 1e-3 and abs(float(plan[9]) - 5.0) < 1e-9
        assert abs(float(plan[10]) - b / 5000) < 0.1  # GB/s = bytes per ns
        wbytes = N * K // 2 + N * (K // 128) * 4
        assert abs(float(plan[11]) - wbytes / 5000 / 8000) < 1e-3
