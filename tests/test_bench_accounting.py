"""bench.py's algorithmic work counts agree with the oracle's brute-force accounting
and with the numbers the workloads imply."""
import oracle
import bench
from workloads import CONFIGS


def test_prefill_flops_match_oracle_accounting():
    for name in ("C1", "C2", "C3", "C4"):
        c = CONFIGS[name]
        pairs = sum(oracle.visible_pairs_partition(c.Sp, c.P, i, c.causal)
                    for i in range(c.q_part0, c.q_part0 + c.n_qparts))
        assert bench.prefill_flops(c) == oracle.attention_flops(pairs, c.Hq * c.B, c.Dqk, c.Dv)
    # causal aligned sequences count S(S+1)/2 pairs per head
    c2 = CONFIGS["C2"]
    assert bench.prefill_flops(c2) == 2 * 256 * c2.Hq * oracle.visible_pairs_aligned_causal(c2.S)
    assert abs(bench.prefill_flops(CONFIGS["C3"]) - 2.8148e14) / 2.8148e14 < 1e-4
    assert abs(bench.prefill_flops(CONFIGS["C4"]) - 2.6388e15) / 2.6388e15 < 1e-4


def test_partition_pairs_match_oracle_accounting():
    for layout in ("contiguous", "striped"):
        for causal in (False, True):
            for P, Sp in ((1, 5), (3, 7), (8, 16384), (8, 65536)):
                for i in range(P):
                    assert bench.partition_pairs(Sp, P, i, causal, layout) == \
                        oracle.visible_pairs_partition(Sp, P, i, causal, layout)
    # the last partition of C3 does 1.875x the pairs of its striped counterpart
    c = CONFIGS["C3"]
    r = bench.partition_pairs(c.Sp, c.P, 7, True, "contiguous") / bench.partition_pairs(c.Sp, c.P, 7, True, "striped")
    assert abs(r - 1.875) < 1e-3


def test_backward_flops():
    # five products per visible pair: 2 (3 Dqk + 2 Dv); 2.5x the forward at Dqk = Dv
    c = CONFIGS["C3"]
    assert bench.backward_flops(c) * 2 == bench.prefill_flops(c) * 5
    c4 = CONFIGS["C4"]
    pairs = bench.prefill_flops(c4) // (2 * (192 + 128))
    assert bench.backward_flops(c4) == pairs * 2 * (3 * 192 + 2 * 128)


def test_decode_bytes():
    c = CONFIGS["C5"]
    kv = oracle.kv_cache_bytes(layers=1, h_kv=c.Hkv, d_h=c.Dqk, n=c.L, bytes_per_value=2, batch=c.B)
    assert kv == 8_589_934_592
    assert bench.decode_partial_bytes(c) > kv
    assert bench.decode_partial_bytes(c) - kv < 5e6


def test_recorded_profiles_parse():
    """profiles/traffic.txt and profiles/sclk.txt hold a row per (kernel, workload)
    that the bench line reports on; bench.py uses a row only while its source hash
    matches the kernel source, so every row carries a 16-digit hash and sane values."""
    rows = {}
    for path, nvals in ((bench.TRAFFIC_FILE, 2), (bench.SCLK_FILE, 1)):
        with open(path) as f:
            for line in f:
                parts = line.split("#", 1)[0].split()
                if not parts:
                    continue
                assert len(parts) == 3 + nvals, line
                kind, wl, sha = parts[:3]
                assert len(sha) == 16 and int(sha, 16) >= 0, line
                vals = [float(x) for x in parts[3:]]
                rows[(path, kind, wl)] = vals
    for wl in ("C4", "C3"):
        fetch, write = rows[(bench.TRAFFIC_FILE, "prefill", wl)]
        assert fetch > write > 0
        (ghz,) = rows[(bench.SCLK_FILE, "prefill", wl)]
        assert 1.0 < ghz < 2.5
    for wl in ("C5", "C5F"):
        assert (bench.TRAFFIC_FILE, "decode", wl) in rows


def test_recorded_ignores_other_sources(tmp_path):
    sha = bench.source_sha("prefill")
    f = tmp_path / "t.txt"
    f.write_text("# comment\nprefill C4 0000000000000000 1.0 2.0\n"
                 f"prefill C4 {sha} 3.0 4.0   # trailing comment\nprefill C3 {sha} 5.0\n")
    assert bench.recorded(str(f), "prefill", "C4", 2) == [3.0, 4.0]
    assert bench.recorded(str(f), "prefill", "C3", 2) is None      # wrong field count
    assert bench.recorded(str(f), "decode", "C4", 2) is None


def test_mfma_peak_per_clock():
    # 256 CUs x 4 SIMDs x 32768 FLOP per 32-cycle 32x32x16 product, at 2.4 GHz
    assert abs(bench.MFMA_BF16_FLOP_PER_CLK * 2.4e9 / 1e12 - 2516.58) < 0.01
    assert bench.PEAK_BF16_TFLOPS == 2500.0


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_guarded_records_a_failure_in_place():
    assert bench.guarded("ok", lambda a, b: a + b, 2, 3) == 5
    r = bench.guarded("fails", lambda: {}["missing"])
    assert r == {"error": "KeyError: 'missing'"}


def test_launch_stats():
    """min / median / max of the per-launch times, odd and even counts."""
    assert bench.launch_stats([3.0, 1.0, 2.0]) == {"min": 1.0, "median": 2.0, "max": 3.0, "n": 3}
    assert bench.launch_stats([4.0, 1.0, 2.0, 3.0]) == {"min": 1.0, "median": 2.5, "max": 4.0, "n": 4}
