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
