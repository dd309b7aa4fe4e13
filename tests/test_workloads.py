"""CPU checks of the bench / test workload bookkeeping against the oracle."""

import itertools

import oracle
import workloads


def test_causal_pair_count_matches_oracle():
    for q0, sq, k0, sk in itertools.product([0, 5, 64, 1000], [1, 7, 64, 130],
                                            [0, 3, 64, 900, 1200], [1, 9, 64, 300]):
        assert workloads.causal_pairs(q0, sq, k0, sk) == \
            oracle.visible_pairs_ref(q0, sq, k0, sk, True), (q0, sq, k0, sk)


def test_workload_flop_counts():
    # zigzag rank 0, cp=4, chunk 1024: 7 FULL + 2 DIAG pairs, 32 heads, d 128
    pairs = sum(workloads.causal_pairs(p * 1024, 1024, kp * 1024, 1024)
                for p in (0, 7) for kp in range(8))
    assert pairs * 32 * 512 == (7 * 1024 ** 2 + 1024 * 1025) * 32 * 512 == 137_455_730_688
    # segmented prefill: 4096 queries at 131072.. over 135168 keys, 128 heads, 192/128
    pairs5 = workloads.causal_pairs(131072, 4096, 0, 135168)
    assert pairs5 == 4096 * 131072 + 4096 * 4097 // 2
    assert abs(pairs5 * 128 * (2 * 192 + 2 * 128) - 4.4668e13) < 1e9
