"""The benchmark's algorithmic byte counts reproduce the per-chunk figures derived from the
definitions (CPU only): Phase 1 is 50 B per K entry, 26 B per Q entry, 4 B per token and the two
dense C x C float32 triangles; DW is the base read and new row written per valid group, each token
row once and a 16-byte record per K entry."""

import bench

# (C, W, R, Phase-1 bytes per chunk) of the five workloads.
P1_PER_CHUNK = [(64, 4, 4, 52480), (128, 16, 16, 287232), (256, 32, 32, 1147904), (256, 8, 8, 680960),
                (256, 32, 32, 1147904)]


def test_phase1_bytes_per_chunk():
    for C, W, R, want in P1_PER_CHUNK:
        assert bench.p1_main_bytes(C, W, R) + bench.p1_pairs_bytes(C) == want


def test_dw_bytes_per_step():
    # Workload 1: P = 8 chunks of C = 128 tokens, W = 16, hd = 128, bf16 bank and token rows.
    groups = 8 * 2015
    total, bank = bench.dw_bytes(groups, 8 * 128, 16, 128, 2, 2)
    assert bank == 2 * groups * 128 * 2
    assert total == bank + 8 * 128 * 128 * 2 + 16 * 8 * 128 * 16


def test_read_side_bytes():
    assert bench.read_gather_bytes(8, 128, 16, 16, 128, 2) == 8 * 128 * 32 * (256 + 8) + 2 * 8 * 128 * 128 * 4
    assert bench.read_solve_bytes(8, 128, 128) == 2 * 8 * 128 * 128 * 4 + 6 * 8 * 128 * 128 * 4 + 8 * 128 * 4


def test_backward_bytes_count_token_rows_once():
    # Workload 1's shape: P = 8, C = 128, W = R = 16, hd = 128, bf16 bank and gradient rows.
    P, C, W, R, hd = 8, 128, 16, 16, 128
    gq = 8 * 2000
    assert bench.gds_bytes(P, C, R, hd, 2, gq, 2) == (P * C * R * (hd * 2 + 12) + P * C * R * 12 + 2 * gq * hd * 2
                                                      + P * C * hd * 4)
    assert bench.gwr_bytes(P, C, W, hd, 2) == P * C * W * (hd * 2 + 12) + 2 * P * C * hd * 4
    g = 8 * 2015
    assert bench.pa_bytes(P, C, W, hd, g, 2, 2) == P * C * W * 36 + g * hd * 8 + P * C * hd * 4
