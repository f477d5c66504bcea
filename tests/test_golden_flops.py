"""The FLOP count the bench reports (6 * slots * hidden * inter: two GEMMs of
2*H*I*2 flops for gate/up and one of 2*I*H for down, per routed slot) against
the figures printed in the aiter issue's "Estimated Performance Scaling" table
(tests/golden/aiter_issue_table.txt)."""
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def test_flop_count_reproduces_printed_tflops():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "aiter_issue_table.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        experts, tpe, inter, hidden = (int(v) for v in r[:4])
        us, tflops = float(r[7]), float(r[8])
        flops = bench.layer_flops(experts * tpe, hidden, inter)
        assert abs(flops / (us * 1e-6) / 1e12 - tflops) < 0.01 * tflops
    # the measured row to the printed precision
    assert round(bench.layer_flops(2048, 7168, 2048) / 484e-6 / 1e12, 2) == 372.70
