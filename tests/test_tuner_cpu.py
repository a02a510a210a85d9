"""The tile-table tuner's host logic (routed_grouped_gemm_amd.tune), without a GPU: the choice
of a winner per M, the bucket rules built from the winners, and the header it writes, read
back and checked against the compiled-in table's form."""
import math
import re

from routed_grouped_gemm_amd import tune


def test_choose_takes_the_fastest_only_when_clearly_faster():
    cand = {(32, 1): 100.0, (64, 1): 99.0, (64, 4): 97.0, (128, 4): 120.0}
    # 97 is more than 2 % faster than the previous winner (32, 1): taken
    assert tune.choose(cand, 16, (32, 1), (32, 1)) == (64, 4)
    # within 2 % of the previous winner: the previous winner stays
    cand2 = {**cand, (64, 4): 98.5}
    assert tune.choose(cand2, 16, (32, 1), (128, 4)) == (32, 1)
    # no previous winner: the table's choice stays when within 2 %
    assert tune.choose(cand2, 16, None, (64, 1)) == (64, 1)
    # the m-tile never shrinks below the floor, even when a smaller one is faster
    assert tune.choose(cand, 64, None, (128, 4)) == (64, 4)
    assert tune.choose({(16, 4): 10.0, (128, 4): 50.0}, 128, None, (16, 4)) == (128, 4)


def _results(pairs):
    return [dict(T=T, mean_rows=m, best=b) for T, m, b in pairs]


def test_rules_merge_runs_and_split_at_geometric_means():
    res = _results([(16, 0.5, (16, 4)), (64, 2.0, (16, 4)), (256, 8.0, (64, 1)), (1024, 32.0, (64, 1)),
                    (4096, 128.0, (160, 4))])
    rules = tune.rules_from(res, 160)
    assert rules == [(math.sqrt(2.0 * 8.0), 16, 4), (math.sqrt(32.0 * 128.0), 64, 1), (1e30, 160, 4)]
    # the largest tile is capped at the row list's maximum
    assert tune.rules_from(_results([(1, 1.0, (160, 1))]), 128) == [(1e30, 128, 1)]


def test_header_round_trip(tmp_path):
    table = {"f32": [(4.0, 16, 4), (1e30, 160, 4)], "bf16": [(4.0, 16, 4), (1e30, 160, 4)],
             "fp8": [(2.0, 16, 4), (20.0, 32, 1), (1e30, 128, 4)],
             "fp8a": [(0.5, 16, 4), (1e30, 160, 1)]}
    path = tmp_path / "moe_tuned.h"
    tune.write_header(str(path), table, ["test"])
    text = path.read_text()
    assert "constexpr int kNumTileRules = 3;" in text
    assert "kTileRules[4][kNumTileRules]" in text
    rows = re.findall(r"// (\w+)\n    \{(.*)\},", text)
    assert [r[0] for r in rows] == list(tune.ROWS)
    fp8 = re.findall(r"\{([0-9.e+]+)f, (\d+), (\d+)\}", rows[2][1])
    assert [(float(b), int(r), int(g)) for b, r, g in fp8] == [(2.0, 16, 4), (20.0, 32, 1), (1e30, 128, 4)]
    # shorter rule lists are padded with their last rule
    fp8a = re.findall(r"\{([0-9.e+]+)f, (\d+), (\d+)\}", rows[3][1])
    assert len(fp8a) == 3 and fp8a[-1] == fp8a[-2]


def test_compiled_in_table_has_the_tuner_form():
    import os
    src = open(os.path.join(os.path.dirname(tune.__file__), "csrc", "moe_tuned.h")).read()
    n = int(re.search(r"kNumTileRules = (\d+);", src).group(1))
    rows = re.findall(r"// (\w+)\n    \{(.*)\},", src)
    assert [r[0] for r in rows] == list(tune.ROWS)
    for name, body in rows:
        rules = [(float(b), int(r), int(g)) for b, r, g in re.findall(r"\{([0-9.e+]+)f, (\d+), (\d+)\}", body)]
        assert len(rules) == n
        bounds = [b for b, _, _ in rules]
        assert bounds == sorted(bounds) and bounds[-1] >= 1e29
        assert all(r in (16, 32, 64, 128, 160) and 1 <= g <= 64 for _, r, g in rules)
        assert [r for _, r, _ in rules] == sorted(r for _, r, _ in rules)
