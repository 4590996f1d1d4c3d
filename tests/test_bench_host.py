"""Host-side checks of bench.py: the one-GPU guard and the algorithmic
byte and flop counts it reports (the per-config figures of the scope table)."""
import math

import pytest

import bench
from workloads import CONFIGS


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name,nbytes", [("C1", 131_328), ("C2", 125_841_408), ("C3", 1_207_971_840),
                                         ("C4", 8_589_938_688), ("C5a", 5_905_604_608), ("C5b", 4_505_624_576)])
def test_algorithmic_bytes(name, nbytes):
    assert bench.min_bytes(CONFIGS[name]) == nbytes


@pytest.mark.parametrize("name,per_token", [("C2", 254), ("C3", 354), ("C4", 434), ("C5a", 561)])
def test_algorithmic_flops_per_token(name, per_token):
    c = CONFIGS[name]
    assert round(bench.algo_flops(c) / (c.B * c.D * c.L)) == per_token
    assert bench.algo_flops(c) == c.N * c.B * c.D * c.L * (10 * math.log2(2 * c.L) + 7)
