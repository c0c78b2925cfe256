"""The CPU lane models against plain definitions (no GPU)."""
import math
import random

from lane_models import WAVE, add, dpp_reduce, max_rule, shfl_down


def test_dpp_reduce_model_is_a_reduction():
    rng = random.Random(5)
    for _ in range(50):
        ints = [rng.randint(-2 ** 40, 2 ** 40) for _ in range(WAVE)]
        assert dpp_reduce(ints, add, 0) == sum(ints)          # exact on integers
        fl = [rng.uniform(-1e3, 1e3) for _ in range(WAVE)]
        assert dpp_reduce(fl, max_rule, -math.inf) == max(fl)
        assert abs(dpp_reduce(fl, add, 0.0) - math.fsum(fl)) <= 64 * 2 ** -52 * sum(map(abs, fl))
    # Each lane contributes exactly once: tags 2^i sum to 2^64 - 1.
    assert dpp_reduce([2 ** i for i in range(WAVE)], add, 0) == 2 ** WAVE - 1


def test_shfl_down_model():
    v = list(range(WAVE))
    assert shfl_down(v, 0) == v
    assert shfl_down(v, 1)[:63] == list(range(1, 64)) and shfl_down(v, 1)[63] == 63
    s = shfl_down(v, 32)
    assert s[:32] == list(range(32, 64)) and s[32:] == list(range(32, 64))
    assert shfl_down(v, 64) == v
