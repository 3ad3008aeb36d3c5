"""Round economics of speculative verify (host arithmetic of bench.py): the
expected-tokens formula against a direct sum over the acceptance process,
the page's printed example, and the break-even solver."""
import math

import pytest

import bench


def _direct(p, k):
    # j drafts accepted then one rejected (j < k), or all k accepted; the
    # verify pass adds one token of its own either way
    probs = [p ** j * (1 - p) for j in range(k)] + [p ** k]
    assert math.isclose(sum(probs), 1.0, rel_tol=1e-12)
    return sum((j + 1) * q for j, q in enumerate(probs))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.65, 0.74, 0.98, 1.0])
def test_expected_tokens_equals_the_direct_sum(p, k):
    assert math.isclose(bench.expected_tokens(p, k), _direct(p, k), rel_tol=1e-12)


def test_page_example():
    """The page prints 1.74 tokens per round at p = 0.74 -- the formula's value
    for one draft (with two drafts it gives 2.29; the example is garbled)."""
    assert round(bench.expected_tokens(0.74, 1), 2) == 1.74
    assert round(bench.expected_tokens(0.74, 2), 2) == 2.29


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("cost", [1.28, 1.6, 2.0])
def test_break_even_solves_the_equation(cost, k):
    p = bench.break_even_acceptance(cost, k)
    if cost >= k + 1:
        assert p is None
        return
    assert 0.0 < p < 1.0
    assert math.isclose(bench.expected_tokens(p, k), cost, rel_tol=1e-10)
    assert bench.expected_tokens(p - 1e-3, k) < cost < bench.expected_tokens(p + 1e-3, k)


def test_break_even_edges():
    assert bench.break_even_acceptance(0.9, 2) == 0.0
    assert bench.break_even_acceptance(3.0, 2) is None
    # one draft: 1 + p = cost
    assert math.isclose(bench.break_even_acceptance(1.28, 1), 0.28, rel_tol=1e-10)
