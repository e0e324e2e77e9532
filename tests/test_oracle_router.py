"""Pins of the oracle's router logits and routing chain (oracle/router.py)
against integer arithmetic, an fp64 matrix product and exact invariants."""
import numpy as np
import pytest

from oracle.router import route_from_hidden, router_logits
from oracle.routing import route


def test_integer_inputs_give_the_integer_product():
    """Small integers: every logit is an exact integer; T, D and E all differ,
    so a transposed operand or a wrong index cannot pass."""
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, (3, 40)).astype(np.float32)
    w = rng.integers(-8, 9, (7, 40)).astype(np.float32)
    want = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(router_logits(x, w), want.astype(np.float32))


@pytest.mark.parametrize("D", [64, 2048])
def test_logits_are_the_rounded_exact_product(D):
    """Each logit is the fp32 value nearest the exact dot product: within half
    an fp32 ulp of the fp64 product (itself within D * 2^-53 of exact)."""
    rng = np.random.default_rng(D)
    x = rng.standard_normal((5, D)).astype(np.float32)
    w = (rng.standard_normal((9, D)) * 0.02).astype(np.float32)
    got = router_logits(x, w).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    ulp = np.spacing(np.abs(got).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp + D * 2.0 ** -52 * np.abs(x).max() * np.abs(w).max())


@pytest.mark.parametrize("k", [-7, 3])
def test_power_of_two_weight_scaling(k):
    """A folded output multiplier of 2^k scales every logit by 2^k exactly."""
    rng = np.random.default_rng(abs(k))
    x = rng.standard_normal((4, 128)).astype(np.float32)
    w = rng.standard_normal((6, 128)).astype(np.float32)
    a = router_logits(x, w)
    b = router_logits(x, (w * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(b, (a * np.float32(2.0 ** k)).astype(np.float32))


def test_chain_with_a_selection_weight_routes_the_selected_inputs():
    """w = 2 * [I_E | 0]: the logits are 2 * x[:, :E] exactly, and the chain's
    ids and weights are those of the routing on them."""
    rng = np.random.default_rng(5)
    T, D, E, K = 6, 48, 16, 4
    x = rng.standard_normal((T, D)).astype(np.float32)
    w = np.zeros((E, D), np.float32)
    w[:, :E] = 2.0 * np.eye(E, dtype=np.float32)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, wts, logits = route_from_hidden(x, w, bias, K)
    assert np.array_equal(logits, (2.0 * x[:, :E]).astype(np.float32))
    oids, owts = route((2.0 * x[:, :E]).astype(np.float32), bias, K)
    assert np.array_equal(ids, oids) and np.array_equal(wts.view(np.uint32), owts.view(np.uint32))


def test_equal_tokens_get_equal_logits():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 96)).astype(np.float32)
    w = rng.standard_normal((5, 96)).astype(np.float32)
    out = router_logits(np.repeat(x, 3, axis=0), w)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])
