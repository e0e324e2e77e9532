"""Pins of the oracle's sampled layer (the one the parity tests at full size
compare against) against its whole layer: for every token of tiny and
decode_b8, the sampled evaluation's route rows, intermediate and outputs are
those of the grouped evaluation over all tokens (the permutation changes no
token's result). A route row taken from the wrong token, expert or k, or a
finalize over the wrong routes, fails it."""
import numpy as np
import pytest

from nvfp4_block_scaled_route_amd import workloads as W
from oracle.layer import layer, layer_sampled


@pytest.mark.parametrize("name", ["tiny", "decode_b8"])
def test_layer_sampled_equals_layer_on_every_token(name):
    inp = W.make_inputs(W.WORKLOADS[name])
    wl = inp.wl
    full = layer(inp)
    e2p = full["meta"]["exp2perm"]
    # all tokens, in a scrambled order so that the sample index differs from the token
    tokens = np.random.default_rng(1).permutation(wl.T)
    smp = layer_sampled(inp, tokens)
    assert np.array_equal(smp["served"], e2p[tokens] >= 0)
    assert np.array_equal(smp["ids"], full["ids"][tokens])
    assert np.array_equal(smp["out"], full["out"][tokens])
    tt, kk = np.nonzero(smp["served"])
    p = e2p[tokens][tt, kk]
    assert np.array_equal(smp["route_rows"][tt, kk], full["rows"][p])
    # per-route intermediate: the grouped one is in permuted row order
    pos = np.searchsorted(full["rows_idx"], p)
    assert np.array_equal(full["rows_idx"][pos], p)
    assert np.array_equal(smp["h_codes"], full["h_codes"][pos])
    assert np.array_equal(smp["h_sf"], full["h_sf"][pos])


def test_layer_sampled_subset_is_a_subset():
    """A strict subset of tokens (with a repeat) gives the same per-token outputs."""
    inp = W.make_inputs(W.WORKLOADS["decode_b8"])
    full = layer(inp)
    tokens = np.array([5, 0, 5, 7])
    smp = layer_sampled(inp, tokens)
    assert np.array_equal(smp["out"], full["out"][tokens])
