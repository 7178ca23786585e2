"""Seeded input generator: determinism, shapes and distributions."""
import numpy as np
import pytest

import workloads as wl


def test_bf16_rounding_is_nearest_even():
    a = np.array([1.0, 1.00390625, 1.005859375, -2.0, 3.0e-3], np.float32)
    b = wl.f32_to_bf16_bits(a)
    back = wl.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0078125)
    assert back[3] == -2.0
    assert abs(back[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # half an ulp of an 8-bit significand


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_inputs_shapes_and_determinism(name):
    w = wl.WORKLOADS[name]
    a = wl.make_inputs(w, T=300)
    b = wl.make_inputs(w, T=300)
    assert a["x"].shape == (300, w.d) and a["W"].shape == (w.E, w.d)
    assert a["x"].dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
    np.testing.assert_array_equal(a["x"], b["x"])
    np.testing.assert_array_equal(a["W"], b["W"])
    if w.dynamic_k:
        assert set(np.unique(a["k_per_token"])) <= set(w.dynamic_k)
        # constant within each request of 256 tokens
        assert np.all(a["k_per_token"][:256] == a["k_per_token"][0])
    if w.hash_vocab:
        tab = a["tid2eid"]
        assert tab.shape == (w.hash_vocab, w.k)
        s = np.sort(tab, axis=1)
        assert np.all(s[:, 1:] != s[:, :-1]) and tab.min() >= 0 and tab.max() < w.E
        assert a["token_ids"].min() >= 0 and a["token_ids"].max() < w.hash_vocab


def test_prefix_of_larger_T_is_the_same():
    w = wl.WORKLOADS["qwen3_dynk"]
    a = wl.make_inputs(w, T=100)
    b = wl.make_inputs(w, T=300)
    np.testing.assert_array_equal(a["W"], b["W"])
    np.testing.assert_array_equal(a["k_per_token"], b["k_per_token"][:100])


def test_distributions():
    w = wl.WORKLOADS["dsv3_grouped"]
    inp = wl.make_inputs(w, T=64)
    W = wl.bf16_bits_to_f32(inp["W"])
    assert abs(W.std() * np.sqrt(w.d) - 1.0) < 0.02
    assert abs(inp["select_bias"].std() - 0.1) < 0.03
    z = wl.zipf_offsets(0, 128)
    assert sorted(z)[-1] == pytest.approx(2.0) and sorted(z)[-2] == pytest.approx(2.0 * 2 ** -1.1)
    assert len(np.unique(z)) == 128
