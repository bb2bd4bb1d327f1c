"""Pins for the oracle's storage step and the layer-wise driver, CPU only.

Packing is pinned by a hand-worked word, by a big-integer construction of the bit stream (a different
route to the same bits) and by the round trip. Dequantization is pinned by hand values and by the
quantizer's own Q. The layer-wise driver is pinned by its wiring: each layer is calibrated on the
outputs of the layers before it after they were quantized ([guide] "How it works", apply_layerwise),
with the limits where quantization disappears (identity quantizer, 8 bits) and the guide's simulation
claim that GPTQ beats round-to-nearest on the wide layers.
"""
from functools import partial

import numpy as np
import pytest

from oracle import gptq_oracle as O
import synthetic as syn


# ------------------------------------------------------------------------------------------------
# Packing
# ------------------------------------------------------------------------------------------------
def test_pack_hand_word_4bit():
    """Symmetric 4-bit codes 1, -2, 7, -8 are stored as 9, 6, 15, 0 (offset 8); nibble j holds code j,
    lowest nibble first: 0x00000F69."""
    w = O.pack_rows(np.array([[1, -2, 7, -8]]), 4)
    assert w.dtype == np.uint32 and w.shape == (1, 1)
    assert int(w[0, 0]) == 0x00000F69


def test_pack_hand_words_3bit_straddle():
    """Eleven asymmetric 3-bit codes fill 33 bits: code 10 (= 5 = 0b101) has its low two bits at stream
    bits 30-31 (word 0: 0b01 there) and its top bit at bit 32 (word 1, bit 0).
    Word 0 = sum_j c_j 8^j for j < 10 plus (5 & 3) << 30, c = 1..7, 0, 1, 2; written from the top bit down:
    01 010 001 000 111 110 101 100 011 010 001 = 0x511F58D1."""
    c = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 5]])
    w = O.pack_rows(c, 3, asymmetric=True)
    assert w.shape == (1, 2)
    expect0 = int("01" "010" "001" "000" "111" "110" "101" "100" "011" "010" "001", 2)
    assert int(w[0, 0]) == expect0 == 0x511F58D1
    assert int(w[0, 1]) == 1


def _bigint_words(stored_row, bits, n_words):
    acc = 0
    for j, v in enumerate(stored_row):
        acc += int(v) << (bits * j)
    return [(acc >> (32 * k)) & 0xFFFFFFFF for k in range(n_words)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("asym", [False, True])
def test_pack_equals_bigint_stream_and_round_trips(bits, asym):
    rng = np.random.default_rng(100 * bits + asym)
    for d in (1, 7, 31, 32, 33, 100):
        if asym:
            c = rng.integers(0, 2 ** bits, size=(3, d))
        else:
            q = 2 ** (bits - 1) - 1
            c = rng.integers(-q, q + 1, size=(3, d))
            c[0, 0] = -q
        w = O.pack_rows(c, bits, asym)
        n_words = -(-d * bits // 32)
        assert w.shape == (3, n_words)
        off = 0 if asym else 2 ** (bits - 1)
        for r in range(3):
            assert [int(x) for x in w[r]] == _bigint_words(c[r] + off, bits, n_words)
        np.testing.assert_array_equal(O.unpack_rows(w, d, bits, asym), c)


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_rows(np.array([[8]]), 4)            # symmetric 4-bit stores -8..7
    with pytest.raises(ValueError):
        O.pack_rows(np.array([[-1]]), 3, True)     # asymmetric codes are non-negative
    with pytest.raises(ValueError):
        O.pack_rows(np.array([[0]]), 9)


# ------------------------------------------------------------------------------------------------
# Dequantization and the consumer
# ------------------------------------------------------------------------------------------------
def test_dequantize_hand_values():
    codes = np.array([[1, -2, 3]])
    scales = np.array([[0.5, 2.0]])
    g_idx = np.array([1, 0, 1])
    np.testing.assert_array_equal(O.dequantize(codes, scales, g_idx), [[2.0, -1.0, 6.0]])
    zeros = np.array([[1, 2]])
    np.testing.assert_array_equal(O.dequantize(np.array([[3, 0, 2]]), scales, g_idx, zeros), [[2.0, -0.5, 0.0]])


@pytest.mark.parametrize("asym", [False, True])
def test_dequantize_reproduces_quantizer_q(asym):
    """With act_order and groups the groups are not contiguous; Q rebuilt through g_idx must equal the
    quantizer's own Q, built inside its loop."""
    rng = np.random.default_rng(5)
    X = np.maximum(rng.standard_normal((80, 24)) * rng.uniform(0.2, 3, 24), 0)
    W = rng.standard_normal((7, 24))
    f = O.gptq_oracle_asym if asym else O.gptq_oracle
    r = f(W, X, bits=3, group=8, act_order=True)
    assert not np.array_equal(r["g_idx"], np.arange(24) // 8)
    Q = O.dequantize(r["codes"], r["scales"], r["g_idx"], r.get("zeros") if asym else None)
    np.testing.assert_array_equal(Q, r["Q"])


def test_linear_forward_hand_values():
    h = np.array([[1.0, 2.0]])
    W = np.array([[1.0, 1.0], [1.0, -1.0]])
    b = np.array([0.5, 0.0])
    np.testing.assert_array_equal(O.linear_forward(h, W, b, relu=True), [[3.5, 0.0]])
    np.testing.assert_array_equal(O.linear_forward(h, W, b, relu=False), [[3.5, -1.0]])
    y = O.linear_forward(np.array([[1.0]]), np.array([[1.0 / 3.0]]), None, relu=False)
    assert y[0, 0] == float(np.float32(1.0 / 3.0))


# ------------------------------------------------------------------------------------------------
# The layer-wise driver
# ------------------------------------------------------------------------------------------------
def _mlp(name="teacher_mlp"):
    w, b, X = syn.gen_mlp(syn.mlp_config_by_name(name))
    return [x.astype(np.float64) for x in w], [x.astype(np.float64) for x in b], X.astype(np.float64)


def _plain_forward(weights, biases, X):
    h = X
    for i, (W, b) in enumerate(zip(weights, biases)):
        h = h @ W.T + b
        if i < len(weights) - 1:
            h = np.maximum(h, 0)
        h = h.astype(np.float32).astype(np.float64)
    return h


def test_layerwise_identity_quantizer_is_the_plain_forward():
    """A quantizer that returns the weights unchanged leaves the network's forward pass."""
    weights, biases, X = _mlp()
    res, inputs, h = O.apply_layerwise(weights, biases, X, lambda W, hh: {"Q": W})
    np.testing.assert_allclose(h, _plain_forward(weights, biases, X), rtol=1e-6, atol=1e-6)
    assert len(inputs) == 4 and inputs[0] is not None and np.array_equal(inputs[0], X)


def test_layerwise_single_layer_is_gptq():
    weights, biases, X = _mlp()
    q = partial(O.gptq_oracle, bits=3, act_order=True)
    res, inputs, _ = O.apply_layerwise(weights[:1], biases[:1], X, q)
    direct = O.gptq_oracle(weights[0], X, bits=3, act_order=True)
    np.testing.assert_array_equal(res[0]["codes"], direct["codes"])


def test_layerwise_calibrates_on_quantized_outputs():
    """Layer 2 is calibrated on relu(X Q1^T + b1) (fp32), Q1 the quantized first layer, not on the
    full-precision layer's outputs; at 2 bits the two differ."""
    weights, biases, X = _mlp()
    q = partial(O.gptq_oracle, bits=2)
    res, inputs, _ = O.apply_layerwise(weights[:3], biases[:3], X, q)
    Q1 = res[0]["Q"].astype(np.float32).astype(np.float64)
    from_q = np.maximum(X @ Q1.T + biases[0], 0).astype(np.float32).astype(np.float64)
    from_w = np.maximum(X @ weights[0].T + biases[0], 0).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(inputs[1], from_q, rtol=1e-6, atol=1e-6)
    assert np.abs(inputs[1] - from_w).max() > 1e-2
    # and layer 2's quantization is GPTQ on exactly that input
    np.testing.assert_array_equal(res[1]["codes"], O.gptq_oracle(weights[1], inputs[1], bits=2)["codes"])


def test_layerwise_skip_last_keeps_output_layer():
    weights, biases, X = _mlp()
    q = partial(O.gptq_oracle, bits=3)
    res, inputs, h = O.apply_layerwise(weights, biases, X, q, skip_last=True)
    assert res[-1] is None and all(r is not None for r in res[:-1])
    Q3 = res[2]["Q"].astype(np.float32).astype(np.float64)
    last_in = inputs[3]
    np.testing.assert_allclose(h, (last_in @ weights[3].T + biases[3]).astype(np.float32), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(last_in, np.maximum(inputs[2] @ Q3.T + biases[2], 0).astype(np.float32),
                               rtol=1e-6, atol=1e-6)


def test_layerwise_8bit_is_close_to_full_precision():
    weights, biases, X = _mlp()
    _, _, h = O.apply_layerwise(weights, biases, X, partial(O.gptq_oracle, bits=8))
    ref = _plain_forward(weights, biases, X)
    assert np.linalg.norm(h - ref) / np.linalg.norm(ref) < 1e-2


def test_layerwise_dead_units_become_dead_inputs():
    """Hidden units that never fire on the calibration data are dead inputs of the next layer: their
    weights come out zero."""
    weights, biases, X = _mlp()
    res, inputs, _ = O.apply_layerwise(weights, biases, X, partial(O.gptq_oracle, bits=3))
    for i in (1, 2, 3):
        dead = res[i]["dead"]
        assert dead.sum() >= 6
        assert np.all(inputs[i][:, dead] == 0)
        assert np.all(res[i]["codes"][:, dead] == 0)


@pytest.mark.parametrize("asym", [False, True])
def test_layerwise_gptq_beats_rtn_on_wide_layers(asym):
    """[guide] "What the simulations show": on the layers with 256 inputs GPTQ cuts the relative output
    error on the inputs each layer sees several times below round-to-nearest; on the 12-input first
    layer the gain is small. Checked per layer, RTN on the same inputs."""
    weights, biases, X = _mlp()
    f = O.gptq_oracle_asym if asym else O.gptq_oracle
    res, inputs, _ = O.apply_layerwise(weights, biases, X, partial(f, bits=3, act_order=True), skip_last=True)
    for i in (1, 2):
        S = inputs[i].T @ inputs[i]
        e_g = O.relative_output_error(weights[i], res[i]["Q"], S)
        rtn = O.rtn_asym if asym else O.rtn
        _, Q_r = rtn(weights[i], 3, dead=res[i]["dead"])
        e_r = O.relative_output_error(weights[i], Q_r, S)
        assert e_g < 0.5 * e_r, (i, e_g, e_r)
