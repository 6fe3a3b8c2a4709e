"""Pins of the oracle's MoE top-k combine against values fixed by hand and by
the routing's own bookkeeping ("MegaMoE：Blackwell 与 Hopper 的融合算子解读",
Blackwell section 13, the top-k reduce; Hopper section 09, the routing
weight on an expert's output)."""
import numpy as np

import datagen
import oracle


def bf16_bits(x):
    """bf16 bit patterns of values that bf16 holds exactly (truncation is exact then)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_combine_hand_example():
    # y[0] = 1*[1,2] + 0.5*[5,6] = [3.5, 5];  y[1] = 2*[3,4] - 1*[3,4] = [3, 4]
    Z = bf16_bits([[1, 2], [3, 4], [5, 6]])
    y = oracle.moe_combine_ref(Z, [[0, 2], [1, 1]], [[1.0, 0.5], [2.0, -1.0]])
    assert np.array_equal(y, [[3.5, 5.0], [3.0, 4.0]])


def test_combine_positions_outside_add_nothing():
    Z = bf16_bits([[1, 2], [3, 4], [5, 6]])
    assert np.array_equal(oracle.moe_combine_ref(Z, [[-1, 3], [2, 7]], [[1.0, 1.0], [1.0, 5.0]]),
                          [[0.0, 0.0], [5.0, 6.0]])


def test_combine_undoes_dispatch_with_equal_weights():
    # every routed row is its token's row: weights 1/top_k give back X exactly
    cfg = datagen.MOE["moe_small"]
    r = datagen.moe_route(cfg)
    X = np.random.RandomState(3).randint(-4, 5, size=(cfg.num_tokens, 40)).astype(np.float32)
    Z = bf16_bits(X[r.token_of_row])
    w = np.full(r.pos.shape, 1.0 / cfg.top_k)
    assert cfg.top_k & (cfg.top_k - 1) == 0
    assert np.array_equal(oracle.moe_combine_ref(Z, r.pos, w), X)


def test_routing_positions_invert_the_dispatch():
    # the routed row of (t, k) holds token t and belongs to expert top[t, k]
    r = datagen.moe_route(datagen.MOE["moe64"])
    t = np.arange(r.pos.shape[0])[:, None]
    assert np.array_equal(r.token_of_row[r.pos], np.broadcast_to(t, r.pos.shape))
    assert np.array_equal(r.expert_of_row[r.pos], r.top)
    assert np.all(r.weight > 0) and np.allclose(r.weight.sum(axis=1), 1.0, atol=1e-6)


def test_combine_linear_in_the_weights():
    rs = np.random.RandomState(5)
    Z = bf16_bits(rs.randint(-3, 4, size=(20, 16)))
    pos = rs.randint(0, 20, size=(7, 4))
    w = rs.randint(-2, 3, size=(7, 4)).astype(np.float64) / 4
    assert np.array_equal(oracle.moe_combine_ref(Z, pos, 2 * w), 2 * oracle.moe_combine_ref(Z, pos, w))


# --- the routing weight taken into FC1's epilogue (Hopper section 09: the
# FC1 chain optionally multiplies SwiGLU's output by the routing weight; with
# p(hW2) = (ph)W2 the combine then adds the contributions as they are) ---

def test_weighted_gate_unit_weights_is_the_gate():
    G = np.random.RandomState(11).randn(9, 48)
    assert np.array_equal(oracle.silu_gate(G, row_weight=np.ones(9)), oracle.silu_gate(G))


def test_weighted_gate_scales_each_row_by_its_own_weight():
    # distinct powers of two per row: scaling is exact, so a weight applied
    # to the wrong row, or twice, or not at all shows up bit for bit
    G = np.random.RandomState(12).randn(7, 32)
    w = 2.0 ** -np.arange(1, 8)
    h, hw = oracle.silu_gate(G), oracle.silu_gate(G, row_weight=w)
    assert np.array_equal(hw, h * w[:, None])
    # and the 16-bit rounding commutes with it (no subnormals here)
    assert np.array_equal(oracle.decode(oracle.encode(hw, "bf16"), "bf16"),
                          oracle.decode(oracle.encode(h, "bf16"), "bf16") * w[:, None])


def test_weighted_gate_zero_gate_or_weight_gives_zero():
    G = np.random.RandomState(13).randn(3, 16)
    G[0, :8] = 0.0                       # gate 0: SiLU(0) = 0 whatever the weight
    h = oracle.silu_gate(G, row_weight=[3.0, 0.0, 1.0])
    assert np.all(h[0] == 0.0) and np.all(h[1] == 0.0)
    assert np.array_equal(h[2], oracle.silu_gate(G)[2])


def test_combine_without_weights_is_the_plain_sum():
    Z = bf16_bits([[1, 2], [3, 4], [5, 6]])
    assert np.array_equal(oracle.moe_combine_ref(Z, [[0, 2], [1, 1]], None), [[6.0, 8.0], [6.0, 8.0]])
    pos = np.random.RandomState(14).randint(0, 3, size=(5, 2))
    assert np.array_equal(oracle.moe_combine_ref(Z, pos, None), oracle.moe_combine_ref(Z, pos, np.ones((5, 2))))


def test_folded_weights_equal_the_weighted_combine():
    """p(hW2) = (ph)W2 through the whole small layer: with power-of-two
    routing weights every scaling is exact, so FC1 with the weights in its
    epilogue, FC2, and a plain combine give the weighted combine of the
    unweighted layer bit for bit."""
    cfg = datagen.MOE["moe_small"]
    r, A, W1, W2 = datagen.moe_inputs_host(cfg, "random")
    rs = np.random.RandomState(15)
    w_tok = 2.0 ** -rs.randint(0, 4, size=r.pos.shape)       # [T][top_k]
    w_row = np.empty(int(r.offsets[-1]))
    w_row[r.pos] = w_tok                                     # the weight of each routed row
    g = oracle.grouped_ref(A, W1, r.offsets)
    h_plain = oracle.encode(oracle.silu_gate(g), "bf16")
    h_fold = oracle.encode(oracle.silu_gate(g, row_weight=w_row), "bf16")
    z_plain = oracle.encode(oracle.grouped_ref(h_plain, W2, r.offsets), "bf16")
    z_fold = oracle.encode(oracle.grouped_ref(h_fold, W2, r.offsets), "bf16")
    y_weighted = oracle.moe_combine_ref(z_plain, r.pos, w_tok)
    y_folded = oracle.moe_combine_ref(z_fold, r.pos, None)
    assert np.array_equal(y_folded, y_weighted)
    # and the weights mattered
    assert not np.array_equal(y_folded, oracle.moe_combine_ref(z_plain, r.pos, None))
