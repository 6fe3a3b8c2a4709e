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
