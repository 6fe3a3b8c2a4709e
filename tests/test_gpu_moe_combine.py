"""GPU parity of the MoE top-k combine (mgemm_moe_combine) against the CPU
oracle: Y[t] = sum_k w[t, k] * Z[pos[t, k]], fp32 accumulate, one rounding.
Integer-valued rows with dyadic weights are exact (bit-exact); random data
within the rounding bound; positions outside Z add nothing."""
import sys

import numpy as np
import pytest

import datagen
import oracle
from helpers import assert_bits_equal, from_dev_bits, to_dev, values

torch = pytest.importorskip("torch")
mg = pytest.importorskip("bf16_gemm_amd")

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def run_combine(Z_bits, pos, w, dtype, T, H, ldy=None):
    """Y pre-filled with 0xFF bytes (and slack columns when ldy > H)."""
    ldy = H if ldy is None else ldy
    Z = to_dev(Z_bits, dtype)
    Y = torch.full((T, ldy), -1, dtype=torch.int16, device="cuda").view(Z.dtype)
    mg.moe_combine(Z, torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda(),
                   torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda(), Y[:, :H], pos.shape[1])
    torch.cuda.synchronize()
    got = from_dev_bits(Y)
    if ldy > H:
        assert np.all(got[:, H:] == 0xFFFF), "combine wrote past H"
    return got[:, :H]


def bound(Z_bits, pos, w, dtype, ref):
    """|got - ref| <= half an ulp of the output type plus the fp32 additions."""
    z = np.abs(oracle.decode(Z_bits, dtype))
    mag = np.zeros_like(ref)
    for k in range(pos.shape[1]):
        p = pos[:, k]
        ok = (p >= 0) & (p < z.shape[0])
        mag[ok] += np.abs(w[ok, k])[:, None] * z[p[ok]]
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    return rel * np.abs(ref) + pos.shape[1] * 2.0 ** -23 * mag


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("variant", ["random", "int"])
def test_combine_against_oracle(dtype, variant):
    T, top_k, H, rows = 150, 8, 1000, 600
    log(f"case combine {dtype} {variant} T={T} top_k={top_k} H={H}")
    rs = np.random.RandomState(11 if variant == "random" else 12)
    pos = rs.randint(-3, rows + 3, size=(T, top_k)).astype(np.int32)   # a few outside Z
    if variant == "random":
        Zb = datagen.matrix((rows, H), ("normal", 1.0), dtype, rs)
        w = rs.uniform(0.0, 1.0, size=(T, top_k)).astype(np.float32)
    else:
        Zb = datagen.matrix((rows, H), ("int", 4), dtype, rs)
        w = (rs.randint(-4, 5, size=(T, top_k)) / 4.0).astype(np.float32)
    got = run_combine(Zb, pos, w, dtype, T, H, ldy=H + 24)
    ref = oracle.moe_combine_ref(Zb, pos, w.astype(np.float64), dtype)
    if variant == "int":
        assert_bits_equal(got, ref, dtype, "combine int")
    else:
        err = np.abs(values(got, dtype) - ref)
        assert np.all(err <= bound(Zb, pos, w, dtype, ref)), f"max err {err.max():.3e}"


def test_combine_strided_rows():
    """Z rows longer than H (ldz = H + 24, the slack NaN): integer data, bit-exact."""
    T, top_k, H, rows = 40, 4, 128, 90
    rs = np.random.RandomState(13)
    Zb = datagen.matrix((rows, H), ("int", 3), "bf16", rs)
    Zw = np.full((rows, H + 24), 0x7FC1, dtype=np.uint16)
    Zw[:, :H] = Zb
    pos = rs.randint(0, rows, size=(T, top_k)).astype(np.int32)
    w = (rs.randint(-4, 5, size=(T, top_k)) / 2.0).astype(np.float32)
    Z = to_dev(Zw, "bf16")[:, :H]
    Y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(Z, torch.from_numpy(pos).cuda(), torch.from_numpy(w).cuda(), Y, top_k)
    torch.cuda.synchronize()
    assert_bits_equal(from_dev_bits(Y), oracle.moe_combine_ref(Zb, pos, w.astype(np.float64)), "bf16", "strided Z")


def test_combine_moe64_routing_sampled_tokens():
    """The 64-expert layer's routing (4096 tokens, top 8, hidden 7168) on
    routed rows of random data; 64 tokens checked against the oracle."""
    cfg = datagen.MOE["moe64"]
    r = datagen.moe_route(cfg)
    rows, H = int(r.offsets[-1]), cfg.hidden
    log(f"case combine moe64 rows={rows} H={H}")
    g = torch.Generator(device="cuda").manual_seed(7)
    Z = torch.randn(rows, H, device="cuda", generator=g).bfloat16()
    Y = torch.empty(cfg.num_tokens, H, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(Z, torch.from_numpy(r.pos).cuda(), torch.from_numpy(r.weight).cuda(), Y, cfg.top_k)
    torch.cuda.synchronize()
    toks = np.random.RandomState(1).choice(cfg.num_tokens, 64, replace=False)
    sub_pos = r.pos[toks]
    uniq, inv = np.unique(sub_pos, return_inverse=True)
    Zs = from_dev_bits(Z[torch.from_numpy(uniq).cuda()])
    ref = oracle.moe_combine_ref(Zs, inv.reshape(sub_pos.shape), r.weight[toks].astype(np.float64))
    got = from_dev_bits(Y[torch.from_numpy(toks).cuda()])
    err = np.abs(values(got, "bf16") - ref)
    assert np.all(err <= bound(Zs, inv.reshape(sub_pos.shape), r.weight[toks], "bf16", ref)), f"max err {err.max():.3e}"


def test_combine_argument_errors_and_empty():
    Z = torch.zeros(4, 12, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    w = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(mg.MgemmError):                 # H = 12 is not a multiple of 8
        mg.moe_combine(Z, pos, w, torch.empty(2, 12, dtype=torch.bfloat16, device="cuda"), 1)
    with pytest.raises(mg.MgemmError):                 # fp32 rows are not supported
        mg.moe_combine(Z.float(), pos, w, torch.empty(2, 12, dtype=torch.float32, device="cuda"), 1)
    Y = torch.full((0, 16), 1.0, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda"), pos, w, Y, 1)   # T == 0: no-op
    torch.cuda.synchronize()
