"""CPU pins of the oracle's fp8 (E4M3) W1 path, against the format's
definition and the bf16 path it reduces to.

The format is OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, subnormals of 2^-9 steps, largest finite value
1.75 * 2^8 = 448 (code 0x7E), 0x7F NaN, no infinities; conversion rounds to
nearest, ties to even, and saturates to +-448 ("[RFC]: Async AFD for Prefill
on Ascend NPU", "Architecture", names a quantised W1 GEMM but no format: this
is the reading taken).
"""
import numpy as np
import pytest

from combine_afd_slot_amd.inputs import make_inputs, small_workload
from oracle import oracle as orc


@pytest.mark.parametrize("v,code", [
    (0.0, 0x00), (1.0, 0x38), (-1.0, 0xB8), (2.0, 0x40), (0.5, 0x30), (448.0, 0x7E), (-448.0, 0xFE),
    (480.0, 0x7E), (1e9, 0x7E), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07),
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (1.0625, 0x38), (1.1875, 0x3A), (240.0, 0x77),
    (-0.0, 0x00), (2.0 ** -12, 0x00),
])
def test_known_codes(v, code):
    # exponent field e -> 2^(e-7), fraction f/8; e = 0: f * 2^-9
    assert int(orc.e4m3_encode([v])[0]) == code


def test_every_code_round_trips_and_orders():
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    vals = orc.e4m3_decode(pos)
    assert vals[0] == 0.0 and vals[1] == 2.0 ** -9 and vals[0x7E] == 448.0
    assert np.all(np.diff(vals) > 0)
    np.testing.assert_array_equal(orc.e4m3_encode(vals.astype(np.float32)), pos)
    neg = (pos[1:] | 0x80).astype(np.uint8)
    np.testing.assert_array_equal(orc.e4m3_decode(neg), -vals[1:])
    np.testing.assert_array_equal(orc.e4m3_encode(-vals[1:].astype(np.float32)), neg)


def test_ties_to_even_and_nearest():
    vals = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mid = (vals[:-1] + vals[1:]) / 2  # exact in fp32 (at most 5 significant bits)
    codes = orc.e4m3_encode(mid.astype(np.float32)).astype(int)
    lo = np.arange(0, 0x7E)
    np.testing.assert_array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))
    eps = (vals[1:] - vals[:-1]) / 8
    np.testing.assert_array_equal(orc.e4m3_encode((mid - eps).astype(np.float32)), lo)
    np.testing.assert_array_equal(orc.e4m3_encode((mid + eps).astype(np.float32)), lo + 1)


def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quant_rows():
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((6, 96)) * np.array([1e-3, 1, 3, 100, 0, 1e-30])[:, None])
    codes, d, deq = orc.quant_rows(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i in range(6):
        amax = np.abs(xf[i]).max()
        if amax == 0:
            assert d[i] == 1.0 and not codes[i].any() and not deq[i].any()
            continue
        # the largest element maps to the largest code, the scale is amax / 448
        j = int(np.abs(xf[i]).argmax())
        assert codes[i, j] & 0x7F == 0x7E
        assert d[i] == np.float32(np.float32(amax) / np.float32(448.0))
        # relative error of a normal code at most 2^-4, absolute at most half a subnormal step
        err = np.abs(deq[i] - xf[i])
        assert np.all(err <= np.abs(xf[i]) * 2.0 ** -4 + 2.0 ** -10 * d[i] * 1.0001)
        np.testing.assert_array_equal(deq[i], orc.e4m3_decode(codes[i]) * np.float64(d[i]))


def test_double_path_reduces_to_bf16_path():
    """With the exact bf16 values as its double operands, the fp8 path's
    per-token routine gives the bf16 path's rows bit for bit."""
    wl = small_workload("fp8_reduce", seq_lens=(9, 5), hidden=64, num_experts=6, top_k=2, intermediate=40,
                        shared_intermediate=24, token_cap=16)
    inp = make_inputs(wl)
    X = np.concatenate(inp["x"])
    L = np.concatenate(inp["l"])
    f = lambda a: (np.asarray(a, np.uint32) << 16).view(np.float32).astype(np.float64)
    tok = np.arange(X.shape[0])
    ref, ids, w = orc.token_rows(X, L, tok, inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=2)
    got, ids_d, w_d = orc.token_rows_d(f(X), L, tok, f(inp["W13"]), inp["W2"], f(inp["Ws13"]), inp["Ws2"], K=2)
    np.testing.assert_array_equal(ids_d, ids)
    np.testing.assert_array_equal(got, ref)


def test_fp8_path_close_to_bf16_path():
    wl = small_workload("fp8_close", seq_lens=(20, 11), hidden=128, num_experts=8, top_k=2, intermediate=64,
                        shared_intermediate=64, token_cap=24)
    inp = make_inputs(wl)
    q = orc.ffn_fp8(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=2)
    b = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=2)["out_p"]
    for p in range(2):
        rel = np.abs(q[p] - b[p]).max(axis=1) / np.abs(b[p]).max(axis=1)
        assert 0 < rel.max() < 0.15, rel.max()


@pytest.mark.parametrize("Is,renorm,rsf", [(48, 1, 1.0), (0, 0, 1.5)])
def test_grouped_fp8_path_equals_per_token_path(Is, renorm, rsf):
    """The grouped fp8 path (experts one dispatch group at a time) gives the
    per-token fp8 routine's rows bit for bit: the same operands and the same
    order of every sum, with the pairs of each token gathered by the
    dispatch permutation."""
    wl = small_workload("fp8_grouped", seq_lens=(23, 0, 40), hidden=96, num_experts=9, top_k=3, intermediate=56,
                        shared_intermediate=Is, token_cap=48, zipf_bias=0.7)
    inp = make_inputs(wl)
    a = orc.ffn_fp8(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=3, rsf=rsf,
                    renorm=renorm)
    b = orc.ffn_fp8_tokens(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=3,
                           rsf=rsf, renorm=renorm)
    for p in range(wl.num_peers):
        np.testing.assert_array_equal(a[p], b[p])


def test_grouped_double_path_reduces_to_bf16_path():
    """experts_d / shared_d on the exact bf16 values equal the bf16 grouped
    routines (experts / shared) bit for bit."""
    wl = small_workload("fp8_reduce_g", seq_lens=(17, 6), hidden=64, num_experts=6, top_k=2, intermediate=40,
                        shared_intermediate=24, token_cap=24)
    inp = make_inputs(wl)
    f = lambda a: (np.asarray(a, np.uint32) << 16).view(np.float32).astype(np.float64)
    X = np.concatenate(inp["x"])
    ids, w = orc.route(np.concatenate(inp["l"]), 2)
    _, eoff, perm, _ = orc.dispatch(ids, wl.num_experts)
    np.testing.assert_array_equal(orc.experts_d(f(X), eoff, perm, 2, f(inp["W13"]), inp["W2"]),
                                  orc.experts(X, eoff, perm, 2, inp["W13"], inp["W2"]))
    np.testing.assert_array_equal(orc.shared_d(f(X), f(inp["Ws13"]), inp["Ws2"]),
                                  orc.shared(X, inp["Ws13"], inp["Ws2"]))
