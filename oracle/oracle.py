"""Python face of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check of __graft_entry__ and the CPU-baseline leg of
bench.py may import this module.  It wraps liboracle.so (plain C, float64
accumulation, built from afd_oracle.c with gcc) and adds nothing to its
arithmetic beyond argument marshalling.  It imports nothing from the HIP
library or its package.

Parity status: every entry point is pinned by the CPU tests
(tests/test_oracle_*.py) against closed forms, invariants, library special
cases and a float64 dense brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "afd_oracle.c")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-fPIC", "-shared", SRC_PATH, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_fanin.argtypes = [i32, P, ctypes.c_int32, P]
        L.oracle_route.argtypes = [i64, i32, i32, i32, P, P, P]
        L.oracle_dispatch.argtypes = [i64, i32, i32, P, P, P, P, P]
        L.oracle_swiglu_row.argtypes = [i64, i64, P, P, P, P]
        L.oracle_experts.argtypes = [i64, i64, i32, i32, i64, P, P, P, P, P, P]
        L.oracle_shared.argtypes = [i64, i64, i64, P, P, P, P]
        L.oracle_combine.argtypes = [i64, i64, i32, dbl, P, P, P, P, P]
        L.oracle_ffn.argtypes = [i32, P, P, P, i64, i32, i32, i64, i64, dbl, i32,
                                 P, P, P, P, P, P, P, P, P, P, P, P]
        L.oracle_token_rows.argtypes = [i64, i64, i32, i32, i64, i64, dbl, i32, P, P, P, P, P, P,
                                        i64, P, P, P, P]
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = dbl
        L.oracle_quant_rows.argtypes = [i64, i64, P, P, P, P]
        L.oracle_token_rows_d.argtypes = [i64, i64, i32, i32, i64, i64, dbl, i32, P, P, P, P, P, P,
                                          i64, P, P, P, P]
        L.oracle_experts_d.argtypes = [i64, i64, i32, i32, i64, P, P, P, P, P, P]
        L.oracle_shared_d.argtypes = [i64, i64, i64, P, P, P, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def fanin(seq_lens, token_cap=0):
    s = np.ascontiguousarray(seq_lens, dtype=np.int32)
    off = np.zeros(len(s) + 1, dtype=np.int32)
    _check(lib().oracle_fanin(len(s), _p(s), int(token_cap), _p(off)), "fanin")
    return off


def route(L, K, renorm=1):
    L = np.ascontiguousarray(L, dtype=np.float32)
    T, E = L.shape
    ids = np.zeros((T, K), dtype=np.int32)
    w = np.zeros((T, K), dtype=np.float64)
    _check(lib().oracle_route(T, E, K, int(renorm), _p(L), _p(ids), _p(w)), "route")
    return ids, w


def dispatch(ids, E):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    counts = np.zeros(E, dtype=np.int32)
    eoff = np.zeros(E + 1, dtype=np.int32)
    perm = np.zeros(T * K, dtype=np.int32)
    inv = np.zeros(T * K, dtype=np.int32)
    _check(lib().oracle_dispatch(T, E, K, _p(ids), _p(counts), _p(eoff), _p(perm), _p(inv)),
           "dispatch")
    return counts, eoff, perm, inv


def swiglu_row(x, w13, w2):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w13 = np.ascontiguousarray(w13, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2, dtype=np.uint16)
    H = x.shape[0]
    I = w13.shape[0] // 2
    y = np.zeros(H, dtype=np.float64)
    _check(lib().oracle_swiglu_row(H, I, _p(x), _p(w13), _p(w2), _p(y)), "swiglu_row")
    return y


def experts(X, eoff, perm, K, W13, W2):
    X = np.ascontiguousarray(X, dtype=np.uint16)
    T, H = X.shape
    E = W13.shape[0]
    I = W13.shape[1] // 2
    Y = np.zeros((T * K, H), dtype=np.float64)
    _check(lib().oracle_experts(T, H, E, K, I, _p(X), _p(np.ascontiguousarray(eoff, np.int32)),
                                _p(np.ascontiguousarray(perm, np.int32)),
                                _p(np.ascontiguousarray(W13)), _p(np.ascontiguousarray(W2)), _p(Y)),
           "experts")
    return Y


def shared(Xs, Ws13, Ws2):
    Xs = np.ascontiguousarray(Xs, dtype=np.uint16)
    T, H = Xs.shape
    Is = Ws13.shape[0] // 2
    S = np.zeros((T, H), dtype=np.float64)
    _check(lib().oracle_shared(T, H, Is, _p(Xs), _p(np.ascontiguousarray(Ws13)),
                               _p(np.ascontiguousarray(Ws2)), _p(S)), "shared")
    return S


def combine(w, inv, Y, S, rsf=1.0):
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, K = w.shape
    H = Y.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    _check(lib().oracle_combine(T, H, K, float(rsf), _p(w), _p(np.ascontiguousarray(inv, np.int32)),
                                _p(np.ascontiguousarray(Y)), _p(None if S is None else np.ascontiguousarray(S)),
                                _p(out)), "combine")
    return out


def ffn(x, l, W13, W2, Ws13=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """The whole path a1..a7 on per-peer inputs x[p] (uint16 [n_p,H]) and
    l[p] (float32 [n_p,E]).  Returns a dict with out (float64 [T,H]), the
    per-peer split out_p, ids, w, counts, expert_offsets, perm, inv, off."""
    P = len(x)
    seq = np.asarray([a.shape[0] for a in x], dtype=np.int32)
    H = W13.shape[2]
    E = W13.shape[0]
    I = W13.shape[1] // 2
    Is = 0 if Ws13 is None else Ws13.shape[0] // 2
    xs = [np.ascontiguousarray(a, dtype=np.uint16) for a in x]
    ls = [np.ascontiguousarray(a, dtype=np.float32) for a in l]
    xp = (ctypes.c_void_p * P)(*[a.ctypes.data for a in xs])
    lp = (ctypes.c_void_p * P)(*[a.ctypes.data for a in ls])
    T = int(seq.sum())
    r = {
        "ids": np.zeros((T, K), np.int32), "w": np.zeros((T, K), np.float64),
        "counts": np.zeros(E, np.int32), "expert_offsets": np.zeros(E + 1, np.int32),
        "perm": np.zeros(T * K, np.int32), "inv": np.zeros(T * K, np.int32),
        "off": np.zeros(P + 1, np.int32), "out": np.zeros((T, H), np.float64),
    }
    _check(lib().oracle_ffn(P, _p(seq), ctypes.cast(xp, ctypes.c_void_p), ctypes.cast(lp, ctypes.c_void_p),
                            H, E, K, I, Is, float(rsf), int(renorm),
                            _p(np.ascontiguousarray(W13)), _p(np.ascontiguousarray(W2)),
                            _p(None if Ws13 is None else np.ascontiguousarray(Ws13)),
                            _p(None if Ws2 is None else np.ascontiguousarray(Ws2)),
                            _p(r["ids"]), _p(r["w"]), _p(r["counts"]), _p(r["expert_offsets"]),
                            _p(r["perm"]), _p(r["inv"]), _p(r["off"]), _p(r["out"])), "ffn")
    r["out_p"] = [r["out"][r["off"][p]:r["off"][p + 1]] for p in range(P)]
    return r


def token_rows(X, L, tokens, W13, W2, Ws13=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """Output rows (float64 [n,H]) for the given fan-in token indices, one
    token at a time; also returns that token's ids and weights."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    L = np.ascontiguousarray(L, dtype=np.float32)
    T, H = X.shape
    E = L.shape[1]
    I = W13.shape[1] // 2
    Is = 0 if Ws13 is None else Ws13.shape[0] // 2
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    out = np.zeros((n, H), np.float64)
    ids = np.zeros((n, K), np.int32)
    w = np.zeros((n, K), np.float64)
    _check(lib().oracle_token_rows(T, H, E, K, I, Is, float(rsf), int(renorm), _p(X), _p(L),
                                   _p(np.ascontiguousarray(W13)), _p(np.ascontiguousarray(W2)),
                                   _p(None if Ws13 is None else np.ascontiguousarray(Ws13)),
                                   _p(None if Ws2 is None else np.ascontiguousarray(Ws2)),
                                   n, _p(tok), _p(out), _p(ids), _p(w)), "token_rows")
    return out, ids, w


def timed_token_rows(X, L, tokens, W13, W2, Ws13=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """token_rows with its wall-clock time (steady clock), for the CPU baseline."""
    t0 = time.perf_counter()
    r = token_rows(X, L, tokens, W13, W2, Ws13, Ws2, K=K, rsf=rsf, renorm=renorm)
    return r, time.perf_counter() - t0


# ---------------------------------------------------------------------------
# fp8 (E4M3) W1 path: codec, per-row quantisation, the per-token path on
# dequantised gate/up operands (afd_oracle.c, "FP8 for the quantised W1").
def e4m3_encode(v):
    v = np.asarray(v, dtype=np.float32)
    return np.array([lib().oracle_e4m3_encode(float(a)) for a in v.ravel()], np.uint8).reshape(v.shape)


def e4m3_decode(c):
    c = np.asarray(c, dtype=np.uint8)
    return np.array([lib().oracle_e4m3_decode(int(a)) for a in c.ravel()], np.float64).reshape(c.shape)


def quant_rows(x):
    """Rows of bf16 bit patterns -> (e4m3 codes, fp32 row scales d, dequantised float64 rows)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    H = x.shape[-1]
    flat = x.reshape(-1, H)
    n = flat.shape[0]
    codes = np.zeros((n, H), np.uint8)
    d = np.zeros(n, np.float32)
    deq = np.zeros((n, H), np.float64)
    _check(lib().oracle_quant_rows(n, H, _p(flat), _p(codes), _p(d), _p(deq)), "quant_rows")
    return codes.reshape(x.shape), d.reshape(x.shape[:-1]), deq.reshape(x.shape)


def token_rows_d(Xd, L, tokens, W13d, W2, Ws13d=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """oracle token_rows with double gate/up operands (the fp8 W1 path)."""
    Xd = np.ascontiguousarray(Xd, dtype=np.float64)
    L = np.ascontiguousarray(L, dtype=np.float32)
    T, H = Xd.shape
    E = W13d.shape[0]
    I = W13d.shape[1] // 2
    Is = 0 if Ws13d is None else Ws13d.shape[0] // 2
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    out = np.zeros((n, H), np.float64)
    ids = np.zeros((n, K), np.int32)
    w = np.zeros((n, K), np.float64)
    _check(lib().oracle_token_rows_d(T, H, E, K, I, Is, float(rsf), int(renorm), _p(Xd), _p(L),
                                     _p(np.ascontiguousarray(W13d, np.float64)), _p(np.ascontiguousarray(W2)),
                                     _p(None if Ws13d is None else np.ascontiguousarray(Ws13d, np.float64)),
                                     _p(None if Ws2 is None else np.ascontiguousarray(Ws2)),
                                     n, _p(tok), _p(out), _p(ids), _p(w)), "token_rows_d")
    return out, ids, w


def experts_d(Xd, eoff, perm, K, W13d, W2):
    """oracle experts (grouped by expert) on double gate/up operands."""
    Xd = np.ascontiguousarray(Xd, dtype=np.float64)
    T, H = Xd.shape
    E = W13d.shape[0]
    I = W13d.shape[1] // 2
    Y = np.zeros((T * K, H), dtype=np.float64)
    _check(lib().oracle_experts_d(T, H, E, K, I, _p(Xd), _p(np.ascontiguousarray(eoff, np.int32)),
                                  _p(np.ascontiguousarray(perm, np.int32)),
                                  _p(np.ascontiguousarray(W13d, np.float64)), _p(np.ascontiguousarray(W2)), _p(Y)),
           "experts_d")
    return Y


def shared_d(Xd, Ws13d, Ws2):
    """oracle shared expert on double gate/up operands."""
    Xd = np.ascontiguousarray(Xd, dtype=np.float64)
    T, H = Xd.shape
    Is = Ws13d.shape[0] // 2
    S = np.zeros((T, H), dtype=np.float64)
    _check(lib().oracle_shared_d(T, H, Is, _p(Xd), _p(np.ascontiguousarray(Ws13d, np.float64)),
                                 _p(np.ascontiguousarray(Ws2)), _p(S)), "shared_d")
    return S


def _fp8_operands(x, W13, Ws13):
    X = np.concatenate([np.asarray(a, np.uint16).reshape(-1, W13.shape[2]) for a in x])
    _, _, Xd = quant_rows(X)
    _, _, W13d = quant_rows(W13)
    Ws13d = None if Ws13 is None else quant_rows(Ws13)[2]
    return Xd, W13d, Ws13d


def ffn_fp8(x, l, W13, W2, Ws13=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """The whole path with the gate/up GEMMs on e4m3 operands (token rows and
    W13 / Ws13 rows quantised per row): route, dispatch, the experts one
    dispatch group at a time, the shared expert, combine; per-peer outputs."""
    Xd, W13d, Ws13d = _fp8_operands(x, W13, Ws13)
    Lc = np.concatenate([np.asarray(a, np.float32).reshape(-1, W13.shape[0]) for a in l])
    ids, w = route(Lc, K, renorm)
    _, eoff, perm, inv = dispatch(ids, W13.shape[0])
    Y = experts_d(Xd, eoff, perm, K, W13d, W2)
    S = None if Ws13d is None else shared_d(Xd, Ws13d, Ws2)
    out = combine(w, inv, Y, S, rsf)
    off = np.concatenate([[0], np.cumsum([np.asarray(a).shape[0] for a in x])])
    return [out[off[p]:off[p + 1]] for p in range(len(x))]


def ffn_fp8_tokens(x, l, W13, W2, Ws13=None, Ws2=None, K=2, rsf=1.0, renorm=1):
    """ffn_fp8 one token at a time (token_rows_d over every token)."""
    Xd, W13d, Ws13d = _fp8_operands(x, W13, Ws13)
    Lc = np.concatenate([np.asarray(a, np.float32).reshape(-1, W13.shape[0]) for a in l])
    out, _, _ = token_rows_d(Xd, Lc, np.arange(Xd.shape[0]), W13d, W2, Ws13d, Ws2, K=K, rsf=rsf, renorm=renorm)
    off = np.concatenate([[0], np.cumsum([np.asarray(a).shape[0] for a in x])])
    return [out[off[p]:off[p + 1]] for p in range(len(x))]
