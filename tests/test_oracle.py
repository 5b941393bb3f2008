"""Pins for the CPU oracle, checked against things other than itself.

The pages print no numeric worked example, so every pin here is a closed
form, an invariant, an exact brute force or an independent library routine:
  * exact integer brute force (Python ints) on tiny chains;
  * identity and signed power-of-two permutation weights (exact);
  * row independence, power-of-two linearity (exact);
  * numpy fp64 matmul cross-check and the associativity error bound;
  * bf16 round-to-nearest-even: IEEE closed-form cases and a brute-force
    nearest-neighbour search over all 65536 bf16 values;
  * tanh-GeLU: odd identity gelu(x) - gelu(-x) = x, gelu(0) = 0, the two
    asymptotes, and a 50-digit mpmath evaluation.
A planted mistake anywhere in oracle_chain.c (dropped term, sign, transposed
operand, wrong rounding) fails at least one of them; see test_planted_*.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tile_dependency_pipelined_amd import inputs as gen

F32, BF16 = oracle.F32, oracle.BF16


def as_f64(a, dtype):
    return oracle.bf16_to_f64(a) if dtype == BF16 else np.asarray(a, np.float64)


def int_chain(X, Ws):
    """Exact chain in Python integers (matrices of ints)."""
    H = [[int(v) for v in row] for row in X]
    for W in Ws:
        Wi = [[int(v) for v in row] for row in W]
        H = [[sum(h[k] * Wi[k][j] for k in range(len(Wi))) for j in range(len(Wi[0]))]
             for h in H]
    return H


# --------------------------------------------------------------------------- GEMM core

@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("seed", range(6))
def test_exact_integer_bruteforce(dtype, seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 4))
    widths = [int(rng.integers(1, 17)) for _ in range(L + 1)]
    M = int(rng.integers(1, 17))
    X = gen.small_int_matrix((M, widths[0]), 10 * seed, dtype)
    Ws = [gen.small_int_matrix((widths[l], widths[l + 1]), 10 * seed + l + 1, dtype)
          for l in range(L)]
    Y = oracle.chain(X, Ws, dtype, round_intermediates=False)
    ref = int_chain(as_f64(X, dtype), [as_f64(w, dtype) for w in Ws])
    assert np.array_equal(Y, np.array(ref, dtype=np.float64))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_exact_integer_with_storage_rounding(dtype):
    # entries in {-2..2} and contraction length 4: every intermediate is an
    # integer of magnitude <= 128, exactly representable in bf16 and fp32, so
    # rounding the stored intermediates must change nothing.
    M, widths = 9, [4, 4, 4, 4]
    X = gen.small_int_matrix((M, 4), 77, dtype, -2, 2)
    Ws = [gen.small_int_matrix((4, 4), 78 + l, dtype, -2, 2) for l in range(3)]
    Y, Hs = oracle.chain(X, Ws, dtype, round_intermediates=True, return_intermediates=True)
    ref = int_chain(as_f64(X, dtype), [as_f64(w, dtype) for w in Ws])
    assert np.array_equal(Y, np.array(ref, dtype=np.float64))
    assert np.array_equal(Hs[0], np.array(int_chain(as_f64(X, dtype), [as_f64(Ws[0], dtype)]),
                                          dtype=np.float64))


def test_numpy_crosscheck_fp32():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((17, 40)).astype(np.float32)
    Ws = [(rng.standard_normal((40, 24)) / 6).astype(np.float32),
          (rng.standard_normal((24, 33)) / 5).astype(np.float32)]
    Y = oracle.chain(X, Ws, F32, round_intermediates=False)
    ref = (X.astype(np.float64) @ Ws[0].astype(np.float64)) @ Ws[1].astype(np.float64)
    assert np.max(np.abs(Y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_associativity_bound_bf16():
    rng = np.random.default_rng(4)
    K = 64
    X = gen.f32_to_bf16_bits(rng.standard_normal((8, K)).astype(np.float32))
    W1 = gen.f32_to_bf16_bits((rng.standard_normal((K, K)) / 8).astype(np.float32))
    W2 = gen.f32_to_bf16_bits((rng.standard_normal((K, K)) / 8).astype(np.float32))
    Y = oracle.chain(X, [W1, W2], BF16, round_intermediates=False)
    x, w1, w2 = (oracle.bf16_to_f64(a) for a in (X, W1, W2))
    alt = x @ (w1 @ w2)
    bound = 4 * K * K * np.finfo(np.float64).eps * (np.abs(x) @ np.abs(w1) @ np.abs(w2))
    assert np.all(np.abs(Y - alt) <= bound)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_identity_weights(dtype):
    X = gen.normal_matrix((12, 32), 1.0, 5, dtype)
    I = np.eye(32, dtype=np.float32)
    I = gen.f32_to_bf16_bits(I) if dtype == BF16 else I
    Y = oracle.chain(X, [I, I, I], dtype, round_intermediates=True)
    assert np.array_equal(Y, as_f64(X, dtype))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_signed_permutation_weights(dtype):
    n = 48
    X = gen.normal_matrix((10, n), 1.0, 6, dtype)
    P1 = gen.signed_permutation(n, 1, dtype, scale_pow2=1)
    P2 = gen.signed_permutation(n, 2, dtype, scale_pow2=-3)
    Y = oracle.chain(X, [P1, P2], dtype, round_intermediates=True)
    # X P (P signed permutation): column j of the product = sign * X[:, i]
    # where P[i, j] != 0 -- computed by indexing, no multiplication-add.
    x = as_f64(X, dtype)
    for P in (P1, P2):
        p = as_f64(P, dtype)
        src = np.argmax(np.abs(p), axis=0)
        x = x[:, src] * p[src, np.arange(n)]
    assert np.array_equal(Y, x)


def test_row_independence_and_row_subset():
    X, Ws = gen.chain_inputs(24, (64, 48, 32), BF16, 1.0, (0.125, 0.125), 9)
    Y = oracle.chain(X, Ws, BF16)
    perm = np.random.default_rng(0).permutation(24)
    Yp = oracle.chain(np.ascontiguousarray(X[perm]), Ws, BF16)
    assert np.array_equal(Yp, Y[perm])
    rows = np.array([23, 0, 7, 7, 11])
    assert np.array_equal(oracle.chain(X, Ws, BF16, rows=rows), Y[rows])


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_power_of_two_linearity(dtype):
    X, Ws = gen.chain_inputs(16, (32, 32, 32), dtype, 1.0, (0.2, 0.2), 11)
    Y = oracle.chain(X, Ws, dtype)
    if dtype == BF16:
        X4 = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(X) * np.float32(4.0))
    else:
        X4 = X * np.float32(4.0)
    Y4 = oracle.chain(X4, Ws, dtype)
    assert np.array_equal(Y4, 4.0 * Y)


def test_block_diagonal_splits():
    rng = np.random.default_rng(12)
    a = (rng.standard_normal((6, 8)) / 2).astype(np.float32)
    b = (rng.standard_normal((8, 8)) / 2).astype(np.float32)
    X = rng.standard_normal((5, 12)).astype(np.float32)
    W1 = np.zeros((12, 16), np.float32); W1[:6, :8] = a; W1[6:, 8:] = a
    W2 = np.zeros((16, 16), np.float32); W2[:8, :8] = b; W2[8:, 8:] = b
    Y = oracle.chain(X, [W1, W2], F32)
    left = oracle.chain(np.ascontiguousarray(X[:, :6]), [a, b], F32)
    right = oracle.chain(np.ascontiguousarray(X[:, 6:]), [a, b], F32)
    assert np.array_equal(Y, np.hstack([left, right]))


def test_rejects_bad_arguments():
    X = np.zeros((4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.chain(X, [np.zeros((7, 8), np.float32)], F32)
    with pytest.raises(ValueError):
        oracle.chain(X, [np.zeros((8, 8), np.float32)], F32, rows=[4])
    with pytest.raises(TypeError):
        oracle.chain(X, [np.zeros((8, 8), np.float32)], BF16)


# --------------------------------------------------------------------------- bf16 rounding

def _all_bf16_values():
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    finite = np.isfinite(vals)
    pairs = sorted((Fraction(float(v)), int(b)) for v, b in zip(vals[finite], bits[finite])
                   if not (v == 0 and b == 0x8000))
    return pairs


_BF16_TABLE = None


def brute_round_bf16(x: float) -> int:
    """Nearest finite bf16 by exhaustive search; ties go to the even bit pattern;
    beyond the largest finite value by half an ulp or more -> infinity."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = _all_bf16_values()
    keys = [p[0] for p in _BF16_TABLE]
    fx = Fraction(x)
    top = keys[-1]
    half_ulp_top = (top - keys[-2]) / 2
    if fx >= top + half_ulp_top:
        return 0x7F80
    if fx <= -top - half_ulp_top:
        return 0xFF80
    k = bisect.bisect_left(keys, fx)
    cands = [c for c in (k - 1, k) if 0 <= c < len(keys)]
    best = min(cands, key=lambda c: (abs(keys[c] - fx), _BF16_TABLE[c][1] & 1))
    b = _BF16_TABLE[best][1]
    if keys[best] == 0 and x < 0:
        b = 0x8000
    return b


def test_bf16_rounding_closed_forms():
    cases = [
        (1.0, 0x3F80),
        (1 + 2.0 ** -8, 0x3F80),                  # tie between 1 and 1+2^-7 -> even (1)
        (1 + 3 * 2.0 ** -8, 0x3F82),              # tie between 0x3F81 and 0x3F82 -> even
        (1 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),     # just above the tie
        (-2.5, 0xC020),
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie with zero -> even (zero)
        (3 * 2.0 ** -134, 0x0002),                 # tie 0x0001 / 0x0002 -> even
        (255 * 2.0 ** 120, 0x7F7F),                # largest finite
        (511 * 2.0 ** 119, 0x7F80),                # tie above the largest finite -> inf
        (-0.0, 0x8000),
        (float("inf"), 0x7F80),
    ]
    got = oracle.round_bf16([c[0] for c in cases])
    for (x, want), g in zip(cases, got):
        assert int(g) == want, (x, hex(int(g)), hex(want))


def test_bf16_rounding_bruteforce():
    rng = np.random.default_rng(21)
    xs = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.integers(-40, 39, 300),
        # exact midpoints between neighbours and their immediate neighbours
        (gen.bf16_bits_to_f32(rng.integers(0, 0x7F00, 200).astype(np.uint16)).astype(np.float64)
         * (1 + 2.0 ** -8)),
    ])
    got = oracle.round_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == brute_round_bf16(float(x)), x


def test_bf16_rounding_agrees_with_float32_path():
    # For float32 inputs, fp64->bf16 RNE equals the bit-trick float32->bf16 RNE
    # of the input generator (a separate implementation).
    a = np.random.default_rng(5).standard_normal(20000).astype(np.float32)
    assert np.array_equal(oracle.round_bf16(a.astype(np.float64)), gen.f32_to_bf16_bits(a))


# --------------------------------------------------------------------------- GeLU

def test_gelu_odd_identity_and_limits():
    x = np.linspace(-12, 12, 4001)
    g, gm = oracle.gelu_tanh(x), oracle.gelu_tanh(-x)
    # tanh is odd, so gelu(x) - gelu(-x) = x/2 (1+t) + x/2 (1-t) = x
    assert np.all(np.abs((g - gm) - x) <= 8 * np.finfo(np.float64).eps * np.maximum(1, np.abs(x)))
    assert oracle.gelu_tanh([0.0])[0] == 0.0
    big = np.array([10.0, 20.0, 40.0])
    assert np.all(np.abs(oracle.gelu_tanh(big) - big) <= 1e-14 * big)
    neg = oracle.gelu_tanh(-big)
    assert np.all(neg <= 0) and np.all(neg > -1e-12)
    # monotone beyond the minimum near x ~ -0.75
    xs = np.linspace(-0.5, 6, 1000)
    assert np.all(np.diff(oracle.gelu_tanh(xs)) > 0)


def test_gelu_against_mpmath():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    xs = [-6.0, -3.0, -1.0, -0.5, -0.1, 0.1, 0.5, 1.0, 2.0, 3.5, 7.0]
    got = oracle.gelu_tanh(xs)
    for x, g in zip(xs, got):
        mx = mpmath.mpf(x)
        ref = mx / 2 * (1 + mpmath.tanh(mpmath.sqrt(2 / mpmath.pi) * (mx + mpmath.mpf("0.044715") * mx ** 3)))
        # 1 + tanh(u) cancels for x << 0, so the fp64 evaluation is accurate
        # to a few ulps of |x| (the scale the chain compares at), not of gelu(x)
        assert abs(g - float(ref)) <= 4 * np.finfo(np.float64).eps * max(abs(x), abs(float(ref)))


def test_gelu_in_chain_applies_before_rounding():
    # identity weights: Y = round_bf16(gelu(X)) . I  exactly
    X = gen.normal_matrix((6, 16), 2.0, 31, BF16)
    I = gen.f32_to_bf16_bits(np.eye(16, dtype=np.float32))
    Y = oracle.chain(X, [I, I], BF16, acts=[oracle.ACT_GELU_TANH, oracle.ACT_NONE])
    want = oracle.bf16_to_f64(oracle.round_bf16(oracle.gelu_tanh(oracle.bf16_to_f64(X))))
    assert np.array_equal(Y, want)


def test_rel_err_metric():
    assert oracle.rel_err([1.0, -2.0], [1.0, -2.0]) == 0.0
    assert oracle.rel_err([1.5, -2.0], [1.0, -2.0]) == 0.25
