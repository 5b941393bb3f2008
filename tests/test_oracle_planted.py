"""Planted mistakes: each mutation of oracle_chain.c below is a plausible bug
(dropped term, wrong sign, transposed operand, wrong rounding rule, GeLU
constant or placement, skipped storage rounding).  The mutated copy is built
on the CPU and must fail at least one pin of the battery; the unmutated
source must pass all of them.  This shows the pins constrain the oracle."""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from tile_dependency_pipelined_amd import inputs as gen

F32, BF16 = oracle.F32, oracle.BF16

MUTATIONS = [
    ("sign of the accumulation", "nxt[j] += a * load_elem", "nxt[j] -= a * load_elem"),
    ("dropped first k term", "for (int64_t k = 0; k < K; ++k) {          /* i-k-j order */",
     "for (int64_t k = 1; k < K; ++k) {"),
    ("transposed weight operand", "load_elem(Wl, k * N + j, dtype)", "load_elem(Wl, j * K + k, dtype)"),
    ("rounding by truncation", "nearbyint(x / q)", "trunc(x / q)"),
    ("rounding ties away from zero", "nearbyint(x / q)", "round(x / q)"),
    ("bf16 keeps one bit too many", "int qexp = e - 8;", "int qexp = e - 9;"),
    ("GeLU cubic constant", "0.044715 * x * x * x", "0.04715 * x * x * x"),
    ("GeLU missing half", "return 0.5 * x * (1.0 + tanh", "return x * (1.0 + tanh"),
    ("activation skipped", "nxt[j] = oracle_gelu_tanh(nxt[j]);", "nxt[j] = nxt[j];"),
    ("intermediates not rounded", "nxt[j] = round_storage(nxt[j], dtype);", "nxt[j] = nxt[j];"),
    ("fp32 storage rounds to bf16", "return (double)(float)x;",
     "return bf16_bits_to_f64(oracle_round_bf16(x));"),
]


def pin_battery(o: oracle.Oracle):
    """A compact battery of the pins in test_oracle.py; returns failed names."""
    failed = []

    def check(name, cond):
        if not cond:
            failed.append(name)

    # exact integers, non-square shapes
    for dtype in (F32, BF16):
        X = gen.small_int_matrix((5, 7), 1, dtype)
        W1 = gen.small_int_matrix((7, 3), 2, dtype)
        W2 = gen.small_int_matrix((3, 6), 3, dtype)
        x, w1, w2 = (np.array(oracle.bf16_to_f64(a) if dtype == BF16 else a, dtype=object)
                     for a in (X, W1, W2))
        ref = np.array((x.dot(w1)).dot(w2), dtype=np.float64)
        check(f"int-{dtype}", np.array_equal(o.chain(X, [W1, W2], dtype, round_intermediates=False), ref))
    # storage rounding: a value between bf16 neighbours must come back rounded
    X = gen.f32_to_bf16_bits(np.array([[1.0, 2.0 ** -8 + 2.0 ** -12]], np.float32))
    W1 = gen.f32_to_bf16_bits(np.array([[1.0], [1.0]], np.float32))
    W2 = gen.f32_to_bf16_bits(np.array([[1.0]], np.float32))
    check("bf16-storage", o.chain(X, [W1, W2], BF16)[0, 0] == 1.0 + 2.0 ** -7)
    # fp32 storage: 1 + 2^-30 rounds to 1, 1 + 2^-20 is kept (bf16 would drop it)
    Xf = np.array([[1.0, 2.0 ** -30], [1.0, 2.0 ** -20]], np.float32)
    Wf1 = np.array([[1.0], [1.0]], np.float32)
    yf = o.chain(Xf, [Wf1, np.array([[1.0]], np.float32)], F32)[:, 0]
    check("f32-storage", yf[0] == 1.0 and yf[1] == 1.0 + 2.0 ** -20)
    # signed permutation, square
    n = 16
    for dtype in (F32, BF16):
        X = gen.normal_matrix((4, n), 1.0, 6, dtype)
        P = gen.signed_permutation(n, 1, dtype, scale_pow2=1)
        p = oracle.bf16_to_f64(P) if dtype == BF16 else P.astype(np.float64)
        x = oracle.bf16_to_f64(X) if dtype == BF16 else X.astype(np.float64)
        src = np.argmax(np.abs(p), axis=0)
        check(f"perm-{dtype}", np.array_equal(o.chain(X, [P], dtype), x[:, src] * p[src, np.arange(n)]))
    # rounding closed forms
    cases = [(1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82), (-(1 + 3 * 2.0 ** -8), 0xBF82),
             (1 + 2.0 ** -8 + 2.0 ** -30, 0x3F81), (2.0 ** -134, 0), (1.0 + 2.0 ** -9, 0x3F80)]
    got = o.round_bf16([c[0] for c in cases])
    check("rne", all(int(g) == w for (_, w), g in zip(cases, got)))
    # GeLU odd identity and asymptote, and inside a chain
    xs = np.linspace(-5, 5, 101)
    g = o.gelu_tanh(xs) - o.gelu_tanh(-xs)
    check("gelu-odd", np.all(np.abs(g - xs) <= 1e-13 * np.maximum(1, np.abs(xs))))
    check("gelu-asym", abs(o.gelu_tanh([10.0])[0] - 10.0) < 1e-12)
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 40
    v = mp.mpf(1) / 2 * (1 + mp.tanh(mp.sqrt(2 / mp.pi) * (1 + mp.mpf("0.044715"))))
    check("gelu-mpmath", abs(o.gelu_tanh([1.0])[0] - float(v)) < 1e-14)
    I = gen.f32_to_bf16_bits(np.eye(4, dtype=np.float32))
    Xg = gen.f32_to_bf16_bits(np.array([[-1.0, 0.5, 2.0, 3.0]], np.float32))
    yg = o.chain(Xg, [I, I], BF16, acts=[oracle.ACT_GELU_TANH, oracle.ACT_NONE])
    check("gelu-chain", not np.array_equal(yg, oracle.bf16_to_f64(Xg)))
    return failed


def test_unmutated_source_passes_battery():
    assert pin_battery(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mutant = os.path.join(tmp_path, "mutant.c")
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.build(src=mutant, lib=os.path.join(tmp_path, "libmutant.so"))
    failed = pin_battery(oracle.Oracle(lib))
    assert failed, f"planted mistake '{name}' passed every pin"
