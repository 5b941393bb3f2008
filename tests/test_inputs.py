"""Host tests of the seeded input generator against its stated recipe:
seeds 1000*cfg (X) and 1000*cfg + l (W_l), N(0, sigma^2) draws from numpy's
PCG64 in fp64, cast to float32, and for bf16 chains rounded to the nearest
bf16 with ties to even; the standard deviations of each workload; and that
the draw is deterministic and row ranges are slices of the full draw."""
import math

import numpy as np
import pytest

from tile_dependency_pipelined_amd import inputs as gen


def nearest_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values by direct search: of the two bf16
    values that bracket x (the truncation and the next one away from zero),
    take the nearer in fp64, and on a tie the one with an even pattern."""
    u = x32.view(np.uint32).astype(np.uint64)
    lo = (u >> 16).astype(np.uint64)                     # truncated pattern
    hi = lo + 1                                          # next magnitude, same sign
    as_f = lambda p: (p.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    x = x32.astype(np.float64)
    d_lo, d_hi = np.abs(x - as_f(lo)), np.abs(as_f(hi) - x)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_stated_standard_deviations():
    s = lambda fan: 1 / math.sqrt(fan)
    want = {"c1": (1.0, (s(512), s(512))), "c2": (1.0, (1 / 64, 1 / 64)),
            "c3": (1.0, (s(8192), s(8192))), "c4": (1.0, (s(8192),) * 4),
            "c5": (1.0, (s(8192), s(28672)))}
    for key, (xs, ws) in want.items():
        cfg = gen.CONFIGS[key]
        assert cfg.x_std == xs and len(cfg.w_stds) == cfg.n_layers
        assert all(math.isclose(a, b, rel_tol=1e-15) for a, b in zip(cfg.w_stds, ws)), key


@pytest.mark.parametrize("key", ["c1", "c2"])
def test_inputs_follow_the_recipe(key):
    cfg = gen.CONFIGS[key]
    X, Ws = gen.config_inputs(cfg)
    mats = [((cfg.M, cfg.widths[0]), cfg.x_std, 1000 * cfg.cfg_id, X)]
    mats += [((cfg.widths[l], cfg.widths[l + 1]), cfg.w_stds[l], 1000 * cfg.cfg_id + l + 1, Ws[l])
             for l in range(cfg.n_layers)]
    for shape, std, seed, got in mats:
        x32 = (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)
        if cfg.dtype == gen.BF16:
            assert got.dtype == np.uint16
            assert np.array_equal(got, nearest_bf16_bits(x32)), seed
        else:
            assert got.dtype == np.float32
            assert np.array_equal(got.view(np.uint32), x32.view(np.uint32)), seed


def test_rounding_ties_go_to_even():
    # float32 patterns exactly halfway between two bf16 values
    halves = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00008000], dtype=np.uint32)
    got = gen.f32_to_bf16_bits(halves.view(np.float32))
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80, 0xBF82, 0x0000]
    assert np.array_equal(got, nearest_bf16_bits(halves.view(np.float32)))


def test_deterministic_and_row_ranges():
    cfg = gen.CONFIGS["c2"]
    X1, W1 = gen.config_inputs(cfg)
    X2, W2 = gen.config_inputs(cfg)
    assert np.array_equal(X1, X2) and all(np.array_equal(a, b) for a, b in zip(W1, W2))
    Xr, Wr = gen.chain_inputs(cfg.M, cfg.widths, cfg.dtype, cfg.x_std, cfg.w_stds, cfg.cfg_id, rows=(100, 300))
    assert np.array_equal(Xr, X1[100:300]) and all(np.array_equal(a, b) for a, b in zip(Wr, W1))
