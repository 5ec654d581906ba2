"""The parity checks' own arithmetic, pinned on the CPU: the directed bf16 rounding behind the
admissible extrema (against the oracle's rounding and torch's bf16 grid), the admissible sets,
and the page-set swap rule (a planted swap beyond the tolerance must fail)."""
import numpy as np
import pytest

from oracle import hhr_oracle as orc

import hhr_case as hc


def test_bf16_down_up_matches_the_oracle_on_fp32_values():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        [0.0, -0.0, 1.0, -1.0, 3e38, -3e38, 1e-40, -1e-40]]).astype(np.float32)
    d0, u0 = orc._bf16_neighbours(x)
    d1, u1 = hc.bf16_down_up(x.astype(np.float64))
    assert np.array_equal(d0, d1) and np.array_equal(u0, u1)


def test_bf16_down_up_brackets_float64_values_on_the_bf16_grid():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))
    down, up = hc.bf16_down_up(x)
    assert np.all(down <= x) and np.all(x <= up)
    for v in (down, up):   # both are bf16 values: a bf16 round trip keeps them
        t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(t.astype(np.float64), v)
    # adjacent: no bf16 value strictly between them
    gap = up - down
    e = np.frexp(x)[1] - 1.0
    assert np.all((gap == 0) | (gap == np.exp2(np.maximum(e, -126) - 7)))


def test_admissible_sets_hold_the_rounding_of_nearby_values():
    rng = np.random.default_rng(7)
    lo32 = (rng.standard_normal(5000) * 4).astype(np.float32)
    hi32 = lo32 + np.abs(rng.standard_normal(5000)).astype(np.float32)
    tol = 1e-4
    (lmin, lmax), (hmin, hmax) = hc.admissible_extrema(lo32, hi32, tol, "bf16")
    for shift in (-tol, -tol / 3, 0.0, tol / 2, tol):
        d, _ = hc.bf16_down_up(lo32.astype(np.float64) + shift)
        _, u = hc.bf16_down_up(hi32.astype(np.float64) + shift)
        assert np.all((lmin <= d) & (d <= lmax)) and np.all((hmin <= u) & (u <= hmax))
    # a maximum rounded the wrong way (down) is rejected wherever that moves it more than tol
    # below the fp32 value; likewise a minimum rounded up
    hdown, _ = hc.bf16_down_up(hi32.astype(np.float64))
    far = hi32 - hdown > tol
    assert np.any(far) and np.all(hdown[far] < hmin[far])
    _, lup = hc.bf16_down_up(lo32.astype(np.float64))
    far = lup - lo32 > tol
    assert np.any(far) and np.all(lup[far] > lmax[far])


def test_page_set_rule_accepts_near_ties_and_rejects_far_swaps():
    U = np.array([10.0, 9.0, 8.0, 7.999999, 5.0, 1.0])
    pages = orc.select_pages(U, 3)                      # 0, 1, 2
    tau = np.full(6, 1e-5)
    # swapping page 2 for page 3 (bounds 1e-6 apart) is a near-tie
    assert hc.check_page_set(np.array([0, 1, 3]), pages, U, 3, tau, "near") == 1
    # swapping page 2 for page 4 (3 apart) is not
    with pytest.raises(AssertionError):
        hc.check_page_set(np.array([0, 1, 4]), pages, U, 3, tau, "far")
