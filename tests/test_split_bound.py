"""The error bound behind the K-min prefilter's two-part bf16 split (CPU only).

The D >= 32 K-min prefilter forms <y, -2x> from bf16 parts, v = v_hi + v_lo with
v_hi = bf16(v) and v_lo = bf16(v - v_hi), as <y_hi, w_hi> + <y_hi, w_lo> +
<y_lo, w_hi> (w = -2x), and relies on
  (1) |split - exact| <= 3.01 * 2^-16 * sum_k |y_k| |w_k| (bf16 keeps 8 significant
      bits: |v - v_hi| <= 2^-8 |v|, and the lo part's own rounding is below 2^-16 |v|;
      the dropped lo * lo product and the two lo roundings give 1 + 2 (1 + 2^-8)), and
  (2) 2^-14 (2|x| + s)^2 covering that bound for every y with |y| <= |x| + s,
so that no candidate whose exact distance is below the row's K-th can fail the
prefilter.  Both are checked here on emulated bf16 arithmetic (round to nearest
even, compared with torch's own bfloat16 cast), in float64 so that only the split
itself is measured; the fp32 accumulation has its own separate term in the margin.
"""
import numpy as np
import pytest
import torch

BOUND = 3.01 * 2.0 ** -16
MARGIN = 2.0 ** -14


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split(v: np.ndarray):
    v = v.astype(np.float32)
    hi = bf16_rne(v)
    rem = v - hi                      # exact in fp32: hi carries v's leading 8 bits
    assert np.array_equal(rem.astype(np.float64), v.astype(np.float64) - hi.astype(np.float64))
    return hi, bf16_rne(rem)


def split_dot(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    yh, yl = (p.astype(np.float64) for p in split(y))
    wh, wl = (p.astype(np.float64) for p in split(w))
    return (yh * wh + yh * wl + yl * wh).sum(-1)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000),
                        # exact ties between two bf16 values, both parities
                        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_rne(v), ref)


@pytest.mark.parametrize("D,scale", [(32, 1.0), (50, 0.1414), (64, 5.0), (100, 300.0), (64, 1e-3)])
def test_split_error_within_bound(D, scale):
    rng = np.random.default_rng(D)
    y = (rng.standard_normal((4000, D)) * scale).astype(np.float32)
    w = (-2.0 * rng.standard_normal((4000, D)) * scale).astype(np.float32)
    exact = (y.astype(np.float64) * w.astype(np.float64)).sum(-1)
    err = np.abs(split_dot(y, w) - exact)
    bound = BOUND * (np.abs(y.astype(np.float64)) * np.abs(w.astype(np.float64))).sum(-1)
    assert np.all(err <= bound)
    assert err.max() > 0.0            # the split is not exact, so the check has teeth


def test_split_error_adversarial():
    """Values whose lo parts sit on rounding ties: the largest per-product errors."""
    rng = np.random.default_rng(7)
    # mantissa bits chosen so v - bf16(v) needs more than 8 bits and rounds at a tie
    mant = rng.integers(0, 1 << 23, (3000, 64), dtype=np.uint32) | 0x00008080
    expo = rng.integers(110, 140, (3000, 64), dtype=np.uint32) << 23
    sign = rng.integers(0, 2, (3000, 64), dtype=np.uint32) << 31
    y = (sign | expo | mant).view(np.float32)
    w = np.roll(y, 1, axis=1) * np.float32(-2.0)
    exact = (y.astype(np.float64) * w.astype(np.float64)).sum(-1)
    err = np.abs(split_dot(y, w) - exact)
    bound = BOUND * (np.abs(y.astype(np.float64)) * np.abs(w.astype(np.float64))).sum(-1)
    assert np.all(err <= bound)
    # per product the error stays within the bound too (no cancellation needed)
    yh, yl = split(y[:, :1])
    wh, wl = split(w[:, :1])
    e1 = np.abs(yh.astype(np.float64) * wh + yh.astype(np.float64) * wl + yl.astype(np.float64) * wh
                - y[:, :1].astype(np.float64) * w[:, :1])
    assert np.all(e1 <= BOUND * np.abs(y[:, :1].astype(np.float64) * w[:, :1]))


def test_margin_covers_split_bound():
    """sum_k |y_k||2x_k| <= 2|x||y| <= (2|x| + s)^2 / 2 when |y| <= |x| + s, so the
    pass margin 2^-14 (2|x| + s)^2 is at least 2.5 times the split bound."""
    rng = np.random.default_rng(3)
    for D in (32, 50, 64, 100):
        x = rng.standard_normal((2000, D)) * rng.uniform(0.01, 50.0, (2000, 1))
        s = rng.uniform(0.0, 30.0, 2000)
        u = rng.standard_normal((2000, D))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        y = u * (np.linalg.norm(x, axis=1) + s)[:, None] * rng.uniform(0.0, 1.0, (2000, 1))
        lhs = BOUND * (np.abs(y) * np.abs(2.0 * x)).sum(-1)
        rhs = MARGIN * (2.0 * np.linalg.norm(x, axis=1) + s) ** 2
        assert np.all(2.5 * lhs <= rhs)


def test_kernel_uses_this_margin():
    """The split term of the kernel's pass margin is the MARGIN proven sufficient above."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "geometric_map_reduce_amd", "csrc",
                            "kmin_mfma_split.h")).read()
    m = re.search(r"kmin_split_margin_coef\(int DP\) \{ return kmin_margin_coef\(3 \* DP\) \+ ([0-9.e+-]+)f; \}", src)
    assert m, "margin definition not found"
    assert float(m.group(1)) == MARGIN
