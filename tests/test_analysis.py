"""Host analysis tools: the three-term MSE model of block quantization ("Is
Finer Better? The Limits of Microscaling Formats in LLMs", theoretical
framework) and the MSE-optimised scale search ("Bridging the Gap Between
Promise and Performance for Microscaling FP4 Quantization", Sec. 2.2).

The model is pinned to Monte-Carlo errors of the oracle quantizer on the same
distributions, which it computes by a different route (integration over the
block maximum instead of quantizing samples); the search to the oracle's
round-to-nearest error and to an exhaustive search on single blocks.
"""
import warnings

import numpy as np
import pytest

import oracle
from microscaling_block_quantization_amd import analysis as A

warnings.filterwarnings("ignore", category=RuntimeWarning)

SCALE_CODE = {"e8m0": oracle.SC_E8M0, "ue4m3": oracle.SC_UE4M3, "ue5m3": oracle.SC_UE5M3}


def mc_mse(sigma, block, scale, n=1 << 20, seed=1):
    x = (np.random.default_rng(seed).standard_normal(n) * sigma).astype(np.float32).reshape(1024, -1)
    st = oracle.quantize(x, oracle.Format(scale=SCALE_CODE[scale], block_cols=block))["stats"]
    return st["err2"] / st["n"]


def test_e2m1_round_ties_and_saturation():
    # ties go to the even code; 5 -> 4 is the 20 % case of the 4..6 gap
    got = A.e2m1_round([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.9, 7.0, 8.0, -0.3, -5.1])
    assert list(got) == [0, 1, 1, 2, 2, 4, 4, 6, 6, 6, -0.5, -6]


def test_scale_rounding_formats():
    # UE4M3: smallest 2^-9, smallest normal 2^-6, max 448; UE5M3: smallest 2^-17
    assert A.scale_round(np.array([2.0 ** -9, 2.0 ** -10, 2.0 ** -10 * 1.01, 500.0]), "ue4m3").tolist() == \
        [2.0 ** -9, 0.0, 2.0 ** -9, 448.0]
    assert A.scale_round(np.array([2.0 ** -17, 2.0 ** -18]), "ue5m3").tolist() == [2.0 ** -17, 0.0]


@pytest.mark.parametrize("sigma,scale,block", [(1.0, "e8m0", 8), (1.0, "e8m0", 64), (2e-2, "ue4m3", 16),
                                               (3e-3, "ue4m3", 16), (1e-3, "ue4m3", 16), (1e-3, "ue5m3", 64)])
def test_mse_model_matches_oracle(sigma, scale, block):
    model = A.mse_model(sigma, block, scale)["total"]
    assert abs(model - mc_mse(sigma, block, scale)) <= 0.02 * model


def test_mse_model_three_parts():
    # E8M0 never rounds a scale to zero
    p = A.mse_model(1.0, 32, "e8m0")
    assert p["zero"] == 0.0 and p["max"] > 0 and p["nonmax"] > p["max"]
    # sigma = 1e-3 under UE4M3 without a tensor scale: block maxima near 3e-3
    # need a scale of ~5e-4, below half of 2^-9, so nearly every block rounds
    # to zero and the error is the signal energy sigma^2
    p = A.mse_model(1e-3, 16, "ue4m3")
    assert p["zero"] > 0.99 * p["total"] and abs(p["total"] - 1e-6) < 1e-8
    # UE5M3 reaches 2^-17: the same data keeps its blocks
    p = A.mse_model(1e-3, 16, "ue5m3")
    assert p["zero"] < 1e-6 * p["total"]
    # a tensor scale (NVFP4) removes the zero rounding as well
    p = A.mse_model(1e-3, 16, "ue4m3", tensor_scale=6e-3 / 2688)
    assert p["zero"] < 1e-6 * p["total"]


def test_inversion_narrow_distributions():
    """UE4M3 without a tensor scale: halving the block from 16 to 8 raises the
    error of narrow distributions (sigma = 3e-3) but not of wider ones
    (sigma = 2e-2); UE5M3 shows no inversion at the narrow width.  The model's
    verdicts agree with the oracle's Monte-Carlo errors."""
    for sigma, inverted in ((3e-3, True), (2e-2, False)):
        inv = A.inversions(sigma, (8, 16), "ue4m3")[0]
        assert inv["inverted"] == inverted
        assert (mc_mse(sigma, 8, "ue4m3") > mc_mse(sigma, 16, "ue4m3")) == inverted
    assert not any(r["inverted"] for r in A.inversions(3e-3, (8, 16, 32), "ue5m3"))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_scale_search_improves_on_round_to_nearest(fmt):
    w = np.random.default_rng(3).laplace(size=(64, 512)).astype(np.float32)
    r = A.mse_scale_search(w, fmt)
    if fmt == "mxfp4":
        rtn = oracle.quantize(w, oracle.Format())["stats"]
    else:
        rtn = oracle.quantize(w, oracle.Format(scale=oracle.SC_NVFP4, block_cols=16))["stats"]
    h = r["mse_history"]
    # the starting point is the round-to-nearest quantizer, and no step raises the error
    # (NVFP4: the oracle dequantizes in fp32, q * s_b then times g, this tool in fp64)
    assert abs(h[0] - rtn["err2"] / rtn["n"]) <= (1e-9 if fmt == "mxfp4" else 1e-6) * h[0]
    assert all(b <= a for a, b in zip(h, h[1:]))
    assert h[-1] < 0.97 * h[0]
    # the returned dequantization is the last error
    assert abs(np.mean((r["dequant"] - w.astype(np.float64)) ** 2) - h[-1]) <= 1e-12
    # group scales are of the format: powers of two, or UE4M3 values
    gs = r["group_scales"]
    if fmt == "mxfp4":
        assert np.all(np.exp2(np.round(np.log2(gs))) == gs)
    else:
        assert set(np.unique(gs)) <= set(A._e4m3_grid())


def test_scale_search_finds_block_optimum():
    """One step of the group search with the global scale fixed picks, for each
    block, the E8M0 scale with the smallest error among all scales within 10
    binades of the FLOOR choice."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((40, 32)) * np.exp2(rng.integers(-6, 6, (40, 1)))).astype(np.float32)
    r = A.mse_scale_search(w, "mxfp4", iters=1, nglobal=0)
    for i in range(w.shape[0]):
        x = w[i].astype(np.float64)
        e0 = np.floor(np.log2(np.abs(x).max())) - 2
        errs = {e: np.sum((x - A.e2m1_round(x / 2.0 ** e) * 2.0 ** e) ** 2) for e in np.arange(e0 - 10, e0 + 11)}
        best = min(errs.values())
        got = np.sum((x - r["dequant"][i]) ** 2)
        assert got == best
