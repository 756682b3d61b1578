"""Property tests of the CPU oracle over generated inputs (hypothesis, CPU only).

Each property is fixed by the pages or by the mathematics, not by the oracle's
own code: the nearest-code rule in exact rational arithmetic, the error bound
that the nearest code implies, the range and rounding of the 8-bit scales,
power-of-two scale invariance of the relative error, the total order of the
top-K cut, and the adjoint identities that tie the backward pass to the
forward pass of the linear map.  Examples are derandomized, so every run draws
the same cases.
"""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests import pins

PROFILE = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                   suppress_health_check=[HealthCheck.too_slow])

KINDS = ("normal", "t3", "outliers", "spike", "zero", "subnormal", "ties", "constant")


def make_blocks(kind: str, seed: int, nblocks: int, exp: int, codebook: str = "nf4") -> np.ndarray:
    """nblocks x 64 fp32 weights of one distribution, scaled by 2**exp."""
    rng = np.random.default_rng(seed)
    n = nblocks * 64
    if kind == "normal":
        w = rng.standard_normal(n)
    elif kind == "t3":
        w = rng.standard_t(3, n)
    elif kind == "outliers":
        w = rng.standard_normal(n)
        hit = rng.random(n) < 0.02
        w[hit] *= 50.0
    elif kind == "spike":
        w = np.zeros(n)
        w[rng.integers(0, 64, nblocks) + 64 * np.arange(nblocks)] = rng.choice([-1.0, 1.0], nblocks) * 3.5
    elif kind == "zero":
        w = np.zeros(n)
    elif kind == "subnormal":
        w = rng.standard_normal(n) * 1e-39
    elif kind == "ties":
        # every weight an exact midpoint of two codebook values times the block's absmax
        t = oracle.codebook_table(codebook).astype(np.float64)
        mids = (t[:-1] + t[1:]) / 2
        w = rng.choice(mids, n)
        w[::64] = 1.0
    else:  # constant
        w = np.full(n, 0.3)
    return (w * 2.0 ** exp).astype(np.float32)


block_cases = st.tuples(st.sampled_from(KINDS), st.integers(0, 2**31 - 1), st.integers(1, 5), st.integers(-20, 20))


@PROFILE
@given(block_cases, st.sampled_from(["nf4", "fp4", "int4"]))
def test_encoder_is_nearest_code(case, codebook):
    """Codes and absmax equal the nearest-code rule worked out in exact rationals
    ("1. NormalFloat": absmax scaling, then the nearest of the 16 values; lower code on a tie)."""
    kind, seed, nb, exp = case
    W = make_blocks(kind, seed, nb, exp, codebook).reshape(1, -1)
    q = oracle.quantize(W, 64, 0, codebook)
    table = oracle.codebook_table(codebook)
    for b in range(nb):
        codes, a = pins.brute_codes(W[0, 64 * b:64 * (b + 1)], table)
        assert list(q.codes[64 * b:64 * (b + 1)]) == codes, (kind, b)
        assert np.float32(q.absmax[b]) == a


@PROFILE
@given(block_cases)
def test_dequant_error_bound_and_sign(case):
    """|w - w_hat| is at most half the widest gap between neighbouring code values times
    the block's absmax (plus fp32 rounding), and w_hat never has the opposite sign of w."""
    kind, seed, nb, exp = case
    W = make_blocks(kind, seed, nb, exp).reshape(1, -1)
    q = oracle.quantize(W, 64)
    wh = oracle.dequantize(q).astype(np.float64).reshape(-1, 64)
    w = W.astype(np.float64).reshape(-1, 64)
    t = oracle.codebook_table("nf4").astype(np.float64)
    half_gap = np.max(np.diff(t)) / 2
    a = np.max(np.abs(w), axis=1, keepdims=True)
    assert np.all(np.abs(w - wh) <= a * half_gap * (1 + 2.0 ** -20) + 1e-45)
    assert np.all(w * wh >= 0)
    assert np.all(wh[a[:, 0] == 0] == 0)


@PROFILE
@given(block_cases, st.integers(1, 8))
def test_dq_scales(case, gblocks):
    """Double quantization ("2. Double quantization"): the codes are those of the plain
    quantizer, c8 is in 0..255, and c8 * S_g is within S_g / 2 (plus fp32 rounding) of the
    block's absmax, S_g being the group's largest absmax over 255."""
    kind, seed, nb, exp = case
    W = make_blocks(kind, seed, nb, exp).reshape(1, -1)
    q0 = oracle.quantize(W, 64)
    q = oracle.quantize(W, 64, gblocks)
    assert np.array_equal(q.codes, q0.codes)
    g = np.arange(nb) // gblocks
    S = q.dq_scale[g].astype(np.float64)
    a = q0.absmax.astype(np.float64)
    for i in range(nb):
        assert S[i] == np.float32(np.float32(a[g == g[i]].max()) / np.float32(255))
    c8 = q.c8.astype(np.float64)
    assert np.all((c8 >= 0) & (c8 <= 255))
    # with a normal S_g its fp32 rounding is relative 2^-24, so a / S_g <= 255 (1 + 2^-23)
    # and the rounding to c8 lands within half a step; a subnormal S_g can round far down,
    # and then the code saturates at 255
    normal = S >= 2.0 ** -126
    assert np.all(np.abs(c8[normal] * S[normal] - a[normal]) <= S[normal] * (0.5 + 2.0 ** -16))
    sub = (S > 0) & ~normal
    quot = (a[sub].astype(np.float32) / S[sub].astype(np.float32)).astype(np.float64)
    assert np.all(c8[sub] == np.minimum(255, np.rint(quot)))
    assert np.all(c8[S == 0] == 0)


@PROFILE
@given(st.sampled_from(("normal", "t3", "outliers", "spike", "constant")), st.integers(0, 2**31 - 1),
       st.integers(1, 4), st.integers(-12, 12), st.sampled_from([0, 2]))
def test_error_power_of_two_invariance(kind, seed, nb, k, dq):
    """The relative Frobenius error (AQLoRA section 3.1, the reading taken) does not change
    when W is scaled by a power of two: every step of the format scales exactly."""
    W = make_blocks(kind, seed, nb, 0).reshape(1, -1)
    e0 = oracle.layer_error(W, 64, dq)
    e1 = oracle.layer_error((W * np.float32(2.0 ** k)).astype(np.float32), 64, dq)
    assert e0 == e1
    assert 0.0 <= e0 < 1.0


def topk_brute(e, k):
    """The k layers that no more than k - 1 others beat, by the pages' cut (largest first,
    ties to the lower index) with a NaN error above every number."""
    def beats(j, i):
        nj, ni = math.isnan(e[j]), math.isnan(e[i])
        if nj != ni:
            return nj
        if nj or e[j] == e[i]:
            return j < i
        return e[j] > e[i]
    rank = [sum(beats(j, i) for j in range(len(e))) for i in range(len(e))]
    return [rank.index(p) for p in range(k)]


@PROFILE
@given(st.lists(st.one_of(st.sampled_from([0.0, 0.125, 0.5, float("nan")]),
                          st.floats(0, 1, allow_nan=False)), min_size=0, max_size=40),
       st.integers(0, 40))
def test_topk_is_the_rank_order(errors, k):
    k = min(k, len(errors))
    assert oracle.topk(errors, k) == topk_brute(errors, k)


layer_shapes = st.tuples(st.integers(1, 9), st.integers(1, 3), st.integers(1, 70), st.integers(1, 12),
                         st.sampled_from([0.5, 1.0, 2.0, 3.0]), st.integers(0, 2**31 - 1))


@PROFILE
@given(layer_shapes)
def test_backward_is_the_adjoint_of_forward(shape):
    """Equation (3) is linear in X, in L1 and in L2 (the others fixed), so the backward pass
    must satisfy <dY, Y(X)> = <dX, X>, <dY, s X L1 L2> = <dL1, L1> = <dL2, L2>."""
    M, hb, o, r, s, seed = shape
    h = 64 * hb
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    W = rng.standard_normal((o, h)) * 0.05
    L1 = rng.standard_normal((h, r)) * 0.1
    L2 = rng.standard_normal((r, o)) * 0.1
    dY = rng.standard_normal((M, o))
    Y, T = oracle.fwd(X, W, L1, L2, s)
    dX, dL1, dL2, G = oracle.bwd(X, dY, W, L1, L2, s)
    Ya, _ = oracle.fwd(X, np.zeros_like(W), L1, L2, s)   # the adapter term alone

    def close(a, b, scale):
        assert abs(a - b) <= 1e-11 * scale, (a, b)

    close(float(np.sum(dY * Y)), float(np.sum(dX * X)), np.abs(dY).sum() * np.abs(Y).max() + 1.0)
    ref = float(np.sum(dY * Ya))
    scale = np.abs(dY).sum() * np.abs(Ya).max() + 1.0
    close(ref, float(np.sum(dL1 * L1)), scale)
    close(ref, float(np.sum(dL2 * L2)), scale)
    assert np.allclose(G, s * dY @ L2.T, rtol=0, atol=1e-12 * (np.abs(dY).max() * np.abs(L2).sum() + 1))


def test_planted_transpose_breaks_the_adjoint():
    """A backward with the adapter factors' roles swapped (dL1 formed with dY L2 instead of
    dY L2^T, as if L2 were stored transposed) fails the identity the property checks."""
    rng = np.random.default_rng(5)
    M, h, o, r, s = 7, 64, 64, 3, 2.0
    X = rng.standard_normal((M, h))
    L1 = rng.standard_normal((h, r)) * 0.1
    L2 = rng.standard_normal((r, o)) * 0.1
    dY = rng.standard_normal((M, o))
    Ya, _ = oracle.fwd(X, np.zeros((o, h)), L1, L2, s)
    bad_G = s * dY @ L2.T[:, ::-1]            # columns of G permuted: a wrong index
    bad_dL1 = X.T @ bad_G
    assert abs(float(np.sum(dY * Ya)) - float(np.sum(bad_dL1 * L1))) > 1e-6
