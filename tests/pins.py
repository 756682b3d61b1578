"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes the oracle functions it checks as arguments (defaulting to the
oracle's own), so the planted-mistake tests can hand it a broken variant and
confirm that the pin fails.  Nothing here re-types an oracle formula and
compares the two: the checks are exact rational brute force, closed forms,
invariants, special cases and finite differences.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import nf4 as onf4
from oracle import lora as olora


# ---------------------------------------------------------------------------
# exact helpers (rationals; independent of the oracle's numpy arithmetic)
# ---------------------------------------------------------------------------

def fr(v) -> Fraction:
    return Fraction(float(v))


def f32_nearest(x: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational, ties to the even significand."""
    a = np.float32(float(x))
    cands = {np.float32(a), np.nextafter(a, np.float32(-np.inf)), np.nextafter(a, np.float32(np.inf))}
    def key(c):
        bits = int(np.array(c, dtype=np.float32).view(np.uint32))
        return (abs(fr(c) - x), bits & 1)
    return min(cands, key=key)


def nearest_code(x: np.float32, table) -> int:
    d = [abs(fr(x) - fr(t)) for t in table]
    m = min(d)
    return d.index(m)           # first minimum: the lower code wins a tie


def brute_codes(block: np.ndarray, table) -> tuple[list[int], np.float32]:
    a = max(abs(fr(w)) for w in block)
    if a == 0:
        return [nearest_code(np.float32(0), table)] * len(block), np.float32(0)
    out = []
    for w in block:
        x = f32_nearest(fr(w) / a)
        out.append(nearest_code(x, table))
    return out, np.float32(float(a))


def phi(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def inv_phi_bisect(p: float) -> float:
    """Normal quantile by bisection on math.erfc (independent of the oracle's routine)."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 0:
            break
    return 0.5 * (lo + hi)


def table_from_quantile(inv) -> np.ndarray:
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    z = inv(delta)
    vals = [inv(delta - j * (delta - 0.5) / 8.0) / z for j in range(8)]
    vals += [-inv(delta - j * (delta - 0.5) / 7.0) / z for j in range(7)]
    vals.append(0.0)
    return np.array(sorted(vals), dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# P1: the code table
# ---------------------------------------------------------------------------

def pin_table_structure(table_fn=onf4.nf4_table):
    t = table_fn()
    assert t.dtype == np.float32 and t.shape == (16,)
    assert t[0] == np.float32(-1.0) and t[15] == np.float32(1.0)
    assert t[7] == np.float32(0.0) and not np.signbit(t[7])
    assert np.all(np.diff(t.astype(np.float64)) > 0), "strictly increasing"
    assert int(np.sum(t < 0)) == 7 and int(np.sum(t > 0)) == 8
    # denser near zero (a normal-shaped layout): gaps grow outward on each side
    g = np.diff(t.astype(np.float64))
    assert np.all(np.diff(g[7:]) > 0), "positive side spacing grows away from 0"
    assert np.all(np.diff(g[:7]) < 0), "negative side spacing grows away from 0"


def pin_table_independent(table_fn=onf4.nf4_table):
    """Two independent normal-quantile routes give the same fp32 table bit for bit."""
    t = table_fn().view(np.uint32)
    ref_bisect = table_from_quantile(inv_phi_bisect).view(np.uint32)
    assert np.array_equal(t, ref_bisect), (t, ref_bisect)
    try:
        from scipy.special import ndtri
        ref_scipy = table_from_quantile(lambda p: float(ndtri(p))).view(np.uint32)
        assert np.array_equal(t, ref_scipy)
    except ImportError:  # pragma: no cover
        pass
    # forward check: each positive value is the quantile at its probability
    tt = table_fn().astype(np.float64)
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    z = inv_phi_bisect(delta)
    for j in range(8):
        p = delta - j * (delta - 0.5) / 8.0
        assert abs(phi(tt[15 - j] * z) - p) < 2e-7
    for j in range(7):
        p = delta - j * (delta - 0.5) / 7.0
        assert abs(phi(-tt[j] * z) - p) < 2e-7


# ---------------------------------------------------------------------------
# P2: the encoder against exact brute force
# ---------------------------------------------------------------------------

def _quant_codes(quantize_fn, W, dq=0):
    q = quantize_fn(np.asarray(W, np.float32).reshape(-1, 64), 64, dq)
    return q


def pin_encoder_bruteforce(quantize_fn=onf4.quantize, table_fn=onf4.nf4_table, seed=1, nblocks=24):
    rng = np.random.default_rng(seed)
    table = table_fn()
    blocks = []
    for b in range(nblocks):
        scale = float(np.exp(rng.uniform(-8, 2)))
        kind = b % 3
        if kind == 0:
            blk = rng.standard_normal(64).astype(np.float32) * np.float32(scale)
        elif kind == 1:
            blk = (rng.standard_t(3, 64) * scale).astype(np.float32)
        else:
            blk = rng.uniform(-scale, scale, 64).astype(np.float32)
        blocks.append(blk)
    W = np.stack(blocks)
    q = _quant_codes(quantize_fn, W)
    codes = q.codes.reshape(nblocks, 64)
    for b in range(nblocks):
        ref, a = brute_codes(W[b], table)
        assert q.absmax[b] == a
        assert list(codes[b]) == ref, (b, list(codes[b]), ref)


def representable_midpoints(table):
    out = []
    for j in range(15):
        m = (fr(table[j]) + fr(table[j + 1])) / 2
        if fr(np.float32(float(m))) == m:
            out.append(j)
    return out


def pin_exact_ties(quantize_fn=onf4.quantize, table_fn=onf4.nf4_table):
    """x landing exactly on a midpoint between two codes takes the lower code."""
    table = table_fn()
    mids = representable_midpoints(table)
    assert len(mids) >= 2, "the table should have fp32-exact midpoints"
    for k in (0, -3, 5):
        for j in mids:
            m = np.float32(float((fr(table[j]) + fr(table[j + 1])) / 2))
            blk = np.zeros(64, np.float32)
            blk[0] = np.float32(2.0 ** k)
            blk[1] = np.float32(m * np.float32(2.0 ** k))
            blk[2] = -blk[1]
            q = _quant_codes(quantize_fn, blk)
            assert q.codes[1] == j, (k, j, q.codes[1])
            ref, _ = brute_codes(blk, table)
            assert list(q.codes) == ref


def pin_midpoint_sweeps(quantize_fn=onf4.quantize, table_fn=onf4.nf4_table, seed=2, n_scales=3, ulps=64):
    """Weights whose quotient falls within +-ulps fp32 steps of every midpoint."""
    table = table_fn()
    rng = np.random.default_rng(seed)
    for _ in range(n_scales):
        a = np.float32(np.exp(rng.uniform(-6, 1)))
        ws = []
        for j in range(15):
            m = np.float32(float((fr(table[j]) + fr(table[j + 1])) / 2))
            x = m
            for _ in range(ulps):
                x = np.nextafter(x, np.float32(-np.inf))
            for _ in range(2 * ulps + 1):
                ws.append(np.float32(x * a))
                x = np.nextafter(x, np.float32(np.inf))
        ws = np.array(ws, np.float32)
        nper = 63
        nb = (ws.size + nper - 1) // nper
        W = np.zeros((nb, 64), np.float32)
        W[:, 0] = a
        flat = np.zeros(nb * nper, np.float32)
        flat[:ws.size] = ws
        W[:, 1:] = flat.reshape(nb, nper)
        q = _quant_codes(quantize_fn, W)
        codes = q.codes.reshape(nb, 64)
        for b in range(nb):
            ref, _ = brute_codes(W[b], table)
            assert list(codes[b]) == ref, b


# ---------------------------------------------------------------------------
# P3-P6: round trips and invariants
# ---------------------------------------------------------------------------

def pin_roundtrip(quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize, table_fn=onf4.nf4_table, seed=3):
    """W built from code values times 2^k (one +-1 element per block) is reproduced exactly."""
    rng = np.random.default_rng(seed)
    table = table_fn()
    nb = 32
    c = rng.integers(0, 16, size=(nb, 64)).astype(np.uint8)
    c[:, 0] = rng.choice([0, 15], size=nb)
    k = rng.integers(-20, 6, size=nb)
    W = (table[c] * np.float32(2.0) ** k[:, None].astype(np.float32)).astype(np.float32)
    q = quantize_fn(W.reshape(4, -1), 64, 0)
    assert np.array_equal(q.codes, c.reshape(-1))
    wh = dequantize_fn(q)
    assert np.array_equal(wh.reshape(-1).view(np.uint32), W.reshape(-1).view(np.uint32))


def pin_absmax_exact(quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize, seed=4):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((16, 256)).astype(np.float32) * np.float32(0.02)
    q = quantize_fn(W, 64, 0)
    wh = dequantize_fn(q).reshape(-1, 64)
    Wb = W.reshape(-1, 64)
    idx = np.argmax(np.abs(Wb), axis=1)
    rows = np.arange(Wb.shape[0])
    assert np.array_equal(wh[rows, idx], Wb[rows, idx])


def pin_scale_invariance(quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize,
                         error_fn=onf4.layer_error, seed=5):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((8, 64 * 300)).astype(np.float32) * np.float32(0.02)
    for dq in (0, 256):
        base = quantize_fn(W, 64, dq)
        for k in (-3, 4):
            f = np.float32(2.0 ** k)
            qs = quantize_fn(W * f, 64, dq)
            assert np.array_equal(qs.codes, base.codes)
            assert np.array_equal(qs.absmax, base.absmax * f)
            if dq:
                assert np.array_equal(qs.c8, base.c8)
                assert np.array_equal(qs.dq_scale, base.dq_scale * f)
            assert np.array_equal(dequantize_fn(qs), dequantize_fn(base) * f)
            assert error_fn(W * f, 64, dq) == error_fn(W, 64, dq)


def pin_dq_codes_unchanged(quantize_fn=onf4.quantize, seed=6):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((4, 64 * 700)).astype(np.float32) * np.float32(0.03)
    assert np.array_equal(quantize_fn(W, 64, 0).codes, quantize_fn(W, 64, 256).codes)


def pin_dq_exact(quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize):
    """Scales on the 8-bit grid of their group are reproduced exactly; half steps round to even."""
    step = np.float32(2.0 ** -10)
    k = np.arange(256, dtype=np.int64)
    k[0] = 255                       # the group max sets S = 255*step/255 = step
    W = np.zeros((256, 64), np.float32)
    W[:, 0] = (k.astype(np.float32) * step)
    q = quantize_fn(W.reshape(16, -1), 64, 256)
    assert q.dq_scale[0] == step
    assert np.array_equal(q.c8.astype(np.int64), k)
    assert np.array_equal(q.scales(), W[:, 0])
    wh = dequantize_fn(q).reshape(256, 64)
    assert np.array_equal(wh[:, 0], W[:, 0])
    # half steps: (k + 1/2) * step rounds to the even neighbour
    W2 = np.zeros((256, 64), np.float32)
    W2[0, 0] = np.float32(255) * step
    half = np.arange(1, 255, dtype=np.float64)
    W2[1:255, 0] = ((half + 0.5) * float(step)).astype(np.float32)
    q2 = quantize_fn(W2.reshape(16, -1), 64, 256)
    want = np.where(half % 2 == 0, half, half + 1)
    assert np.array_equal(q2.c8[1:255].astype(np.float64), want)


def pin_dq_bound(quantize_fn=onf4.quantize, seed=7):
    """8-bit linear scale quantizer: c8 <= 255, the group max maps to 255, |a_hat - a| <= S/2."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(4, (10, 64 * 700)) * 0.02).astype(np.float32)
    q = quantize_fn(W, 64, 256)
    nb = q.nblocks
    g = np.arange(nb) // 256
    S = q.dq_scale[g].astype(np.float64)
    ah = q.scales().astype(np.float64)
    a = q.absmax.astype(np.float64)
    assert q.c8.max() <= 255
    for gi in range(q.dq_scale.size):
        sl = slice(gi * 256, min(nb, (gi + 1) * 256))
        assert q.c8[sl][np.argmax(q.absmax[sl])] == 255
    slack = S * 255 * 2.0 ** -23 + np.abs(ah) * 2.0 ** -23
    assert np.all(np.abs(ah - a) <= 0.5 * S + slack)


def pin_pack(pack_fn=onf4.pack_codes, unpack_fn=onf4.unpack_codes, seed=8):
    assert list(pack_fn(np.array([1, 2, 3, 4], np.uint8))) == [0x21, 0x43]
    assert list(pack_fn(np.array([15, 0], np.uint8))) == [0x0F]
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 16, 1000).astype(np.uint8)
    assert np.array_equal(unpack_fn(pack_fn(c)), c)


def pin_storage(storage_fn=onf4.storage_bytes):
    """The QLoRA blog's worked budget for 65e9 weights, 64-weight blocks, 256-scale groups."""
    n = 65_000_000_000
    rows, cols = n // 64, 64
    codes, a32, _ = storage_fn(rows, cols, 64, 0)
    assert codes == 32_500_000_000                     # 32.5 GB of 4-bit codes
    assert abs(a32 / 1e9 - 4.1) < 0.05                 # about 4.1 GB of fp32 scales
    assert abs(8 * a32 / n - 0.5) < 1e-12              # half a bit per weight
    c2, a8, s32 = storage_fn(rows, cols, 64, 256)
    assert c2 == codes
    bits = 8 * (a8 + s32) / n
    assert abs(bits - 0.127) < 5e-4                    # about 0.127 bit per weight
    assert abs((codes + a8 + s32) / 1e9 - 33.5) < 0.05  # about 33.5 GB in total
    assert abs(0.5 - bits - 0.37) < 0.01               # about 0.37 bit saved
    assert abs((a32 - a8 - s32) / 1e9 - 3.0) < 0.1     # about 3 GB saved


# ---------------------------------------------------------------------------
# P8-P10: the layer
# ---------------------------------------------------------------------------

def _small_layer(seed, M=3, h=64, o=5, r=2):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    W = rng.standard_normal((o, h)) * 0.1
    L1 = rng.standard_normal((h, r)) * 0.1
    L2 = rng.standard_normal((r, o)) * 0.1
    dY = rng.standard_normal((M, o))
    return X, W, L1, L2, dY


def pin_fwd_bruteforce(fwd_fn=olora.fwd, seed=9):
    """Equation (3) summed term by term in Python loops (W stored [o][h])."""
    X, W, L1, L2, _ = _small_layer(seed)
    s = 2.0
    Y, T = fwd_fn(X, W, L1, L2, s)
    M, h = X.shape
    o, r = W.shape[0], L1.shape[1]
    for m in range(M):
        for j in range(r):
            t = sum(X[m][k] * L1[k][j] for k in range(h))
            assert abs(T[m][j] - t) < 1e-12
        for n in range(o):
            base = sum(X[m][k] * W[n][k] for k in range(h))
            ad = sum(sum(X[m][k] * L1[k][j] for k in range(h)) * L2[j][n] for j in range(r))
            assert abs(Y[m][n] - (base + s * ad)) < 1e-12


def pin_fwd_merge(fwd_fn=olora.fwd, merge_fn=olora.merge, seed=10):
    """The adapter merged into the base gives the same output (LoRA blog, merge section)."""
    X, W, L1, L2, _ = _small_layer(seed, M=4, h=128, o=7, r=3)
    s = 0.75
    Y, _ = fwd_fn(X, W, L1, L2, s)
    Wm = merge_fn(W, L1, L2, s)
    assert Wm.shape == W.shape
    Y2 = np.array([[sum(X[m][k] * Wm[n][k] for k in range(X.shape[1])) for n in range(W.shape[0])]
                   for m in range(X.shape[0])])
    assert np.max(np.abs(Y - Y2)) < 1e-12


def pin_fwd_special(fwd_fn=olora.fwd, seed=11):
    X, W, L1, L2, _ = _small_layer(seed)
    s = 2.0
    # L2 = 0 (the LoRA init: the adapter adds nothing) -> Y = base term
    Y, _ = fwd_fn(X, W, L1, np.zeros_like(L2), s)
    Yb, _ = fwd_fn(X, W, np.zeros_like(L1), L2, s)
    assert np.array_equal(Y, Yb)
    # W = 0 -> Y is the adapter term alone, linear in s
    Y1, _ = fwd_fn(X, np.zeros_like(W), L1, L2, 1.0)
    Y2, _ = fwd_fn(X, np.zeros_like(W), L1, L2, 2.0)
    assert np.max(np.abs(Y2 - 2 * Y1)) < 1e-13
    # zero X -> zero output
    Y0, T0 = fwd_fn(np.zeros_like(X), W, L1, L2, s)
    assert not Y0.any() and not T0.any()


def pin_bwd_finite_diff(fwd_fn=olora.fwd, bwd_fn=olora.bwd, seed=12):
    """Central differences of f = <dY, Y>; the layer is bilinear so they are exact up to rounding."""
    X, W, L1, L2, dY = _small_layer(seed, M=3, h=64, o=6, r=3)
    s = 1.5
    dX, dL1, dL2, _ = bwd_fn(X, dY, W, L1, L2, s)

    def f(Xv, A, B):
        Y, _ = fwd_fn(Xv, W, A, B, s)
        return float(np.sum(dY * Y))

    eps = 1e-3
    rng = np.random.default_rng(seed + 1)
    for _ in range(12):
        m, k = rng.integers(0, X.shape[0]), rng.integers(0, X.shape[1])
        Xp, Xm = X.copy(), X.copy()
        Xp[m, k] += eps
        Xm[m, k] -= eps
        g = (f(Xp, L1, L2) - f(Xm, L1, L2)) / (2 * eps)
        assert abs(g - dX[m, k]) < 1e-8 * max(1.0, abs(g))
        k2, j = rng.integers(0, L1.shape[0]), rng.integers(0, L1.shape[1])
        Ap, Am = L1.copy(), L1.copy()
        Ap[k2, j] += eps
        Am[k2, j] -= eps
        g = (f(X, Ap, L2) - f(X, Am, L2)) / (2 * eps)
        assert abs(g - dL1[k2, j]) < 1e-8 * max(1.0, abs(g))
        j2, n = rng.integers(0, L2.shape[0]), rng.integers(0, L2.shape[1])
        Bp, Bm = L2.copy(), L2.copy()
        Bp[j2, n] += eps
        Bm[j2, n] -= eps
        g = (f(X, L1, Bp) - f(X, L1, Bm)) / (2 * eps)
        assert abs(g - dL2[j2, n]) < 1e-8 * max(1.0, abs(g))


def pin_bwd_special(bwd_fn=olora.bwd, fwd_fn=olora.fwd, seed=13):
    X, W, L1, L2, dY = _small_layer(seed)
    s = 2.0
    dX, dL1, dL2, G = bwd_fn(X, dY, W, L1, np.zeros_like(L2), s)
    assert not G.any() and not dL1.any()
    # dX with no adapter equals the gradient of <dY, X W^T> by brute force
    for m in range(X.shape[0]):
        for k in range(X.shape[1]):
            ref = sum(dY[m][n] * W[n][k] for n in range(W.shape[0]))
            assert abs(dX[m][k] - ref) < 1e-12
    _, _, dL2b, _ = bwd_fn(X, dY, W, np.zeros_like(L1), L2, s)
    assert not dL2b.any()


def pin_adapter_grads(grads_fn=olora.adapter_grads, fwd_fn=olora.fwd, seed=19):
    """The adapter gradients on their own, as the chunked full-size checks use them.

    Central differences of f = <dY, Y> in each adapter factor (exact up to
    rounding: Y is linear in L1 and in L2 separately), G against its
    definition by brute force, and token additivity: the gradients of a batch
    are the sums over any split of its tokens, and G's rows are those of the
    parts.
    """
    X, W, L1, L2, dY = _small_layer(seed, M=5, h=64, o=7, r=3)
    s = 0.75
    G, dL1, dL2 = grads_fn(X, dY, L1, L2, s)
    assert G.shape == (5, 3) and dL1.shape == (64, 3) and dL2.shape == (3, 7)
    for m in range(5):
        for j in range(3):
            ref = s * sum(float(dY[m][n]) * float(L2[j][n]) for n in range(7))
            assert abs(G[m][j] - ref) < 1e-12 * max(1.0, abs(ref))

    def f(A, B):
        Y, _ = fwd_fn(X, W, A, B, s)
        return float(np.sum(dY * Y))

    eps = 1e-3
    rng = np.random.default_rng(seed + 1)
    for _ in range(10):
        k, j = rng.integers(0, 64), rng.integers(0, 3)
        Ap, Am = L1.copy(), L1.copy()
        Ap[k, j] += eps
        Am[k, j] -= eps
        g = (f(Ap, L2) - f(Am, L2)) / (2 * eps)
        assert abs(g - dL1[k, j]) < 1e-8 * max(1.0, abs(g))
        j2, n = rng.integers(0, 3), rng.integers(0, 7)
        Bp, Bm = L2.copy(), L2.copy()
        Bp[j2, n] += eps
        Bm[j2, n] -= eps
        g = (f(L1, Bp) - f(L1, Bm)) / (2 * eps)
        assert abs(g - dL2[j2, n]) < 1e-8 * max(1.0, abs(g))
    for cut in (1, 3):
        Ga, a1, a2 = grads_fn(X[:cut], dY[:cut], L1, L2, s)
        Gb, b1, b2 = grads_fn(X[cut:], dY[cut:], L1, L2, s)
        assert np.allclose(np.concatenate([Ga, Gb]), G, rtol=1e-12, atol=1e-14)
        assert np.allclose(a1 + b1, dL1, rtol=1e-12, atol=1e-14)
        assert np.allclose(a2 + b2, dL2, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P11-P12: error, counts
# ---------------------------------------------------------------------------

def pin_error_bruteforce(error_fn=onf4.layer_error, table_fn=onf4.nf4_table, seed=14):
    rng = np.random.default_rng(seed)
    table = table_fn()
    W = (rng.standard_normal((2, 128)) * 0.05).astype(np.float32)
    num = Fraction(0)
    den = Fraction(0)
    for blk in W.reshape(-1, 64):
        codes, a = brute_codes(blk, table)
        for w, c in zip(blk, codes):
            wh = fr(np.float32(table[c]) * a)       # fp32 product, as stored
            num += (fr(w) - wh) ** 2
            den += fr(w) ** 2
    ref = math.sqrt(float(num)) / math.sqrt(float(den))
    got = error_fn(W, 64, 0)
    assert abs(got - ref) <= 1e-12 * ref
    assert error_fn(np.zeros((2, 64), np.float32), 64, 0) == 0.0


def pin_error_zero_on_grid(error_fn=onf4.layer_error, table_fn=onf4.nf4_table, seed=15):
    rng = np.random.default_rng(seed)
    table = table_fn()
    c = rng.integers(0, 16, size=(8, 64)).astype(np.uint8)
    c[:, 0] = 15
    W = (table[c] * np.float32(0.125)).astype(np.float32)
    assert error_fn(W, 64, 0) == 0.0


def pin_error_tails(error_fn=onf4.layer_error, seed=16):
    """Heavier tails at the same variance give a larger NF4 error."""
    rng = np.random.default_rng(seed)
    sigma = 0.02
    Wn = (rng.standard_normal((128, 512)) * sigma).astype(np.float32)
    df = 3
    Wt = (rng.standard_t(df, (128, 512)) * sigma * math.sqrt((df - 2) / df)).astype(np.float32)
    assert error_fn(Wt, 64, 0) > error_fn(Wn, 64, 0)


def pin_counts(protect_fn=onf4.protect_count):
    assert protect_fn(0.2, 144) == 29          # AQLoRA: K = 29 at rho = .2 on 144 linears
    h = o = 4096
    r = 8
    assert r * (h + o) == 65_536               # LoRA blog: both adapter matrices at 4096^2, r = 8


def pin_topk(topk_fn=onf4.topk, seed=17):
    rng = np.random.default_rng(seed)
    e = rng.integers(0, 20, 200).astype(np.float64) / 7.0   # many ties
    k = 13
    got = topk_fn(e, k)
    # brute force: rank = number of entries that beat i (larger, or equal with lower index)
    rank = [sum(1 for j in range(len(e)) if e[j] > e[i] or (e[j] == e[i] and j < i)) for i in range(len(e))]
    want = [rank.index(p) for p in range(k)]
    assert got == want


def pin_topk_nan(topk_fn=onf4.topk, seed=18):
    """A NaN error (non-finite weights) ranks above every number, +inf included; NaNs among
    themselves and equal numbers by index.  Brute force over all pairs."""
    rng = np.random.default_rng(seed)
    e = rng.integers(0, 6, 60).astype(np.float64) / 3.0
    e[[4, 17, 40]] = np.nan
    e[[9, 33]] = np.inf
    e[25] = -0.0

    def beats(j, i):
        nj, ni = math.isnan(e[j]), math.isnan(e[i])
        if nj != ni:
            return nj
        if nj or e[j] == e[i]:
            return j < i
        return e[j] > e[i]
    rank = [sum(1 for j in range(len(e)) if beats(j, i)) for i in range(len(e))]
    assert sorted(rank) == list(range(len(e)))
    for k in (1, 3, 5, len(e)):
        assert topk_fn(e, k) == [rank.index(p) for p in range(k)], k


# ---------------------------------------------------------------------------
# bf16 operand rounding
# ---------------------------------------------------------------------------

def bf16_nearest_bits(bits: int) -> int:
    """bf16 bits of the fp32 value with these bits, by exact rational comparison.

    The two bf16 candidates are the fp32 patterns with the low 16 bits cleared
    (toward zero) and the next one away from zero (2^128 standing in for
    infinity, as rounding with an unbounded exponent range and then overflowing
    gives); the nearer wins, and on an exact tie the one whose last bf16
    mantissa bit is 0.  Infinities map to themselves."""
    sign, mag = bits & 0x80000000, bits & 0x7FFFFFFF
    assert mag <= 0x7F800000, "finite or infinite values only"
    if mag == 0x7F800000:
        return (sign | mag) >> 16

    def value(m):
        if m >= 0x7F800000:
            return Fraction(2) ** 128
        e, f = m >> 23, m & 0x7FFFFF
        return Fraction(f, 1 << 23) * Fraction(2) ** -126 if e == 0 else \
            (1 + Fraction(f, 1 << 23)) * Fraction(2) ** (e - 127)
    lo = mag & 0xFFFF0000
    hi = lo + 0x10000
    v, vl, vh = value(mag), value(lo), value(hi)
    if v - vl < vh - v or (v - vl == vh - v and (lo >> 16) % 2 == 0):
        out = lo
    else:
        out = hi
    return (sign | min(out, 0x7F800000)) >> 16


# hand-built fp32 patterns: ties to even and to odd, one below and one above a tie, a carry into the
# exponent, subnormals (including a carry into the smallest normal), +-0, negatives, overflow to inf
BF16_CASES = [
    0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x3F7FFFFF, 0x3FFF8000, 0x3F800000,
    0x00008000, 0x00018000, 0x0000FFFF, 0x007FFFFF, 0x007F8000, 0x00000001, 0x00000000, 0x80000000,
    0xBF818000, 0xBF808000, 0x80018000, 0x807FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000,
    0x7F800000, 0xFF800000, 0x3E9A8000, 0x3E9B8000,
]


def pin_bf16_rounding(bf16_fn=onf4.bf16_bits, dequantize_bf16_fn=onf4.dequantize_bf16_bits,
                      quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize, seed=22):
    """The bf16 form of the dequantized weight is round-to-nearest-even of its fp32 value
    ("1. NormalFloat": weights reconstructed into bf16): the hand-built cases above, random
    finite fp32 patterns of every exponent, and the dequantized weights of quantized tensors
    (with and without double quantization), each against exact rational rounding."""
    cases = np.array(BF16_CASES, np.uint32)
    got = bf16_fn(cases.view(np.float32))
    want = np.array([bf16_nearest_bits(int(b)) for b in cases], np.uint16)
    assert np.array_equal(got, want), [(hex(c), hex(g), hex(w)) for c, g, w in zip(cases, got, want) if g != w]
    rng = np.random.default_rng(seed)
    r = rng.integers(0, 1 << 32, 4000, dtype=np.uint64).astype(np.uint32)
    r = r[(r & 0x7F800000) != 0x7F800000]           # finite only
    r[:200] = (r[:200] & 0xFFFF0000) | 0x8000        # exact ties
    got = bf16_fn(r.view(np.float32))
    want = np.array([bf16_nearest_bits(int(b)) for b in r], np.uint16)
    assert np.array_equal(got, want)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    for dq in (0, 256):
        q = quantize_fn(W, 64, dq)
        wh = dequantize_fn(q).reshape(-1).view(np.uint32)
        want = np.array([bf16_nearest_bits(int(b)) for b in wh], np.uint16)
        assert np.array_equal(dequantize_bf16_fn(q).reshape(-1), want), dq


# ---------------------------------------------------------------------------
# other 4-bit codebooks (int4, fp4) through the same encoder and decoder
# ---------------------------------------------------------------------------

def _codebook_fns(cb, quantize_fn=onf4.quantize, table_fn=onf4.codebook_table):
    return (lambda W, block=64, dq=0: quantize_fn(W, block, dq, cb)), (lambda: table_fn(cb))


def pin_codebook_tables(table_fn=onf4.codebook_table):
    """int4 = (c-8)/7 and fp4 = E2M1 / 6, each value the fp32 nearest to the exact rational."""
    assert np.array_equal(table_fn("nf4").view(np.uint32), onf4.nf4_table().view(np.uint32))
    t = table_fn("int4")
    for c in range(16):
        assert t[c] == f32_nearest(Fraction(c - 8, 7)), c
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    exact = [-m / 6 for m in reversed(mags)] + [m / 6 for m in mags]
    f = table_fn("fp4")
    for c in range(16):
        assert fr(f[c]) == fr(f32_nearest(exact[c])), c
    assert np.signbit(f[7]) and not np.signbit(f[8]) and f[7] == 0 and f[8] == 0
    for tab in (t, f):
        assert np.all(np.diff(tab.astype(np.float64)) >= 0)
    assert t[1] == -1 and t[8] == 0 and t[15] == 1 and f[0] == -1 and f[15] == 1


def pin_codebook_encoders(quantize_fn=onf4.quantize, table_fn=onf4.codebook_table):
    """Exact brute force (nearest code, lower index on ties) for int4 and fp4, including
    sweeps of +-16 fp32 steps around every midpoint and any fp32-exact midpoint."""
    for cb in ("int4", "fp4"):
        q, t = _codebook_fns(cb, quantize_fn, table_fn)
        pin_encoder_bruteforce(q, t, seed=11, nblocks=12)
        pin_midpoint_sweeps(q, t, seed=12, n_scales=2, ulps=16)
        table = t()
        for j in representable_midpoints(table):
            m = np.float32(float((fr(table[j]) + fr(table[j + 1])) / 2))
            blk = np.zeros(64, np.float32)
            blk[0] = np.float32(1.0)
            blk[1] = m
            ref, _ = brute_codes(blk, table)
            assert list(q(blk.reshape(1, 64)).codes) == ref, (cb, j)
    # fp4 never produces +0 (code 8): it ties with -0 at every x and the lower code wins
    q, _ = _codebook_fns("fp4", quantize_fn, table_fn)
    W = np.random.default_rng(13).standard_normal((32, 64)).astype(np.float32)
    W[:, 5] = 0.0
    assert not np.any(q(W).codes == 8)


def pin_codebook_roundtrip(quantize_fn=onf4.quantize, dequantize_fn=onf4.dequantize,
                           table_fn=onf4.codebook_table, seed=14):
    """Weights built from the reachable code values times 2^k come back exactly."""
    rng = np.random.default_rng(seed)
    for cb, unreachable, ends in (("int4", {0}, [1, 15]), ("fp4", {8}, [0, 15])):
        table = table_fn(cb)
        allowed = np.array([c for c in range(16) if c not in unreachable], np.uint8)
        nb = 24
        c = rng.choice(allowed, size=(nb, 64)).astype(np.uint8)
        c[:, 0] = rng.choice(ends, size=nb)
        k = rng.integers(-20, 6, size=nb)
        W = (table[c] * np.float32(2.0) ** k[:, None].astype(np.float32)).astype(np.float32)
        qq = quantize_fn(W.reshape(4, -1), 64, 0, cb)
        assert np.array_equal(qq.codes, c.reshape(-1)), cb
        wh = dequantize_fn(qq)
        assert np.array_equal(wh.reshape(-1).view(np.uint32), W.reshape(-1).view(np.uint32)), cb


# ---------------------------------------------------------------------------
# residual second stage
# ---------------------------------------------------------------------------

def pin_residual(quantize_res_fn=onf4.quantize_residual, dequantize_res_fn=onf4.dequantize_residual,
                 table_fn=onf4.nf4_table, seed=21):
    """The second stage quantizes fl32(W - w_hat1) exactly as brute force does; on an exactly
    representable W the residual is zero (codes of 0, zero scales) and w_hat == W; and since 0 is a
    code, every residual element is reconstructed at least as well as by 0, so the two-stage error
    never exceeds the one-stage error."""
    rng = np.random.default_rng(seed)
    table = table_fn()
    W = (rng.standard_t(4, size=(6, 128)) * 0.02).astype(np.float32)
    q1, q2 = quantize_res_fn(W, 64, 0)
    R = (W.astype(np.float64) - onf4.dequantize(q1).astype(np.float64))  # exact difference
    Rf = np.array([f32_nearest(fr(v)) for v in R.reshape(-1)], np.float32).reshape(R.shape)
    for b, blk in enumerate(Rf.reshape(-1, 64)):
        ref, a = brute_codes(blk, table)
        assert list(q2.codes.reshape(-1, 64)[b]) == ref and q2.absmax[b] == a, b
    r2 = np.abs(R - onf4.dequantize(q2).astype(np.float64))
    assert np.all(r2 <= np.abs(Rf.astype(np.float64)) + 1e-12), "0 is a code: never worse than 0"
    e1 = np.linalg.norm(W.astype(np.float64) - onf4.dequantize(q1))
    e2 = np.linalg.norm(W.astype(np.float64) - dequantize_res_fn(q1, q2))
    assert e2 <= e1 * (1 + 1e-6) and e2 < 0.5 * e1
    # exact grid: the residual vanishes
    c = rng.integers(0, 16, size=(8, 64)).astype(np.uint8)
    c[:, 0] = 15
    Wg = (table[c] * np.float32(0.125)).astype(np.float32)
    for dq in (0, 256):
        g1, g2 = quantize_res_fn(Wg.reshape(2, -1), 64, dq)
        assert np.all(g2.codes == 7) and np.all(g2.absmax == 0)
        assert np.array_equal(dequantize_res_fn(g1, g2).reshape(-1), Wg.reshape(-1))


ALL_PINS = [
    pin_table_structure, pin_table_independent, pin_encoder_bruteforce, pin_exact_ties,
    pin_midpoint_sweeps, pin_roundtrip, pin_absmax_exact, pin_scale_invariance,
    pin_dq_codes_unchanged, pin_dq_exact, pin_dq_bound, pin_pack, pin_storage,
    pin_fwd_bruteforce, pin_fwd_merge, pin_fwd_special, pin_bwd_finite_diff, pin_bwd_special,
    pin_error_bruteforce, pin_error_zero_on_grid, pin_error_tails, pin_counts, pin_topk,
    pin_codebook_tables, pin_codebook_encoders, pin_codebook_roundtrip, pin_residual, pin_bf16_rounding,
    pin_topk_nan, pin_adapter_grads,
]
