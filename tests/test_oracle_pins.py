"""The CPU oracle against its pins, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle
from oracle import lora as olora
from oracle import nf4 as onf4

from . import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_representable_midpoints():
    # the exact-tie pin is only meaningful if some midpoints are fp32 values
    assert pins.representable_midpoints(oracle.nf4_table()) == [2, 6, 7, 14]


def test_golden_table():
    """Stored table (written by tests/golden/make_golden.py from the oracle) still matches."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nf4_table.txt")
    bits = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits.append(int(line.split()[1], 16))
    assert np.array_equal(np.array(bits, np.uint32), oracle.nf4_table().view(np.uint32))


# ---------------------------------------------------------------------------
# planted mistakes: each broken oracle variant must fail at least one pin
# ---------------------------------------------------------------------------

def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def test_mistake_symmetric_table():
    # 8 negative / 7 positive instead of 7 / 8 (sign flipped construction)
    bad = lambda: -oracle.nf4_table()[::-1].copy()
    assert _fails(pins.pin_table_structure, bad) or _fails(pins.pin_table_independent, bad)


def test_mistake_table_offset():
    import statistics
    def bad():
        inv = statistics.NormalDist().inv_cdf
        delta = 0.97                              # wrong outermost probability
        z = inv(delta)
        v = [inv(delta - j * (delta - .5) / 8) / z for j in range(8)]
        v += [-inv(delta - j * (delta - .5) / 7) / z for j in range(7)] + [0.0]
        return np.array(sorted(v)).astype(np.float32)
    assert _fails(pins.pin_table_independent, bad)


def test_mistake_upper_tie():
    def bad_quantize(W, block=64, dq=0):
        q = onf4.quantize(W, block, dq)
        t = onf4.nf4_table().astype(np.float64)
        Wb = np.asarray(W, np.float32).reshape(-1, block)
        a = np.max(np.abs(Wb), axis=1)
        x = (Wb / np.where(a == 0, 1, a)[:, None]).astype(np.float32).astype(np.float64)
        d = np.abs(x[..., None] - t)
        # last minimum instead of the first
        q.codes = (15 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8).reshape(-1)
        return q
    assert _fails(pins.pin_exact_ties, bad_quantize)


def test_mistake_reciprocal_multiply():
    # w * (1/a) instead of the correctly rounded w / a
    def bad_quantize(W, block=64, dq=0):
        q = onf4.quantize(W, block, dq)
        Wb = np.asarray(W, np.float32).reshape(-1, block)
        a = np.max(np.abs(Wb), axis=1).astype(np.float32)
        inv = (np.float32(1) / np.where(a == 0, np.float32(1), a)).astype(np.float32)
        x = (Wb * inv[:, None]).astype(np.float32)
        q.codes = onf4._encode(x, onf4.nf4_table()).reshape(-1)
        return q
    assert _fails(pins.pin_midpoint_sweeps, bad_quantize, n_scales=6)


def test_mistake_nibble_order():
    bad = lambda c: (np.asarray(c, np.uint8)[1::2] | (np.asarray(c, np.uint8)[0::2] << 4)).astype(np.uint8)
    assert _fails(pins.pin_pack, bad)


def test_mistake_dq_256_levels():
    def bad_quantize(W, block=64, dq=0):
        q = onf4.quantize(W, block, dq)
        if dq:
            nb = q.absmax.size
            for g in range(q.dq_scale.size):
                q.dq_scale[g] = np.float32(q.absmax[g * dq:(g + 1) * dq].max()) / np.float32(256)
            Sb = q.dq_scale[np.arange(nb) // dq]
            q.c8 = np.minimum(255, np.rint(q.absmax / Sb)).astype(np.uint8)
        return q
    assert _fails(pins.pin_dq_exact, bad_quantize)


def test_mistake_dq_truncation():
    def bad_quantize(W, block=64, dq=0):
        q = onf4.quantize(W, block, dq)
        if dq:
            Sb = q.dq_scale[np.arange(q.absmax.size) // dq]
            q.c8 = np.floor(q.absmax / Sb).astype(np.uint8)
        return q
    assert _fails(pins.pin_dq_bound, bad_quantize) or _fails(pins.pin_dq_exact, bad_quantize)


def test_mistake_transposed_weight():
    # reads the [o][h] storage as if it were laid out [h][o]
    def bad_fwd(X, W, L1, L2, s):
        X, W, A, B = (np.asarray(v, np.float64) for v in (X, W, L1, L2))
        T = X @ A
        return X @ W.reshape(W.shape[1], W.shape[0]) + s * (T @ B), T
    assert _fails(pins.pin_fwd_bruteforce, bad_fwd)


def test_mistake_dropped_scale():
    def bad_fwd(X, W, L1, L2, s):
        return olora.fwd(X, W, L1, L2, 1.0)
    assert _fails(pins.pin_fwd_bruteforce, bad_fwd)
    assert _fails(pins.pin_fwd_special, bad_fwd)


def test_mistake_bwd_missing_scale():
    def bad_bwd(X, dY, W, L1, L2, s):
        dX, dL1, dL2, G = olora.bwd(X, dY, W, L1, L2, s)
        return dX, dL1, dL2 / s, G                  # dL2 without s
    assert _fails(pins.pin_bwd_finite_diff, bwd_fn=bad_bwd)


def test_mistake_bwd_adapter_term():
    def bad_bwd(X, dY, W, L1, L2, s):
        X64, dY64, W64 = (np.asarray(v, np.float64) for v in (X, dY, W))
        dX, dL1, dL2, G = olora.bwd(X, dY, W, L1, L2, s)
        return dY64 @ W64, dL1, dL2, G              # dX without the G L1^T term
    assert _fails(pins.pin_bwd_finite_diff, bwd_fn=bad_bwd)


def test_mistake_adapter_grads_unscaled_dl2():
    # dL2 without the adapter scale s
    def bad(X, dY, L1, L2, s):
        G, dL1, dL2 = olora.adapter_grads(X, dY, L1, L2, s)
        return G, dL1, dL2 / s
    assert _fails(pins.pin_adapter_grads, grads_fn=bad)


def test_mistake_adapter_grads_dl1_from_dy():
    # dL1 taken against dY L2^T without s (G before scaling)
    def bad(X, dY, L1, L2, s):
        G, dL1, dL2 = olora.adapter_grads(X, dY, L1, L2, s)
        return G, dL1 / s, dL2
    assert _fails(pins.pin_adapter_grads, grads_fn=bad)


def test_mistake_adapter_grads_unscaled_g():
    def bad(X, dY, L1, L2, s):
        G, dL1, dL2 = olora.adapter_grads(X, dY, L1, L2, s)
        return G / s, dL1, dL2
    assert _fails(pins.pin_adapter_grads, grads_fn=bad)


def test_mistake_adapter_grads_mean_over_tokens():
    # averaging instead of summing over tokens breaks additivity
    def bad(X, dY, L1, L2, s):
        G, dL1, dL2 = olora.adapter_grads(X, dY, L1, L2, s)
        m = len(X)
        return G, dL1 / m, dL2 / m
    assert _fails(pins.pin_adapter_grads, grads_fn=bad)


def test_mistake_error_without_sqrt():
    def bad_error(W, block=64, dq=0):
        return onf4.layer_error(W, block, dq) ** 2
    assert _fails(pins.pin_error_bruteforce, bad_error)


def test_mistake_topk_ties():
    def bad_topk(e, k):
        return list(np.argsort(-np.asarray(e), kind="stable")[::-1][:k][::-1])
    assert _fails(pins.pin_topk, bad_topk)


def test_mistake_codebooks():
    # int4 with the grid shifted by one code, fp4 with +0 before -0, fp4 divided by 4 instead of 6
    def shifted(cb):
        t = oracle.codebook_table(cb)
        return (np.arange(16, dtype=np.float64) - 7.0).astype(np.float32) / np.float32(7) if cb == "int4" else t
    assert _fails(pins.pin_codebook_tables, shifted)

    def zero_order(cb):
        t = oracle.codebook_table(cb).copy()
        if cb == "fp4":
            t[7], t[8] = np.float32(0.0), np.float32(-0.0)
        return t
    assert _fails(pins.pin_codebook_tables, zero_order)

    def wrong_norm(cb):
        t = oracle.codebook_table(cb)
        return (t * np.float32(1.5)).astype(np.float32) if cb == "fp4" else t
    assert _fails(pins.pin_codebook_tables, wrong_norm)
    # an encoder that breaks ties toward the upper code fails the brute force
    def upper_tie_quantize(W, block=64, dq=0, cb="nf4"):
        q = oracle.nf4.quantize(W, block, dq, cb)
        t = oracle.codebook_table(cb).astype(np.float64)
        x = (np.asarray(W, np.float32).reshape(-1, block) /
             np.where(q.absmax == 0, 1, q.absmax)[:, None].astype(np.float32)).astype(np.float32).reshape(-1)
        d = np.abs(x.astype(np.float64)[:, None] - t[None, :])
        q.codes = (15 - np.argmin(d[:, ::-1], axis=1)).astype(np.uint8)
        return q
    assert _fails(pins.pin_codebook_encoders, upper_tie_quantize)


def test_mistake_residual():
    # the second stage dropped from the dequantized weight, or quantizing W twice instead of the residual
    ignore_q2 = lambda q1, q2: oracle.dequantize(q1)
    assert _fails(pins.pin_residual, dequantize_res_fn=ignore_q2)
    def twice(W, block=64, dq=0, codebook="nf4"):
        q1 = oracle.quantize(W, block, dq, codebook)
        return q1, oracle.quantize(W, block, dq, codebook)
    assert _fails(pins.pin_residual, quantize_res_fn=twice)


def test_mistake_bf16_truncation():
    # bf16 by dropping the low 16 bits, or rounding ties away from zero
    trunc = lambda w: (np.asarray(w, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert _fails(pins.pin_bf16_rounding, bf16_fn=trunc)
    away = lambda w: ((np.asarray(w, np.float32).view(np.uint32).astype(np.uint64) + 0x8000) >> 16).astype(np.uint16)
    assert _fails(pins.pin_bf16_rounding, bf16_fn=away)
    # the bf16 form of the dequantized weight taken by truncation
    deq_trunc = lambda q: trunc(oracle.dequantize(q))
    assert _fails(pins.pin_bf16_rounding, dequantize_bf16_fn=deq_trunc)


def test_mistake_topk_nan_last():
    # NaN treated as the smallest error (numpy's argsort places it last)
    def nan_last(e, k):
        e = np.asarray(e, np.float64)
        return [int(i) for i in np.lexsort((np.arange(e.size), -np.nan_to_num(e, nan=-np.inf)))[:k]]
    assert _fails(pins.pin_topk_nan, nan_last)
