"""Property sweep of the HIP path against the oracle over generated layers (hypothesis).

Shapes: h and o multiples of 64 up to 1536; M from 1 to 300 or at the token
counts where the adapter kernels switch between split and whole-K / all-token
forms (512, 1024 and 2048 rows, and their neighbours); r from 1 to 256 across
the 16-column padding steps; double quant on or off; normal, Student-t,
outlier and spike weights, some with all-zero blocks; the backward with the
saved T or recomputing it.  Each example checks the codes and scales bit for
bit, the layer error within 1e-6 relative, and Y, T, dX, dL1 and dL2 to the
bar of the parity tests.  Examples are derandomized: every run draws the same
cases, and each prints its parameters before it touches the GPU.  The example
count is 24; NF4LORA_PROPERTY_EXAMPLES raises it for a wider sweep.

A second sweep (16 draws by default) covers the rows built on the same kernels:
protected bf16 layers, the int4 and fp4 codebooks, the residual second stage
and the merge from an fp32 or NF4 base, over the same kinds of shapes.
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth

pytestmark = pytest.mark.gpu

try:
    import quantized_lora_fine_amd as nf4
except ImportError as exc:
    if torch.cuda.is_available():
        raise
    pytest.skip(f"libnf4lora.so not loaded: {exc}", allow_module_level=True)

from tests.test_gpu_parity import (check_bf16_layer, check_close, check_quant, dev, heavy_weight, oracle_layer,
                                   run_layer, say)

DEV_T = "cuda"

layers = st.tuples(
    st.integers(1, 24),                      # o / 64
    st.integers(1, 24),                      # h / 64
    st.one_of(st.integers(1, 300),           # M
              st.sampled_from([504, 505, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049])),
    st.sampled_from([1, 8, 16, 17, 31, 32, 33, 48, 64, 65, 128, 256]),
    st.sampled_from([0, 256]),
    st.sampled_from(["normal", "t3", "outliers", "spike"]),
    st.booleans(),                           # zero a run of blocks
    st.sampled_from([0.5, 2.0]),
    st.booleans(),                           # backward with the saved T (else recomputed)
    st.integers(0, 2**31 - 1),
)


@settings(max_examples=int(os.environ.get("NF4LORA_PROPERTY_EXAMPLES", "24")), deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(layers)
def test_layer_properties(case):
    ob, hb, M, r, dq, kind, zeros, s, use_T, seed = case
    o, h = 64 * ob, 64 * hb
    say(f"property case: M={M} o={o} h={h} r={r} dq={dq} weights={kind} zero-blocks={zeros} s={s} "
        f"T={'saved' if use_T else 'recomputed'} seed={seed}")
    rng = np.random.default_rng(seed)
    d = synth.random_case(seed=seed % 100000, rows=o, cols=h, M=M, r=r)
    if kind != "normal":
        d["W"] = heavy_weight(rng, (o, h), kind)
    if zeros:
        flat = d["W"].reshape(-1, 64)
        b0 = int(rng.integers(0, flat.shape[0]))
        flat[b0:b0 + int(rng.integers(1, 300))] = 0.0
    q = nf4.quantize(dev(d["W"]), dq)
    check_quant(q, oracle.quantize(d["W"], 64, dq))
    got = float(nf4.layer_error(dev(d["W"]), dq).cpu()[0])
    want = oracle.layer_error(d["W"], 64, dq)
    assert abs(got - want) <= 1e-6 * max(want, 1e-300), (got, want)
    Y, T, dX, dL1, dL2 = run_layer(d, s, dq, use_T=use_T)
    Yr, Tr, dXr, dL1r, dL2r = oracle_layer(d, s, dq)
    check_close("T", T, Tr)
    check_close("Y", Y, Yr)
    check_close("dX", dX, dXr)
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


next_rows = st.tuples(
    st.sampled_from(["bf16", "int4", "fp4", "residual", "merge-fp32", "merge-nf4"]),
    st.integers(1, 24),                      # o / 64
    st.integers(1, 24),                      # h / 64
    st.one_of(st.integers(1, 300), st.sampled_from([511, 512, 513, 1024, 2048])),
    st.sampled_from([1, 8, 16, 17, 33, 64, 65, 128, 256]),
    st.sampled_from([0, 256]),
    st.sampled_from(["normal", "t3", "outliers", "spike"]),
    st.sampled_from([0.5, 2.0]),
    st.booleans(),                           # backward with the saved T (else recomputed)
    st.integers(0, 2**31 - 1),
)


def check_merge(src, ref_base, d, s, r):
    """The merge against the oracle within the bounds its roundings allow (as test_merge states them)."""
    ref = oracle.merge(ref_base, d["L1"], d["L2"], s)
    L1, L2 = dev(d["L1"]), dev(d["L2"])
    got = nf4.merge(src, L1, L2, s).cpu().numpy().astype(np.float64)
    u = 2.0 ** -24
    terms = s * (np.abs(oracle.lora._f64(d["L1"])) @ np.abs(oracle.lora._f64(d["L2"]))).T
    tol32 = (r + 2) * u * terms + 2 * u * np.abs(ref)
    assert np.all(np.abs(got - ref) <= tol32), float(np.max(np.abs(got - ref) - tol32))
    gotb = nf4.merge(src, L1, L2, s, bf16=True).cpu().float().numpy().astype(np.float64)
    tolb = 2.0 ** -8 * (np.abs(ref) + tol32) + tol32
    assert np.all(np.abs(gotb - ref) <= tolb), float(np.max(np.abs(gotb - ref) - tolb))


@settings(max_examples=int(os.environ.get("NF4LORA_PROPERTY_EXAMPLES", "16")), deadline=None, derandomize=True,
          database=None, suppress_health_check=[HealthCheck.too_slow])
@given(next_rows)
def test_next_rows_properties(case):
    """The rows built on the same kernels, over generated shapes: protected bf16 layers, the int4 and fp4
    codebooks (codes, scales and dequantized weights bit for bit, the error within 1e-6, the layer), the
    residual second stage (both stages bit for bit, the layer, the merge) and the merge from an fp32 or an
    NF4 base."""
    kind, ob, hb, M, r, dq, dist, s, use_T, seed = case
    o, h = 64 * ob, 64 * hb
    say(f"next-row case: {kind} M={M} o={o} h={h} r={r} dq={dq} weights={dist} s={s} "
        f"T={'saved' if use_T else 'recomputed'} seed={seed}")
    d = synth.random_case(seed=seed % 100000, rows=o, cols=h, M=M, r=r)
    if dist != "normal":
        d["W"] = heavy_weight(np.random.default_rng(seed), (o, h), dist)
    if kind == "bf16":
        check_bf16_layer(d, s, use_T=use_T)
        return
    if kind == "merge-fp32":
        check_merge(dev(d["W"]), d["W"], d, s, r)
        return
    if kind == "merge-nf4":
        check_merge(nf4.quantize(dev(d["W"]), dq), oracle.dequantize(oracle.quantize(d["W"], 64, dq)), d, s, r)
        return
    if kind == "residual":
        q = nf4.quantize(dev(d["W"]), dq, residual=True)
        r1, r2 = oracle.quantize_residual(d["W"], 64, dq)
        check_quant(q, r1)
        check_quant(q.residual, r2)
        wh = oracle.dequantize_residual(r1, r2)
    else:
        q = nf4.quantize(dev(d["W"]), dq, codebook=kind)
        ref = oracle.quantize(d["W"], 64, dq, kind)
        check_quant(q, ref)
        wh = oracle.dequantize(ref)
        got = float(nf4.layer_error(dev(d["W"]), dq, codebook=kind).cpu()[0])
        want = oracle.layer_error(d["W"], 64, dq, kind)
        assert abs(got - want) <= 1e-6 * max(want, 1e-300), (got, want)
    assert np.array_equal(nf4.dequantize(q).cpu().numpy().view(np.uint32), wh.view(np.uint32)), "dequantized weight"
    X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = nf4.fwd(q, X, L1, L2, s)
    dX, dL1, dL2 = nf4.bwd(q, X, dY, L1, L2, s, T=T if use_T else None)
    Yr, Tr = oracle.fwd(d["X"], wh, d["L1"], d["L2"], s)
    dXr, dL1r, dL2r, _ = oracle.bwd(d["X"], d["dY"], wh, d["L1"], d["L2"], s)
    for name, g, w in (("T", T, Tr), ("Y", Y, Yr), ("dX", dX, dXr), ("dL1", dL1, dL1r), ("dL2", dL2, dL2r)):
        check_close(name, g, w)
    if kind == "residual":
        check_merge(q, wh, d, s, r)


passes = st.tuples(
    st.lists(st.tuples(st.integers(1, 600), st.integers(1, 16)), min_size=1, max_size=8),  # (rows, cols / 64)
    st.sampled_from([0, 256]),                # double quantization of the stored codes
    st.booleans(),                            # the one-pass error with 8-bit scales (else fp32 scales)
    st.sampled_from(["nf4", "int4", "fp4"]),
    st.sampled_from(["normal", "t3", "outliers", "spike"]),
    st.integers(0, 2**31 - 1),
)


@settings(max_examples=int(os.environ.get("NF4LORA_PROPERTY_EXAMPLES", "12")), deadline=None, derandomize=True,
          database=None, suppress_health_check=[HealthCheck.too_slow])
@given(passes)
def test_profiling_pass_properties(case):
    """The passes over W on generated lists of weights (rows need not be multiples of 64, so the last
    double-quantization group is ragged): the batched error equals the per-linear error bit for bit and
    the oracle within 1e-6; the one-pass quantize + error gives the quantize's codes and scales bit for
    bit and the per-linear error bit for bit."""
    shapes, dq, err_dq, cb, dist, seed = case
    say(f"profiling-pass case: {len(shapes)} weights {[(r, 64 * c) for r, c in shapes]} dq={dq} "
        f"err_dq={err_dq} codebook={cb} weights={dist} seed={seed}")
    rng = np.random.default_rng(seed)
    Wh = [heavy_weight(rng, (r, 64 * c), dist) if dist != "normal"
          else (rng.standard_normal((r, 64 * c)) * 0.02).astype(np.float32) for r, c in shapes]
    Ws = [dev(w) for w in Wh]
    edq = dq if err_dq else 0
    batch = nf4.layer_error_batch(Ws, edq, codebook=cb)
    for i, (w, W) in enumerate(zip(Wh, Ws)):
        one = nf4.layer_error(W, edq, codebook=cb)
        assert torch.equal(batch[i:i + 1], one), (i, float(batch[i]), float(one[0]))
        want = oracle.layer_error(w, 64, edq, cb)
        assert abs(float(one[0]) - want) <= 1e-6 * max(want, 1e-300), (i, float(one[0]), want)
    q, err = nf4.quantize_error(Ws[0], dq, edq, out=nf4.NF4Weight(*Wh[0].shape, dq, DEV_T, cb))
    check_quant(q, oracle.quantize(Wh[0], 64, dq, cb))
    assert torch.equal(err, nf4.layer_error(Ws[0], edq, codebook=cb)), (float(err[0]),)


@settings(max_examples=int(os.environ.get("NF4LORA_PROPERTY_EXAMPLES", "24")), deadline=None, derandomize=True,
          database=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.integers(1, 3000), st.integers(0, 3000), st.sampled_from([2, 5, 1000, 0]), st.booleans(),
       st.integers(0, 2**31 - 1))
def test_topk_properties(n, k, distinct, nans, seed):
    """top-K against the oracle's order on generated error vectors: few distinct values (many ties),
    many, or all distinct; with some NaN errors or none."""
    k = min(k, n)
    rng = np.random.default_rng(seed)
    e = rng.integers(0, distinct, n).astype(np.float64) if distinct else rng.random(n)
    if nans:
        e[rng.choice(n, size=max(1, n // 50), replace=False)] = np.nan
    say(f"top-K case: n={n} k={k} distinct={distinct or 'all'} nans={nans} seed={seed}")
    got = nf4.topk(torch.from_numpy(e).to(DEV_T), k).cpu().numpy().tolist()
    assert got == oracle.topk(e, k)


@settings(max_examples=int(os.environ.get("NF4LORA_PROPERTY_EXAMPLES", "8")), deadline=None, derandomize=True,
          database=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.tuples(st.sampled_from(["nf4", "nf4dq", "bf16"]), st.integers(1, 6), st.integers(1, 6),
                          st.sampled_from([0, 1, 8, 16, 17])), min_size=1, max_size=5),
       st.integers(1, 600), st.data())
def test_stack_properties(spec, M, data):
    """The stack runner on generated stacks equals the per-linear calls bit for bit above the cut and
    leaves every gradient buffer below it untouched."""
    cut = data.draw(st.integers(0, len(spec)))
    say(f"stack case: M={M} cut={cut} linears={[(f, 64 * a, 64 * b, r) for f, a, b, r in spec]}")
    sentinel = 7.0
    lins, hosts = [], []
    for i, (fmt, ob, hb, r) in enumerate(spec):
        o, h = 64 * ob, 64 * hb
        d = synth.random_case(seed=31 * i + M, rows=o, cols=h, M=M, r=max(r, 1))
        L = {"X": dev(d["X"]), "dY": dev(d["dY"]), "r": r, "s": 2.0,
             "Y": torch.empty(M, o, dtype=torch.bfloat16, device=DEV_T),
             "dX": torch.full((M, h), sentinel, dtype=torch.bfloat16, device=DEV_T)}
        if fmt == "bf16":
            L["w"] = dev(synth.bf16(d["W"]))
        else:
            L["q"] = nf4.quantize(dev(d["W"]), 256 if fmt == "nf4dq" else 0)
        if r:
            L["L1"], L["L2"] = dev(d["L1"]), dev(d["L2"])
            L["T"] = torch.empty(M, r, dtype=torch.bfloat16, device=DEV_T)
            L["dL1"] = torch.full((h, r), sentinel, dtype=torch.float32, device=DEV_T)
            L["dL2"] = torch.full((r, o), sentinel, dtype=torch.float32, device=DEV_T)
        lins.append(L)
        hosts.append(d)
    stack = nf4.Stack(lins, M)
    stack.fwd()
    stack.bwd(cut=cut)
    torch.cuda.synchronize()
    for i, L in enumerate(lins):
        r = L["r"]
        if r:
            if "q" in L:
                Y, T = nf4.fwd(L["q"], L["X"], L["L1"], L["L2"], 2.0)
                dX, dL1, dL2 = nf4.bwd(L["q"], L["X"], L["dY"], L["L1"], L["L2"], 2.0, T=T)
            else:
                Y, T = nf4.bf16_fwd(L["w"], L["X"], L["L1"], L["L2"], 2.0)
                dX, dL1, dL2 = nf4.bf16_bwd(L["w"], L["X"], L["dY"], L["L1"], L["L2"], 2.0, T=T)
            assert torch.equal(L["Y"], Y) and torch.equal(L["T"], T), i
            if i >= cut:
                assert torch.equal(L["dL1"], dL1) and torch.equal(L["dL2"], dL2) and torch.equal(L["dX"], dX), i
            else:
                assert bool((L["dL1"] == sentinel).all()) and bool((L["dL2"] == sentinel).all()), i
        elif "q" in L:
            # the plain product is the fused GEMM without a tail, as nf4_matmul runs it
            assert torch.equal(L["Y"], nf4.matmul(L["q"], L["X"])), i
            if i >= cut:
                assert torch.equal(L["dX"], nf4.matmul(L["q"], L["dY"], transpose=True)), i
        else:
            d = hosts[i]
            Wb = synth.bf16(d["W"])
            z1, z2 = np.zeros((Wb.shape[1], 1)), np.zeros((1, Wb.shape[0]))
            check_close("Y", L["Y"], oracle.fwd(d["X"], Wb, z1, z2, 2.0)[0])
            if i >= cut:
                check_close("dX", L["dX"], oracle.bwd(d["X"], d["dY"], Wb, z1, z2, 2.0)[0])
        if i < cut:
            assert bool((L["dX"] == sentinel).all()), i
