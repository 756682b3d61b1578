"""HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Bar: bit-exact for codes, scales and dequantized weights; for Y, dX, dL1 and
dL2 max |err| <= 2e-2 * max |ref| (bf16 operands, fp32 accumulation), plus a
tighter relative-RMS check; layer error within 1e-6 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

try:
    import quantized_lora_fine_amd as nf4
except ImportError as exc:
    # on a GPU machine a missing or broken libnf4lora.so is a failure, not a skip
    if torch.cuda.is_available():
        raise
    pytest.skip(f"libnf4lora.so not loaded: {exc}", allow_module_level=True)

DEV = "cuda"
TOL_MAX = 2e-2
TOL_RMS = 5e-3


def say(*a):
    print(*a, flush=True)


def dev(a):
    if isinstance(a, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return a.to(DEV).contiguous()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(name, got, want, tol_max=TOL_MAX, tol_rms=TOL_RMS):
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    ref = np.max(np.abs(w))
    err = np.max(np.abs(g - w))
    rms = np.sqrt(np.mean((g - w) ** 2)) / max(np.sqrt(np.mean(w ** 2)), 1e-300)
    say(f"  {name}: max|err|/max|ref| = {err / max(ref, 1e-300):.2e}  rel-rms = {rms:.2e}")
    assert err <= tol_max * ref, f"{name}: max|err| {err:.3e} > {tol_max} * {ref:.3e}"
    if ref > 0:
        assert rms <= tol_rms, f"{name}: relative rms {rms:.3e}"


def check_quant(q, ref):
    assert np.array_equal(q.packed_codes.cpu().numpy(), ref.packed), "codes"
    if ref.dq_group:
        assert np.array_equal(q.c8.cpu().numpy(), ref.c8), "c8"
        assert np.array_equal(q.dq_step.cpu().numpy().view(np.uint32), ref.dq_scale.view(np.uint32)), "dq step"
    else:
        assert np.array_equal(q.absmax_f32.cpu().numpy().view(np.uint32), ref.absmax.view(np.uint32)), "absmax"


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dq", [0, 256])
def test_quantize_c1(dq):
    W = synth.layer_inputs(synth.C1)["W"]
    q = nf4.quantize(dev(W), dq)
    check_quant(q, oracle.quantize(W, 64, dq))


def test_quantize_dequantize_c2():
    W = synth.layer_weight(synth.C2)
    q = nf4.quantize(dev(W), 256)
    ref = oracle.quantize(W, 64, 256)
    check_quant(q, ref)
    wh = nf4.dequantize(q).cpu().numpy()
    assert np.array_equal(wh.view(np.uint32), oracle.dequantize(ref).view(np.uint32))
    whb = nf4.dequantize(q, bf16=True).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(whb, oracle.dequantize_bf16_bits(ref))


def edge_weights(codebook="nf4"):
    """Blocks that stress the encoder: exact ties, zero/subnormal/huge blocks, spikes, ragged groups."""
    rng = np.random.default_rng(11)
    t = oracle.codebook_table(codebook)
    blocks = []
    # exact midpoints at several scales (ties take the lower code)
    for k in (0, -7, 9):
        for j in range(15):
            m = np.float32((np.float64(t[j]) + np.float64(t[j + 1])) / 2)
            b = np.zeros(64, np.float32)
            b[0] = np.float32(2.0 ** k)
            b[1] = m * np.float32(2.0 ** k)
            b[2] = -b[1]
            b[3:] = rng.uniform(-1, 1, 61).astype(np.float32) * np.float32(2.0 ** k)
            blocks.append(b)
    # sweeps of +-8 ulp around every midpoint for a random scale
    a = np.float32(0.0371)
    for j in range(15):
        m = np.float32((np.float64(t[j]) + np.float64(t[j + 1])) / 2)
        xs = [m]
        for _ in range(8):
            xs.insert(0, np.nextafter(xs[0], np.float32(-2)))
            xs.append(np.nextafter(xs[-1], np.float32(2)))
        b = np.zeros(64, np.float32)
        b[0] = a
        b[1:1 + len(xs)] = np.array(xs, np.float32) * a
        blocks.append(b)
    blocks.append(np.zeros(64, np.float32))                                 # all zero
    blocks.append(np.full(64, -0.0, np.float32))                             # negative zeros
    sub = np.zeros(64, np.float32)
    sub[:8] = np.array([1e-40, -3e-41, 7e-42, 1e-45, -1e-45, 2e-40, 0, 5e-39], np.float32)
    blocks.append(sub)                                                       # subnormal block
    blocks.append((rng.standard_normal(64) * 1e30).astype(np.float32))       # huge
    blocks.append((rng.standard_normal(64) * 1e-30).astype(np.float32))      # tiny
    spike = np.zeros(64, np.float32)
    spike[17] = -3.5
    blocks.append(spike)                                                     # single spike
    blocks.append(np.full(64, 0.25, np.float32))                              # constant
    while len(blocks) % 5:
        blocks.append((rng.standard_normal(64) * 0.02).astype(np.float32))
    return np.stack(blocks).reshape(5, -1)                                   # 5 rows, ragged group count


@pytest.mark.parametrize("dq", [0, 256])
def test_quantize_edges(dq):
    W = edge_weights()
    q = nf4.quantize(dev(W), dq)
    ref = oracle.quantize(W, 64, dq)
    check_quant(q, ref)
    wh = nf4.dequantize(q).cpu().numpy()
    assert np.array_equal(wh.view(np.uint32), oracle.dequantize(ref).view(np.uint32))


@pytest.mark.parametrize("rows,cols,dq", [(1, 64, 0), (3, 64 * 100, 256), (7, 64 * 37, 256), (300, 64 * 9, 0)])
def test_quantize_shapes(rows, cols, dq):
    rng = np.random.default_rng(rows * 1000 + cols)
    W = (rng.standard_t(4, (rows, cols)) * 0.03).astype(np.float32)
    q = nf4.quantize(dev(W), dq)
    ref = oracle.quantize(W, 64, dq)
    check_quant(q, ref)
    whb = nf4.dequantize(q, bf16=True).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(whb, oracle.dequantize_bf16_bits(ref))


# ---------------------------------------------------------------------------
# error and top-K
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dq", [0, 256])
def test_layer_error(dq):
    for W in (synth.layer_inputs(synth.C1)["W"], edge_weights(),
              (np.random.default_rng(3).standard_t(3, (640, 1280)) * 0.02).astype(np.float32)):
        got = float(nf4.layer_error(dev(W), dq).cpu()[0])
        want = oracle.layer_error(W, 64, dq)
        say(f"  error dq={dq}: gpu {got:.12g} oracle {want:.12g}")
        assert abs(got - want) <= 1e-6 * want
    assert float(nf4.layer_error(dev(np.zeros((4, 128), np.float32)), dq).cpu()[0]) == 0.0


@pytest.mark.parametrize("codebook", ["nf4", "int4", "fp4"])
@pytest.mark.parametrize("dq,err_dq", [(0, 0), (256, 0), (256, 256)])
def test_quantize_error_one_pass(codebook, dq, err_dq):
    """nf4_quantize_error: codes and scales bit-exact against the oracle, and the error bit for bit what
    nf4_layer_error returns (so within the same bound of the oracle's)."""
    rng = np.random.default_rng(5)
    cases = [synth.layer_inputs(synth.C1)["W"], edge_weights(codebook),
             (rng.standard_t(4, (7, 64 * 37)) * 0.03).astype(np.float32),       # ragged last group
             np.zeros((4, 128), np.float32)]
    for W in cases:
        say(f"  {codebook} dq={dq} err_dq={err_dq} shape={W.shape}")
        Wd = dev(W)
        q, err = nf4.quantize_error(Wd, dq, err_dq, codebook=codebook)
        check_quant(q, oracle.quantize(W, 64, dq, codebook))
        sep = nf4.layer_error(Wd, err_dq, codebook=codebook)
        got, want_sep = float(err.cpu()[0]), float(sep.cpu()[0])
        assert np.float64(got).view(np.uint64) == np.float64(want_sep).view(np.uint64), (got, want_sep)
        want = oracle.layer_error(W, 64, err_dq, codebook)
        assert abs(got - want) <= 1e-6 * want, (got, want)
    # into an existing weight, twice in a row (the second call overwrites the first's outputs)
    W1 = synth.layer_inputs(synth.C1)["W"]
    W2 = (rng.standard_normal(W1.shape) * 0.05).astype(np.float32)
    q = nf4.NF4Weight(W1.shape[0], W1.shape[1], dq, DEV, codebook)
    for W in (W1, W2):
        _, err = nf4.quantize_error(dev(W), out=q, err_dq_group=err_dq)
        check_quant(q, oracle.quantize(W, 64, dq, codebook))
        assert abs(float(err.cpu()[0]) - oracle.layer_error(W, 64, err_dq, codebook)) <= \
            1e-6 * oracle.layer_error(W, 64, err_dq, codebook)


@pytest.mark.parametrize("codebook", ["nf4", "int4"])
@pytest.mark.parametrize("dq", [0, 256])
def test_layer_error_batch(codebook, dq):
    """nf4_layer_error_batch over 70 linears (two launch pairs: 64 + 6): every error bit for bit what
    nf4_layer_error gives that linear; a few also against the oracle."""
    rng = np.random.default_rng(21)
    shapes = [(4, 128), (7, 64 * 37), (0, 64), (640, 1280), (1088, 4096), (3, 64)]
    shapes += [(int(rng.integers(1, 40)), 64 * int(rng.integers(1, 70))) for _ in range(64)]
    Ws = []
    for i, (r, c) in enumerate(shapes):
        W = (rng.standard_t(3 + i % 5, (r, c)) * 0.02).astype(np.float32)
        if i == 5:
            W[:] = 0.0                                    # an all-zero linear: error 0
        Ws.append(W)
    Wd = [dev(W) for W in Ws]
    got = nf4.layer_error_batch(Wd, dq, codebook=codebook).cpu().numpy()
    assert got.shape == (len(shapes),)
    for i, W in enumerate(Wd):
        one = nf4.layer_error(W, dq, codebook=codebook).cpu().numpy()[0]
        assert got.view(np.uint64)[i] == np.float64(one).view(np.uint64), (i, shapes[i], got[i], one)
    assert got[2] == 0.0 and got[5] == 0.0
    for i in (0, 1, 3, 4):
        want = oracle.layer_error(Ws[i], 64, dq, codebook)
        say(f"  batch {codebook} dq={dq} {shapes[i]}: gpu {got[i]:.12g} oracle {want:.12g}")
        assert abs(got[i] - want) <= 1e-6 * want
    # an empty batch does nothing
    assert nf4.layer_error_batch([], dq).numel() == 0


def test_topk():
    rng = np.random.default_rng(5)
    for n, k in ((280, 8), (144, 29), (1000, 1000), (5, 1), (3000, 17), (1, 1), (1024, 5), (1025, 3)):
        e = rng.integers(0, 40, n).astype(np.float64) / 13.0
        got = nf4.topk(dev(e), k).cpu().numpy().tolist()
        assert got == oracle.topk(e, k), (n, k)


def test_topk_nan():
    """Errors of non-finite weights are NaN: they rank first, by index, as the oracle orders them."""
    rng = np.random.default_rng(6)
    for n, k in ((280, 8), (50, 50), (2000, 30)):
        e = rng.integers(0, 40, n).astype(np.float64) / 13.0
        e[rng.choice(n, size=max(2, n // 40), replace=False)] = np.nan
        e[rng.integers(0, n)] = np.inf
        got = nf4.topk(dev(e), k).cpu().numpy().tolist()
        assert got == oracle.topk(e, k), (n, k)
        assert len(set(got)) == k


def test_check_finite():
    """The checked mode: NF4_ERR_NONFINITE for an infinity or a NaN anywhere (first, middle, in the
    last count % 4 values), NF4_OK otherwise; finite extremes and subnormals pass."""
    rng = np.random.default_rng(8)
    n = 4 * 100003 + 3
    base = (rng.standard_normal(n) * 0.02).astype(np.float32)
    base[7] = np.float32(3.4e38)
    base[9] = np.float32(1e-45)
    W = dev(base)
    assert nf4.check_finite(W)
    assert nf4.check_finite(W[:5])
    for pos, val in ((0, np.inf), (n // 2, np.nan), (n - 1, -np.inf), (n - 3, np.nan)):
        b = base.copy()
        b[pos] = val
        assert not nf4.check_finite(dev(b)), pos
        if pos == n - 1:
            assert nf4.check_finite(dev(b)[: n - 1])    # the bad value is past the count


def test_zero_weight_isolates_adapter():
    """W = 0 (all codes of 0, zero scales, so w_hat = 0): Y = s T L2 and dX = G L1^T, checked at the
    adapter term's own scale (the base term would otherwise hide it), with and without double quant."""
    for dq in (0, 256):
        d = synth.random_case(seed=26 + dq, rows=320, cols=448, M=300, r=16)
        d["W"] = np.zeros_like(d["W"])
        Y, T, dX, dL1, dL2 = run_layer(d, 2.0, dq)
        Yr, Tr, dXr, dL1r, dL2r = oracle_layer(d, 2.0, dq)
        say(f"W = 0, dq={dq}: max|Y| = {np.max(np.abs(Yr)):.3e}")
        check_close("Y = s T L2", Y, Yr)
        check_close("dX = G L1^T", dX, dXr)
        check_close("dL1", dL1, dL1r)
        check_close("dL2", dL2, dL2r)


def heavy_weight(rng, shape, kind, sigma=0.02):
    """Weights with the tails of the workloads: Student-t (df 3 or 5) scaled to variance sigma^2, or
    normal with 0.1 % of the values x20, or a single large spike per row."""
    if kind in ("t3", "t5"):
        df = int(kind[1])
        return (rng.standard_t(df, size=shape) * sigma * np.sqrt((df - 2) / df)).astype(np.float32)
    W = (rng.standard_normal(shape) * sigma).astype(np.float32)
    if kind == "outliers":
        idx = rng.choice(W.size, size=max(1, W.size // 1000), replace=False)
        W.reshape(-1)[idx] *= np.float32(20)
    elif kind == "spike":
        W[np.arange(shape[0]), rng.integers(0, shape[1], shape[0])] = np.float32(50 * sigma)
    return W


@pytest.mark.parametrize("M,o,h,r,dq,kind", [
    (300, 256, 320, 128, 256, "t3"),        # two 64-column tail chunks
    (200, 192, 256, 256, 0, "outliers"),    # the largest rank: four tail chunks, split adapter kernels
    (520, 320, 192, 200, 256, "t5"),        # ragged padded rank 208
    (2048, 256, 384, 128, 256, "spike"),    # many tokens at a rank past the unsplit kernels
])
def test_layer_wide_rank_heavy_tails(M, o, h, r, dq, kind):
    say(f"wide rank M={M} o={o} h={h} r={r} dq={dq} weights={kind}")
    d = synth.random_case(seed=500 + r, rows=o, cols=h, M=M, r=r)
    d["W"] = heavy_weight(np.random.default_rng(600 + r), (o, h), kind)
    check_layer(d, 2.0, dq)


def test_layer_property_sweep():
    """Seeded draws over the layer's parameter space (h and o multiples of 64 up to 768, M from 1 to
    700, r from 1 to 256, double quant on or off, four weight distributions), each against the oracle."""
    rng = np.random.default_rng(2024)
    kinds = ("normal", "t3", "outliers", "spike")
    for case in range(14):
        o, h = 64 * int(rng.integers(1, 13)), 64 * int(rng.integers(1, 13))
        M = int(rng.integers(1, 701))
        r = int(rng.choice([1, 2, 8, 15, 16, 17, 33, 64, 65, 100, 128, 200, 256]))
        dq = int(rng.choice([0, 256]))
        kind = kinds[case % 4]
        s = float(rng.choice([0.5, 1.0, 2.0, 16.0 / np.sqrt(r)]))
        say(f"sweep {case}: M={M} o={o} h={h} r={r} dq={dq} s={s:.3f} weights={kind}")
        d = synth.random_case(seed=700 + case, rows=o, cols=h, M=M, r=r)
        if kind != "normal":
            d["W"] = heavy_weight(rng, (o, h), kind)
        check_layer(d, s, dq)


# ---------------------------------------------------------------------------
# forward / backward
# ---------------------------------------------------------------------------

def run_layer(d, s, dq, use_T=True, want_dX=True):
    W = dev(d["W"])
    q = nf4.quantize(W, dq)
    X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = nf4.fwd(q, X, L1, L2, s)
    dX, dL1, dL2 = nf4.bwd(q, X, dY, L1, L2, s, T=T if use_T else None, want_dX=want_dX)
    torch.cuda.synchronize()
    return Y, T, dX, dL1, dL2


def oracle_layer(d, s, dq):
    wh = oracle.dequantize(oracle.quantize(d["W"], 64, dq))
    Y, T = oracle.fwd(d["X"], wh, d["L1"], d["L2"], s)
    dX, dL1, dL2, _ = oracle.bwd(d["X"], d["dY"], wh, d["L1"], d["L2"], s)
    return Y, T, dX, dL1, dL2


def check_layer(d, s, dq):
    Y, T, dX, dL1, dL2 = run_layer(d, s, dq)
    Yr, Tr, dXr, dL1r, dL2r = oracle_layer(d, s, dq)
    check_close("T", T, Tr)
    check_close("Y", Y, Yr)
    check_close("dX", dX, dXr)
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


def test_layer_c1():
    d = synth.layer_inputs(synth.C1)
    say("c1 512x512 r=8 M=128")
    check_layer(d, d["s"], d["dq_group"])


@pytest.mark.parametrize("M,o,h,r,dq,s", [
    (1, 64, 64, 1, 0, 2.0),
    (37, 320, 192, 17, 256, 0.5),
    (300, 128, 576, 8, 0, 2.0),
    (257, 384, 256, 64, 256, 2.0),
    (129, 192, 128, 100, 0, 1.0 / 3.0),
    (513, 704, 640, 16, 256, 2.0),
])
def test_layer_ragged(M, o, h, r, dq, s):
    say(f"ragged M={M} o={o} h={h} r={r} dq={dq}")
    d = synth.random_case(seed=M + o + h + r, rows=o, cols=h, M=M, r=r)
    check_layer(d, s, dq)


@pytest.mark.parametrize("kt", list(range(1, 17)))
def test_gemm_k_steps(kt):
    """The fused GEMM alone at every K-step count from 1 to 16 (K = 64*kt), both
    directions, with a 16-column adapter tail and a ragged M: covers each length of
    the pipeline's prologue and tail, which load and dequantize nothing past K."""
    n = 64 * kt
    d = synth.random_case(seed=300 + kt, rows=n, cols=n, M=70, r=16)
    q = nf4.quantize(dev(d["W"]), 256)
    wh = oracle.dequantize(oracle.quantize(d["W"], 64, 256)).astype(np.float64)
    A2 = (d["X"][:, :16].float() * 0.5).bfloat16()
    B2 = (d["dY"][:16, :].t().float() * 0.02).bfloat16().contiguous()  # [n][16]
    say(f"gemm K-steps {kt}: M=70, o=h={n}")
    Y = nf4.matmul(q, dev(d["X"]), False, dev(A2), dev(B2))
    dX = nf4.matmul(q, dev(d["dY"]), True, dev(A2), dev(B2))
    torch.cuda.synchronize()
    tail = f64(A2) @ f64(B2).T
    check_close("Y", Y, f64(d["X"]) @ wh.T + tail)
    check_close("dX", dX, f64(d["dY"]) @ wh + tail)


def test_gemm_long_k():
    """The fused GEMM with K = 16448 (257 K steps) in both directions: past 16384 the tile order
    takes one row panel at a time; 300 rows give two row panels and a ragged tail."""
    for o, h in ((128, 16448), (16448, 128)):
        d = synth.random_case(seed=700 + o, rows=o, cols=h, M=300, r=16)
        q = nf4.quantize(dev(d["W"]), 256)
        wh = oracle.dequantize(oracle.quantize(d["W"], 64, 256)).astype(np.float64)
        say(f"gemm long K: M=300, o={o}, h={h}")
        if h > o:
            A2 = (d["X"][:, :16].float() * 0.5).bfloat16()
            B2 = (d["dY"][:16, :].t().float() * 0.02).bfloat16().contiguous()  # [o][16]
            Y = nf4.matmul(q, dev(d["X"]), False, dev(A2), dev(B2))
            torch.cuda.synchronize()
            check_close("Y", Y, f64(d["X"]) @ wh.T + f64(A2) @ f64(B2).T)
        else:
            A2 = (d["dY"][:, :16].float() * 0.5).bfloat16()
            B2 = (d["X"][:16, :].t().float() * 0.02).bfloat16().contiguous()  # [h][16]
            dX = nf4.matmul(q, dev(d["dY"]), True, dev(A2), dev(B2))
            torch.cuda.synchronize()
            check_close("dX", dX, f64(d["dY"]) @ wh + f64(A2) @ f64(B2).T)


@pytest.mark.parametrize("M,o,h,r", [
    (1000, 320, 192, 16),    # padded rank 16: 8-row whole-K workgroups, 16-wave token chunks
    (1024, 320, 192, 8),     # rank 8 padded to 16: the whole-line G product reads zero rows of L2
    (2048, 256, 320, 1),     # rank 1 padded to 16
    (2048, 320, 192, 20),    # padded rank 32, r not a multiple of 8 (padded T)
    (2048, 384, 256, 40),    # padded rank 48
    (2048, 320, 576, 64),    # padded rank 64
])
def test_layer_unsplit_adapter_kernels(M, o, h, r):
    """Token counts large enough for the whole-K and all-token adapter kernels at
    every padded rank they serve, with ragged K steps, column bands and chunks."""
    say(f"unsplit adapter products M={M} o={o} h={h} r={r}")
    d = synth.random_case(seed=400 + r, rows=o, cols=h, M=M, r=r)
    check_layer(d, 2.0, 256)


def test_layer_options_and_determinism():
    d = synth.random_case(seed=21, rows=256, cols=320, M=200, r=16)
    a = run_layer(d, 2.0, 256, use_T=True)
    b = run_layer(d, 2.0, 256, use_T=False)
    c = run_layer(d, 2.0, 256, use_T=True, want_dX=False)
    e = run_layer(d, 2.0, 256, use_T=True)
    for x, y in zip(a, e):                      # repeat: identical bits
        assert torch.equal(x, y)
    for i in (2, 3, 4):                         # T recomputed inside bwd: identical bits
        assert torch.equal(a[i], b[i])
    assert c[2] is None                          # early backward stop: no dX, same adapter grads
    assert torch.equal(a[3], c[3]) and torch.equal(a[4], c[4])


def test_adapter_zero_cases():
    d = synth.random_case(seed=23, rows=192, cols=256, M=96, r=8)
    d["L2"] = torch.zeros_like(d["L2"])
    Y, T, dX, dL1, dL2 = run_layer(d, 2.0, 0)
    Yr, _, dXr, _, dL2r = oracle_layer(d, 2.0, 0)
    assert not torch.any(dL1)                   # G = 0 -> dL1 = 0 exactly
    check_close("Y (L2=0)", Y, Yr)
    check_close("dL2 (L2=0)", dL2, dL2r)
    d = synth.random_case(seed=24, rows=192, cols=256, M=96, r=8)
    d["L1"] = torch.zeros_like(d["L1"])
    _, T, _, _, dL2 = run_layer(d, 2.0, 0)
    assert not torch.any(T) and not torch.any(dL2)   # T = 0 -> dL2 = 0 exactly


def test_empty_batch():
    d = synth.random_case(seed=25, rows=128, cols=128, M=1, r=8)
    q = nf4.quantize(dev(d["W"]), 0)
    X = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    L1, L2 = dev(d["L1"]), dev(d["L2"])
    Y, T = nf4.fwd(q, X, L1, L2, 2.0)
    assert Y.shape == (0, 128)
    dL1 = torch.full((128, 8), 7.0, device=DEV)
    dL2 = torch.full((8, 128), 7.0, device=DEV)
    nf4.bwd(q, X, torch.empty(0, 128, dtype=torch.bfloat16, device=DEV), L1, L2, 2.0, outs=(None, dL1, dL2))
    torch.cuda.synchronize()
    assert not torch.any(dL1) and not torch.any(dL2)


def test_layer_c2_full():
    say("c2 4096x4096 r=16 M=2048, double quant")
    d = synth.layer_inputs(synth.C2)
    check_layer(d, d["s"], d["dq_group"])
    # the step's one-pass quantize + error at this size (codes with 8-bit scales, error with plain absmax)
    q, err = nf4.quantize_error(dev(d["W"]), d["dq_group"], 0)
    check_quant(q, oracle.quantize(d["W"], 64, d["dq_group"]))
    got, want = float(err.cpu()[0]), oracle.layer_error(d["W"], 64, 0)
    say(f"  one-pass error {got:.12g} oracle {want:.12g}")
    assert abs(got - want) <= 1e-6 * want


# ---------------------------------------------------------------------------
# protected (bf16) linears through the same fused kernels
# ---------------------------------------------------------------------------

def check_bf16_layer(d, s, use_T=True):
    Wb = synth.bf16(d["W"])  # the protected weight, stored in bf16
    W = dev(Wb)
    X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = nf4.bf16_fwd(W, X, L1, L2, s)
    dX, dL1, dL2 = nf4.bf16_bwd(W, X, dY, L1, L2, s, T=T if use_T else None)
    torch.cuda.synchronize()
    Yr, Tr = oracle.fwd(d["X"], Wb, d["L1"], d["L2"], s)
    dXr, dL1r, dL2r, _ = oracle.bwd(d["X"], d["dY"], Wb, d["L1"], d["L2"], s)
    check_close("T", T, Tr)
    check_close("Y", Y, Yr)
    check_close("dX", dX, dXr)
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


def test_bf16_layer_c1():
    d = synth.layer_inputs(synth.C1)
    check_bf16_layer(d, d["s"])


@pytest.mark.parametrize("M,o,h,r,s", [
    (1, 64, 64, 1, 2.0),
    (37, 320, 192, 17, 0.5),
    (300, 128, 576, 8, 2.0),
    (513, 704, 640, 16, 2.0),
])
def test_bf16_layer_ragged(M, o, h, r, s):
    say(f"bf16 layer M={M} o={o} h={h} r={r}")
    d = synth.random_case(seed=M + o + h, rows=o, cols=h, M=M, r=r)
    check_bf16_layer(d, s, use_T=(r % 2 == 0))


def test_bf16_layer_c2_full():
    say("bf16 layer 4096x4096 r=16 M=2048")
    d = synth.layer_inputs(synth.C2)
    check_bf16_layer(d, d["s"])


# ---------------------------------------------------------------------------
# stack runner: forward over every linear, backward down to a cut
# ---------------------------------------------------------------------------

def test_stack_runner_matches_layer_calls():
    M = 96
    spec = [  # (format, o, h, r, dq)
        ("nf4", 128, 192, 8, 0), ("bf16", 192, 128, 8, 0), ("nf4", 256, 128, 0, 256),
        ("nf4", 128, 256, 16, 0), ("bf16", 64, 128, 0, 0), ("nf4", 128, 64, 4, 256),
    ]
    cut = 1
    lins, refs = [], []
    sentinel = 7.0
    for i, (fmt, o, h, r, dq) in enumerate(spec):
        d = synth.random_case(seed=100 + i, rows=o, cols=h, M=M, r=max(r, 1))
        L = {"X": dev(d["X"]), "dY": dev(d["dY"]), "r": r, "s": 2.0,
             "Y": torch.empty(M, o, dtype=torch.bfloat16, device=DEV)}
        if fmt == "nf4":
            L["q"] = nf4.quantize(dev(d["W"]), dq)
        else:
            L["w"] = dev(synth.bf16(d["W"]))
        if r:
            L["L1"], L["L2"] = dev(d["L1"]), dev(d["L2"])
            L["T"] = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
            L["dL1"] = torch.full((h, r), sentinel, dtype=torch.float32, device=DEV)
            L["dL2"] = torch.full((r, o), sentinel, dtype=torch.float32, device=DEV)
        if i != cut:  # the lowest linear above the cut needs no input gradient
            L["dX"] = torch.full((M, h), sentinel, dtype=torch.bfloat16, device=DEV)
        lins.append(L)
        refs.append(d)
    st = nf4.Stack(lins, M)
    st.fwd()
    st.bwd(cut=cut)
    torch.cuda.synchronize()
    for i, (L, d, (fmt, o, h, r, dq)) in enumerate(zip(lins, refs, spec)):
        say(f"  linear {i}: {fmt} {o}x{h} r={r}")
        if r:
            if fmt == "nf4":
                Y, T = nf4.fwd(L["q"], L["X"], L["L1"], L["L2"], 2.0)
                dX, dL1, dL2 = nf4.bwd(L["q"], L["X"], L["dY"], L["L1"], L["L2"], 2.0, T=T)
            else:
                Y, T = nf4.bf16_fwd(L["w"], L["X"], L["L1"], L["L2"], 2.0)
                dX, dL1, dL2 = nf4.bf16_bwd(L["w"], L["X"], L["dY"], L["L1"], L["L2"], 2.0, T=T)
            assert torch.equal(L["Y"], Y) and torch.equal(L["T"], T)
            if i >= cut:
                assert torch.equal(L["dL1"], dL1) and torch.equal(L["dL2"], dL2)
            else:
                assert bool((L["dL1"] == sentinel).all()) and bool((L["dL2"] == sentinel).all())
            if "dX" in L:
                if i >= cut:
                    assert torch.equal(L["dX"], dX)
                else:
                    assert bool((L["dX"] == sentinel).all())
        else:
            # plain product: Y = X W^T (and dX = dY W above the cut), against the oracle
            Wref = synth.bf16(d["W"]) if fmt == "bf16" else oracle.dequantize(oracle.quantize(d["W"], 64, dq))
            z1, z2 = np.zeros((h, 1)), np.zeros((1, o))
            Yr, _ = oracle.fwd(d["X"], Wref, z1, z2, 2.0)
            check_close("Y", L["Y"], Yr)
            if "dX" in L and i >= cut:
                dXr, _, _, _ = oracle.bwd(d["X"], d["dY"], Wref, z1, z2, 2.0)
                check_close("dX", L["dX"], dXr)
    # one adapted linear against the oracle as well
    d = refs[3]
    wh = oracle.dequantize(oracle.quantize(d["W"], 64, 0))
    Yr, _ = oracle.fwd(d["X"], wh, d["L1"], d["L2"], 2.0)
    check_close("Y[3]", lins[3]["Y"], Yr)


# ---------------------------------------------------------------------------
# merge: W' = base + s (L1 L2)^T
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("o,h,r,base", [(512, 512, 8, "fp32"), (320, 192, 17, "nf4"), (4096, 4096, 16, "nf4dq"),
                                        (192, 640, 100, "fp32"), (64, 64, 1, "nf4dq")])
def test_merge(o, h, r, base):
    d = synth.random_case(seed=o + r, rows=o, cols=h, M=1, r=r)
    s = 2.0
    if base == "fp32":
        src, ref_base = dev(d["W"]), d["W"]
    else:
        dq = 256 if base == "nf4dq" else 0
        src = nf4.quantize(dev(d["W"]), dq)
        ref_base = oracle.dequantize(oracle.quantize(d["W"], 64, dq))
    ref = oracle.merge(ref_base, d["L1"], d["L2"], s)
    L1, L2 = dev(d["L1"]), dev(d["L2"])
    got = nf4.merge(src, L1, L2, s).cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    say(f"  merge {o}x{h} r={r} {base}: max|err| {err.max():.2e}, max|ref| {np.abs(ref).max():.2e}")
    # fp32 bound: bf16 x bf16 products are exact in fp32; the r-term FMA chain,
    # the scaling by s and the final add each round to nearest (unit 2^-24)
    u = 2.0 ** -24
    terms = s * (np.abs(oracle.lora._f64(d["L1"])) @ np.abs(oracle.lora._f64(d["L2"]))).T
    tol32 = (r + 2) * u * terms + 2 * u * np.abs(ref)
    assert np.all(err <= tol32), float(np.max(err - tol32))
    gotb = nf4.merge(src, L1, L2, s, bf16=True).cpu().float().numpy().astype(np.float64)
    # bf16: round-to-nearest of the fp32 value v, within half a bf16 ulp of it:
    # 2^(floor(log2|v|) - 8) <= 2^-8 |v|
    tolb = 2.0 ** -8 * (np.abs(ref) + tol32) + tol32
    assert np.all(np.abs(gotb - ref) <= tolb), float(np.max(np.abs(gotb - ref) - tolb))


# ---------------------------------------------------------------------------
# other 4-bit codebooks (int4, fp4) through the same kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("codebook", ["int4", "fp4"])
@pytest.mark.parametrize("dq", [0, 256])
def test_codebook_quantize(codebook, dq):
    for W in (synth.layer_inputs(synth.C1)["W"], edge_weights(codebook)):
        q = nf4.quantize(dev(W), dq, codebook=codebook)
        ref = oracle.quantize(W, 64, dq, codebook)
        check_quant(q, ref)
        wh = nf4.dequantize(q).cpu().numpy()
        assert np.array_equal(wh.view(np.uint32), oracle.dequantize(ref).view(np.uint32))
        whb = nf4.dequantize(q, bf16=True).cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(whb, oracle.dequantize_bf16_bits(ref))


@pytest.mark.parametrize("codebook", ["int4", "fp4"])
def test_codebook_layer_error(codebook):
    for W, dq in ((synth.layer_weight(synth.C2)[:512], 0), (edge_weights(codebook), 256)):
        got = float(nf4.layer_error(dev(W), dq, codebook=codebook).cpu())
        want = oracle.layer_error(W, 64, dq, codebook)
        say(f"  {codebook} dq={dq}: {got:.9f} vs {want:.9f}")
        assert abs(got - want) <= 1e-6 * want


@pytest.mark.parametrize("codebook", ["int4", "fp4"])
def test_codebook_layer(codebook):
    for d, s, dq in ((synth.layer_inputs(synth.C1), 2.0, 0),
                     (synth.random_case(seed=9, rows=320, cols=192, M=37, r=17), 0.5, 256)):
        q = nf4.quantize(dev(d["W"]), dq, codebook=codebook)
        X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
        Y, T = nf4.fwd(q, X, L1, L2, s)
        dX, dL1, dL2 = nf4.bwd(q, X, dY, L1, L2, s, T=T)
        torch.cuda.synchronize()
        wh = oracle.dequantize(oracle.quantize(d["W"], 64, dq, codebook))
        Yr, Tr = oracle.fwd(d["X"], wh, d["L1"], d["L2"], s)
        dXr, dL1r, dL2r, _ = oracle.bwd(d["X"], d["dY"], wh, d["L1"], d["L2"], s)
        check_close("Y", Y, Yr)
        check_close("dX", dX, dXr)
        check_close("dL1", dL1, dL1r)
        check_close("dL2", dL2, dL2r)



# ---------------------------------------------------------------------------
# residual second stage through the same kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dq", [0, 256])
def test_residual_quantize(dq):
    for W in (synth.layer_inputs(synth.C1)["W"], edge_weights()):
        q = nf4.quantize(dev(W), dq, residual=True)
        r1, r2 = oracle.quantize_residual(W, 64, dq)
        check_quant(q, r1)
        check_quant(q.residual, r2)
        wh = nf4.dequantize(q).cpu().numpy()
        assert np.array_equal(wh.view(np.uint32), oracle.dequantize_residual(r1, r2).view(np.uint32))
        whb = nf4.dequantize(q, bf16=True).cpu().view(torch.int16).numpy().view(np.uint16)
        ref_b = torch.from_numpy(oracle.dequantize_residual(r1, r2)).to(torch.bfloat16)
        assert np.array_equal(whb, ref_b.view(torch.int16).numpy().view(np.uint16))


def test_residual_layer_and_merge():
    for d, s, dq in ((synth.layer_inputs(synth.C1), 2.0, 0),
                     (synth.random_case(seed=19, rows=384, cols=256, M=257, r=64), 2.0, 256)):
        q = nf4.quantize(dev(d["W"]), dq, residual=True)
        X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
        Y, T = nf4.fwd(q, X, L1, L2, s)
        dX, dL1, dL2 = nf4.bwd(q, X, dY, L1, L2, s, T=T)
        torch.cuda.synchronize()
        wh = oracle.dequantize_residual(*oracle.quantize_residual(d["W"], 64, dq))
        Yr, _ = oracle.fwd(d["X"], wh, d["L1"], d["L2"], s)
        dXr, dL1r, dL2r, _ = oracle.bwd(d["X"], d["dY"], wh, d["L1"], d["L2"], s)
        check_close("Y", Y, Yr)
        check_close("dX", dX, dXr)
        check_close("dL1", dL1, dL1r)
        check_close("dL2", dL2, dL2r)
        # the residual stage tightens the base: closer to the fp32 W than one stage
        one = oracle.dequantize(oracle.quantize(d["W"], 64, dq))
        assert np.linalg.norm(wh - d["W"]) < 0.5 * np.linalg.norm(one - d["W"])
        # merge on the two-stage base
        got = nf4.merge(q, L1, L2, s).cpu().numpy().astype(np.float64)
        ref = oracle.merge(wh, d["L1"], d["L2"], s)
        u = 2.0 ** -24
        terms = s * (np.abs(oracle.lora._f64(d["L1"])) @ np.abs(oracle.lora._f64(d["L2"]))).T
        tol = (d["L1"].shape[1] + 2) * u * terms + 2 * u * np.abs(ref)
        viol = np.abs(got - ref) - tol
        i = np.unravel_index(np.argmax(viol), viol.shape)
        assert viol[i] <= 0, (i, got[i], ref[i], wh[i], tol[i], terms[i])


def test_binding_rejects_bad_arguments():
    """The library takes raw pointers, so the binding checks every tensor's device, dtype, shape and layout
    against the weight before any launch; each bad argument below raises ValueError and nothing runs."""
    d = synth.random_case(seed=27, rows=128, cols=192, M=64, r=16)
    q = nf4.quantize(dev(d["W"]), 0)
    X, L1, L2, dY = dev(d["X"]), dev(d["L1"]), dev(d["L2"]), dev(d["dY"])
    Y, T = nf4.fwd(q, X, L1, L2, 2.0)
    bad = [
        ("X width", lambda: nf4.fwd(q, X[:, :128].contiguous(), L1, L2, 2.0)),
        ("X not contiguous", lambda: nf4.fwd(q, torch.empty(192, 64, dtype=torch.bfloat16, device=DEV).t(), L1, L2,
                                             2.0)),
        ("X on the host", lambda: nf4.fwd(q, X.cpu(), L1, L2, 2.0)),
        ("X dtype", lambda: nf4.fwd(q, X.float(), L1, L2, 2.0)),
        ("L1 rows", lambda: nf4.fwd(q, X, L1[:128].contiguous(), L2, 2.0)),
        ("L2 shape", lambda: nf4.fwd(q, X, L1, L2[:8].contiguous(), 2.0)),
        ("out shape", lambda: nf4.fwd(q, X, L1, L2, 2.0, out=torch.empty(64, 64, dtype=torch.bfloat16, device=DEV))),
        ("T_out shape", lambda: nf4.fwd(q, X, L1, L2, 2.0, T_out=torch.empty(32, 16, dtype=torch.bfloat16,
                                                                              device=DEV))),
        ("ws dtype", lambda: nf4.fwd(q, X, L1, L2, 2.0, ws=torch.empty(1 << 20, dtype=torch.float32, device=DEV))),
        ("dY rows", lambda: nf4.bwd(q, X, dY[:32].contiguous(), L1, L2, 2.0)),
        ("T rows", lambda: nf4.bwd(q, X, dY, L1, L2, 2.0, T=T[:32].contiguous())),
        ("dL1 dtype", lambda: nf4.bwd(q, X, dY, L1, L2, 2.0, outs=(None, torch.empty(192, 16, dtype=torch.bfloat16,
                                                                                      device=DEV),
                                                                  torch.empty(16, 128, device=DEV)))),
        ("quantize into another shape", lambda: nf4.quantize(dev(d["W"])[:64].contiguous(), 0, out=q)),
        ("dequantize out shape", lambda: nf4.dequantize(q, out=torch.empty(64, 192, device=DEV))),
        ("bf16 W width", lambda: nf4.bf16_fwd(torch.empty(128, 128, dtype=torch.bfloat16, device=DEV), X, L1, L2,
                                              2.0)),
        ("matmul A2 without B2", lambda: nf4.matmul(q, X, A2=T)),
        ("matmul A width", lambda: nf4.matmul(q, X, transpose=True)),
        ("topk out too short", lambda: nf4.topk(torch.zeros(8, dtype=torch.float64, device=DEV), 4,
                                                out=torch.empty(2, dtype=torch.int32, device=DEV))),
        ("error batch out too short", lambda: nf4.layer_error_batch([dev(d["W"])] * 3, 0,
                                                                    out=torch.empty(2, dtype=torch.float64,
                                                                                    device=DEV))),
        ("merge L2 shape", lambda: nf4.merge(q, L1, L2[:, :64].contiguous(), 2.0)),
        ("stack X shape", lambda: nf4.Stack([{"q": q, "r": 16, "s": 2.0, "L1": L1, "L2": L2,
                                              "X": X[:, :64].contiguous(), "Y": Y}], 64)),
    ]
    for name, call in bad:
        with pytest.raises(ValueError):
            call()
        torch.cuda.synchronize()
    Y2, _ = nf4.fwd(q, X, L1, L2, 2.0)     # the same call with good arguments still runs
    assert torch.equal(Y2, Y)
