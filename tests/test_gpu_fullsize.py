"""Full-size workloads on the HIP path against the CPU oracle (needs an MI355X).

The layer workloads run at their real shapes in the launch configuration the
benchmark uses; the oracle checks what it can compute at that size:
  * codes, scales and dequantized weights (fp32 and bf16) over the whole matrix, bit-exact,
    and the layer error from the same one-pass quantize within 1e-6;
  * Y and dX on sampled token rows (each output row depends only on its own
    input row, so the oracle runs on those rows alone);
  * dL1 and dL2 over all tokens: every token contributes its own term, so the
    oracle's gradients of consecutive token chunks are added up.
The 280-linear stack checks the per-linear errors of sampled linears against
the oracle, the batched pass over all 280 against the per-linear errors bit
for bit, and the top-K selection against the errors it ranks.
Tolerances are those of the other parity tests.
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


def check_close(name, got, want):
    g = f64(got)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    ref = np.max(np.abs(w))
    err = np.max(np.abs(g - w))
    rms = np.sqrt(np.mean((g - w) ** 2)) / max(np.sqrt(np.mean(w ** 2)), 1e-300)
    say(f"  {name}: max|err|/max|ref| = {err / max(ref, 1e-300):.2e}  rel-rms = {rms:.2e}")
    assert err <= TOL_MAX * ref, f"{name}: max|err| {err:.3e} > {TOL_MAX} * {ref:.3e}"
    assert rms <= TOL_RMS, f"{name}: relative rms {rms:.3e}"


def check_quant(q, ref):
    assert np.array_equal(q.packed_codes.cpu().numpy(), ref.packed), "codes"
    if ref.dq_group:
        assert np.array_equal(q.c8.cpu().numpy(), ref.c8), "c8"
        assert np.array_equal(q.dq_step.cpu().numpy().view(np.uint32), ref.dq_scale.view(np.uint32)), "dq step"
    else:
        assert np.array_equal(q.absmax_f32.cpu().numpy().view(np.uint32), ref.absmax.view(np.uint32)), "absmax"


def sampled_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=n - 2, replace=False).tolist()) | {0, M - 1}
    return sorted(rows)


def check_layer_fullsize(layer, n_rows=16, chunk=1024):
    say(f"{layer.name}: W [{layer.rows}][{layer.cols}], M={layer.M}, r={layer.r}, dq={layer.dq_group}")
    d = synth.layer_inputs(layer)
    W, s, dq, M = d["W"], d["s"], d["dq_group"], layer.M

    say("  HIP path: quantize + layer error (one pass), fwd, bwd")
    q, err = nf4.quantize_error(dev(W), dq, dq)
    X, L1, L2, dY = (dev(d[k]) for k in ("X", "L1", "L2", "dY"))
    Y, T = nf4.fwd(q, X, L1, L2, s)
    dX, dL1, dL2 = nf4.bwd(q, X, dY, L1, L2, s, T=T)
    torch.cuda.synchronize()
    del X, dY

    say("  oracle quantize (whole matrix)")
    ref = oracle.quantize(W, 64, dq)
    check_quant(q, ref)
    wh = oracle.dequantize(ref)
    assert np.array_equal(nf4.dequantize(q).cpu().numpy().view(np.uint32), wh.view(np.uint32)), "dequantized W"
    # bf16 output: at c5 the dequantize kernel's grid-stride loop takes several rounds
    whb = nf4.dequantize(q, bf16=True).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(whb, oracle.dequantize_bf16_bits(ref)), "dequantized W, bf16"
    del q, whb
    say("  oracle layer error")
    got, want = float(err.cpu()[0]), oracle.layer_error(W, 64, dq)
    say(f"  error: gpu {got:.12g} oracle {want:.12g}")
    assert abs(got - want) <= 1e-6 * want, (got, want)

    rows = sampled_rows(M, n_rows, layer.seed)
    say(f"  oracle rows {rows[:4]}... ({len(rows)} rows)")
    Yr, Tr = oracle.fwd(d["X"][rows], wh, d["L1"], d["L2"], s)
    check_close("T rows", T[rows], Tr)
    check_close("Y rows", Y[rows], Yr)
    dXr, _, _, _ = oracle.bwd(d["X"][rows], d["dY"][rows], wh, d["L1"], d["L2"], s)
    check_close("dX rows", dX[rows], dXr)
    del wh

    say(f"  oracle adapter gradients over all {M} tokens ({chunk}-token chunks)")
    dL1r = np.zeros((layer.cols, layer.r))
    dL2r = np.zeros((layer.r, layer.rows))
    for c0 in range(0, M, chunk):
        _, a, b = oracle.adapter_grads(d["X"][c0:c0 + chunk], d["dY"][c0:c0 + chunk], d["L1"], d["L2"], s)
        dL1r += a
        dL2r += b
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


@pytest.mark.parametrize("layer", [synth.C3_GATE, synth.C3_UP, synth.C3_DOWN], ids=["gate", "up", "down"])
def test_c3_mlp_fullsize(layer):
    check_layer_fullsize(layer)


def test_c5_up_projection_fullsize():
    check_layer_fullsize(synth.C5, n_rows=8, chunk=1024)


def test_c4_stack_error_topk():
    stack = synth.c4_stack()
    n = len(stack)
    # one oracle check per tail weight (df 3, 5, 30), on 5120 x 5120 linears
    sample = []
    for df in synth.C4_DFS:
        sample.append(next(l.index for l in stack if l.df == df and l.kind in ("q", "k", "v", "o")))
    say(f"c4: {n} linears, oracle on linears {sample}")
    # 16-byte spaced slots: the C ABI wants 16-byte aligned output pointers
    slots = torch.empty(n, 2, dtype=torch.float64, device=DEV)
    ws = torch.empty(nf4.workspace_bytes(nf4.NF4_OP_ERROR, 0, synth.C4_FFN, synth.C4_HIDDEN, 1),
                     dtype=torch.uint8, device=DEV)
    kept, Ws = {}, []
    for lin in stack:
        W = synth.c4_weight(lin, device=DEV)
        nf4.layer_error(W, 0, out=slots[lin.index], ws=ws[: nf4.workspace_bytes(nf4.NF4_OP_ERROR, 0, lin.rows,
                                                                                lin.cols, 1)])
        Ws.append(W)   # all 280 weights stay resident (50.75 GB) for the batched pass below
        if lin.index in sample:
            kept[lin.index] = W.cpu().numpy()
        if lin.index % 40 == 39:
            torch.cuda.synchronize()
            say(f"  {lin.index + 1} linears done")
    errors = slots[:, 0].contiguous()
    say("  the same pass batched (nf4_layer_error_batch, 64 linears per launch pair)")
    eb = nf4.layer_error_batch(Ws, 0)
    torch.cuda.synchronize()
    del Ws
    assert np.array_equal(eb.cpu().numpy().view(np.uint64), errors.cpu().numpy().view(np.uint64))
    top = nf4.topk(errors, synth.C4_TOPK).cpu().numpy().tolist()
    e = errors.cpu().numpy()
    say(f"  top-{synth.C4_TOPK}: {top}, errors {np.round(e[top], 5).tolist()}")
    # the selection ranks the errors it was given (descending, ties to the lower index)
    assert top == oracle.topk(e, synth.C4_TOPK)
    assert np.all(np.isfinite(e)) and np.all(e > 0)
    for i, Wc in kept.items():
        want = oracle.layer_error(Wc, 64, 0)
        say(f"  linear {i} ({stack[i].kind}, df {stack[i].df}): {e[i]:.9f} vs oracle {want:.9f}")
        assert abs(e[i] - want) <= 1e-6 * want
    # heavier tails quantize worse: the mean error falls as df grows
    by_df = {df: float(np.mean([e[l.index] for l in stack if l.df == df])) for df in synth.C4_DFS}
    say(f"  mean error by df: {by_df}")
    assert by_df[3] > by_df[5] > by_df[30]


def test_c4_stack_layers_fullsize():
    """The c4 stack's forward and early-stopped backward at its own shapes (AQLoRA, section 3.2
    Precision allocation and section 3.3 Adapter placement): an NF4 q projection (5120 x 5120), an NF4
    gate projection (13824 x 5120) and a protected bf16 down projection (5120 x 13824), M = 4096
    tokens, r = 16, s = 2, run as one stack through nf4_stack_fwd / nf4_stack_bwd.  The q projection is
    the lowest adapted linear: it gets its adapter gradients but no input gradient.  Y and dX are
    checked on sampled token rows, dL1 and dL2 over all tokens, each against the oracle."""
    stack = synth.c4_stack()
    picks = [next(l for l in stack if l.kind == k) for k in ("q", "gate", "down")]
    M, r, s = synth.C4_TOKENS, 16, 2.0
    rng = np.random.default_rng(41)
    lins, refs = [], []
    sentinel = 7.0
    for i, lin in enumerate(picks):
        o, h = lin.rows, lin.cols
        Wd = synth.c4_weight(lin, device=DEV)
        X = synth.bf16((rng.standard_normal((M, h))).astype(np.float32))
        dY = synth.bf16((rng.standard_normal((M, o))).astype(np.float32))
        L1 = synth.bf16((rng.standard_normal((h, r)) * 0.02).astype(np.float32))
        L2 = synth.bf16((rng.standard_normal((r, o)) * 0.02).astype(np.float32))
        L = {"X": dev(X), "dY": dev(dY), "r": r, "s": s, "L1": dev(L1), "L2": dev(L2),
             "Y": torch.empty(M, o, dtype=torch.bfloat16, device=DEV),
             "T": torch.empty(M, r, dtype=torch.bfloat16, device=DEV),
             "dL1": torch.full((h, r), sentinel, dtype=torch.float32, device=DEV),
             "dL2": torch.full((r, o), sentinel, dtype=torch.float32, device=DEV),
             "dX": torch.full((M, h), sentinel, dtype=torch.bfloat16, device=DEV) if i > 0 else None}
        if lin.kind == "down":                  # the protected linear: bf16 weight, no dequantization
            L["w"] = Wd.to(torch.bfloat16).contiguous()
            wref = L["w"].float().cpu().numpy()
        else:
            L["q"] = nf4.quantize(Wd, 256)
            wref = oracle.dequantize(oracle.quantize(Wd.cpu().numpy(), 64, 256))
            check_quant(L["q"], oracle.quantize(Wd.cpu().numpy(), 64, 256))
        del Wd
        lins.append(L)
        refs.append(dict(X=X, dY=dY, L1=L1, L2=L2, W=wref, lin=lin))
    st = nf4.Stack(lins, M)
    say(f"c4 stack linears {[p.kind for p in picks]} at M={M}, r={r}: fwd, bwd (cut 0, no dX for q)")
    st.fwd()
    st.bwd(cut=0)
    torch.cuda.synchronize()
    for i, (L, d) in enumerate(zip(lins, refs)):
        lin = d["lin"]
        say(f"  {lin.kind} [{lin.rows}][{lin.cols}] df {lin.df}")
        rows = sampled_rows(M, 12, 50 + i)
        Yr, Tr = oracle.fwd(d["X"][rows], d["W"], d["L1"], d["L2"], s)
        check_close("T rows", L["T"][rows], Tr)
        check_close("Y rows", L["Y"][rows], Yr)
        if L["dX"] is not None:
            dXr, _, _, _ = oracle.bwd(d["X"][rows], d["dY"][rows], d["W"], d["L1"], d["L2"], s)
            check_close("dX rows", L["dX"][rows], dXr)
        dL1r = np.zeros((lin.cols, r))
        dL2r = np.zeros((r, lin.rows))
        for c0 in range(0, M, 1024):
            _, a, b = oracle.adapter_grads(d["X"][c0:c0 + 1024], d["dY"][c0:c0 + 1024], d["L1"], d["L2"], s)
            dL1r += a
            dL2r += b
        check_close("dL1", L["dL1"], dL1r)
        check_close("dL2", L["dL2"], dL2r)


MAX_O, MAX_H = 1 << 20, 4096   # o * h = 2^32: the largest weight the fused kernels take


def test_max_size_weight():
    """The largest weight the header admits: o * h = 2^32 (1048576 x 4096, 16 GiB in fp32), where
    the quantize pass and the input-grad GEMM (K = 1048576, 16384 K steps) address the codes
    through 32-bit buffer ranges up to their ends.  W comes from the counter-based hash of synth
    on both sides, so the oracle draws only what it checks: codes and scales of sampled 4-row
    groups (one double-quantization group each) with and without the 8-bit scales, T and Y on
    sampled output columns, dX on one 64-column block of h (all 1048576 rows of that block), and
    dL1, dL2 over all 64 tokens."""
    o, h, M, r, s, seed = MAX_O, MAX_H, 64, 16, 2.0, 11
    say(f"max-size weight: W [{o}][{h}] ({o * h * 4 >> 30} GiB fp32), M={M}, r={r}")
    W = torch.empty((o, h), dtype=torch.float32, device=DEV)
    for r0 in range(0, o, 16384):
        W[r0:r0 + 16384] = synth.hash_weight_rows_torch(r0, 16384, h, seed, DEV)
    torch.cuda.synchronize()
    groups = [0, o // 2 + 4, o - 4]      # first rows of sampled 4-row groups

    say("  quantize with 8-bit scales, sampled groups against the oracle")
    q8 = nf4.quantize(W, 256)
    for r0 in groups:
        ref = oracle.quantize(synth.hash_weight(np.arange(r0, r0 + 4), np.arange(h), seed), 64, 256)
        got = q8.packed_codes[r0 * h // 2:(r0 + 4) * h // 2].cpu().numpy()
        assert np.array_equal(got, ref.packed), ("codes, dq", r0)
        assert np.array_equal(q8.c8[r0 * h // 64:(r0 + 4) * h // 64].cpu().numpy(), ref.c8), ("c8", r0)
        step = q8.dq_step[r0 // 4:r0 // 4 + 1].cpu().numpy()
        assert step.view(np.uint32)[0] == ref.dq_scale.view(np.uint32)[0], ("dq step", r0)
    del q8

    say("  quantize with fp32 scales, sampled groups against the oracle")
    q = nf4.quantize(W, 0)
    del W
    torch.cuda.empty_cache()
    for r0 in groups:
        ref = oracle.quantize(synth.hash_weight(np.arange(r0, r0 + 4), np.arange(h), seed), 64, 0)
        assert np.array_equal(q.packed_codes[r0 * h // 2:(r0 + 4) * h // 2].cpu().numpy(), ref.packed), ("codes", r0)
        got = q.absmax_f32[r0 * h // 64:(r0 + 4) * h // 64].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.absmax.view(np.uint32)), ("absmax", r0)

    rng = np.random.default_rng(seed)
    X = synth.bf16(rng.standard_normal((M, h), dtype=np.float32))
    L1 = synth.bf16(rng.standard_normal((h, r), dtype=np.float32) * np.float32(0.02))
    L2 = synth.bf16(rng.standard_normal((r, o), dtype=np.float32) * np.float32(0.02))
    dY = synth.bf16(rng.standard_normal((M, o), dtype=np.float32))
    say("  HIP path: fwd, bwd")
    Y, T = nf4.fwd(q, dev(X), dev(L1), dev(L2), s)
    dX, dL1, dL2 = nf4.bwd(q, dev(X), dev(dY), dev(L1), dev(L2), s, T=T)
    torch.cuda.synchronize()
    del q

    cols = np.array(sorted(set(rng.choice(o, size=30, replace=False).tolist()) | {0, o - 1}))
    say(f"  oracle Y on {cols.size} output columns")
    wh = oracle.dequantize(oracle.quantize(synth.hash_weight(cols, np.arange(h), seed), 64, 0))
    Yr, Tr = oracle.fwd(X, wh, L1, L2[:, torch.from_numpy(cols)], s)
    check_close("T", T, Tr)
    check_close("Y columns", Y[:, torch.from_numpy(cols).to(DEV)], Yr)

    b = 37
    hc = np.arange(64 * b, 64 * b + 64)
    say(f"  oracle dX on columns {hc[0]}..{hc[-1]} (all {o} rows of that block of W)")
    whs = oracle.dequantize(oracle.quantize(synth.hash_weight(np.arange(o), hc, seed), 64, 0))
    dXr = oracle.bwd(X[:, torch.from_numpy(hc)], dY, whs, L1[torch.from_numpy(hc)], L2, s)[0]
    check_close("dX block", dX[:, torch.from_numpy(hc).to(DEV)], dXr)
    del whs

    say("  oracle adapter gradients over all tokens")
    _, dL1r, dL2r = oracle.adapter_grads(X, dY, L1, L2, s)
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


def test_max_size_bf16_weight():
    """The largest protected bf16 weight the boundary admits (rows * cols < 2^31: 1048512 x 2048,
    4 GiB), whose input-grad GEMM reads the bf16 weight through a 32-bit buffer range of almost
    4 GiB; its last column tile of the forward is ragged (1048512 = 8191.5 x 128).  W is the bf16
    rounding of the counter-based hash on both sides; T and Y on sampled output columns, dX on
    one 64-column block of h, dL1 and dL2 over all tokens against the oracle."""
    o, h, M, r, s, seed = (1 << 20) - 64, 2048, 64, 16, 2.0, 12
    say(f"max-size bf16 weight: W [{o}][{h}] ({o * h * 2 / 2 ** 30:.2f} GiB bf16), M={M}, r={r}")
    W = torch.empty((o, h), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, o, 16384):
        n = min(16384, o - r0)
        W[r0:r0 + n] = synth.hash_weight_rows_torch(r0, n, h, seed, DEV).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    X = synth.bf16(rng.standard_normal((M, h), dtype=np.float32))
    L1 = synth.bf16(rng.standard_normal((h, r), dtype=np.float32) * np.float32(0.02))
    L2 = synth.bf16(rng.standard_normal((r, o), dtype=np.float32) * np.float32(0.02))
    dY = synth.bf16(rng.standard_normal((M, o), dtype=np.float32))
    say("  HIP path: bf16 fwd, bwd")
    Y, T = nf4.bf16_fwd(W, dev(X), dev(L1), dev(L2), s)
    dX, dL1, dL2 = nf4.bf16_bwd(W, dev(X), dev(dY), dev(L1), dev(L2), s, T=T)
    torch.cuda.synchronize()
    del W

    cols = np.array(sorted(set(rng.choice(o, size=30, replace=False).tolist()) | {0, o - 1}))
    say(f"  oracle Y on {cols.size} output columns")
    wr = synth.bf16(synth.hash_weight(cols, np.arange(h), seed))
    Yr, Tr = oracle.fwd(X, wr, L1, L2[:, torch.from_numpy(cols)], s)
    check_close("T", T, Tr)
    check_close("Y columns", Y[:, torch.from_numpy(cols).to(DEV)], Yr)

    hc = np.arange(64 * 21, 64 * 22)
    say(f"  oracle dX on columns {hc[0]}..{hc[-1]} (all {o} rows of that block of W)")
    ws = synth.bf16(synth.hash_weight(np.arange(o), hc, seed))
    dXr = oracle.bwd(X[:, torch.from_numpy(hc)], dY, ws, L1[torch.from_numpy(hc)], L2, s)[0]
    check_close("dX block", dX[:, torch.from_numpy(hc).to(DEV)], dXr)
    del ws

    say("  oracle adapter gradients over all tokens")
    _, dL1r, dL2r = oracle.adapter_grads(X, dY, L1, L2, s)
    check_close("dL1", dL1, dL1r)
    check_close("dL2", dL2, dL2r)


def test_token_count_past_one_launch():
    """A token count whose rank-16 adapter products need more work-items than one launch holds
    (2^32 - 1; the whole-K kernel spends 1024 on 8 rows, so M > 2^25 used to overflow the grid):
    M = 2^25 + 77 runs as three row ranges.  X is the counter-based hash (x 32) on both sides, so
    the oracle draws only sampled rows, chosen at the range edges, at 2^24 and 2^25 and at random.
    dY is zero except on half of those rows, so dL1 and dL2 over all M tokens come from those
    rows alone, and dX is exactly zero on the others.  The backward runs with the saved T and
    again recomputing T, whose product has row ranges of its own."""
    M, h, o, r, s, seed = (1 << 25) + 77, 64, 64, 16, 2.0, 13
    n = -(-M // (1 << 24))
    per = (-(-M // n) + 63) // 64 * 64
    edges = {0, 1, per - 1, per, per + 1, 2 * per - 1, 2 * per, (1 << 24) - 1, 1 << 24,
             (1 << 25) - 1, 1 << 25, M - 2, M - 1}
    rng = np.random.default_rng(seed)
    rows = np.array(sorted(edges | set(rng.choice(M, size=24, replace=False).tolist())))
    hot = rows[::2]                     # rows with a nonzero dY
    say(f"token count past one launch: M={M} ({n} ranges of {per} rows), W [{o}][{h}], r={r}, "
        f"{rows.size} sampled rows")
    X = torch.empty((M, h), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, M, 1 << 21):
        k = min(1 << 21, M - r0)
        X[r0:r0 + k] = (synth.hash_weight_rows_torch(r0, k, h, seed, DEV) * 32).to(torch.bfloat16)
    W = rng.standard_normal((o, h), dtype=np.float32)
    L1 = synth.bf16(rng.standard_normal((h, r), dtype=np.float32) * np.float32(0.1))
    L2 = synth.bf16(rng.standard_normal((r, o), dtype=np.float32) * np.float32(0.1))
    dYh = synth.bf16(rng.standard_normal((hot.size, o), dtype=np.float32))
    dY = torch.zeros((M, o), dtype=torch.bfloat16, device=DEV)
    dY[torch.from_numpy(hot).to(DEV)] = dev(dYh)
    q = nf4.quantize(dev(W), 256)
    say("  HIP path: fwd, bwd")
    Y, T = nf4.fwd(q, X, dev(L1), dev(L2), s)
    dX, dL1, dL2 = nf4.bwd(q, X, dY, dev(L1), dev(L2), s, T=T)
    say("  HIP path: bwd recomputing T (its own row ranges)")
    dXb, dL1b, dL2b = nf4.bwd(q, X, dY, dev(L1), dev(L2), s)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(DEV)
    T, Y, dX, dXb = T[idx], Y[idx], dX[idx], dXb[idx]
    del X, dY
    torch.cuda.empty_cache()

    wh = oracle.dequantize(oracle.quantize(W, 64, 256))
    Xs = synth.bf16(synth.hash_weight(rows, np.arange(h), seed) * np.float32(32))
    dYs = torch.zeros((rows.size, o), dtype=torch.bfloat16)
    dYs[torch.from_numpy(np.searchsorted(rows, hot))] = dYh
    say("  oracle on the sampled rows")
    Yr, Tr = oracle.fwd(Xs, wh, L1, L2, s)
    check_close("T rows", T, Tr)
    check_close("Y rows", Y, Yr)
    dXr = oracle.bwd(Xs, dYs, wh, L1, L2, s)[0]
    check_close("dX rows", dX, dXr)
    cold = np.setdiff1d(np.arange(rows.size), np.searchsorted(rows, hot))
    assert not dX[torch.from_numpy(cold).to(DEV)].any(), "dX on rows with dY = 0"
    _, dL1r, dL2r = oracle.adapter_grads(Xs, dYs, L1, L2, s)
    check_close("dL1 (all tokens)", dL1, dL1r)
    check_close("dL2 (all tokens)", dL2, dL2r)
    check_close("dX rows, T recomputed", dXb, dXr)
    check_close("dL1, T recomputed", dL1b, dL1r)
    check_close("dL2, T recomputed", dL2b, dL2r)
