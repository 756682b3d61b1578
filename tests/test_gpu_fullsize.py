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

nf4 = pytest.importorskip("quantized_lora_fine_amd")

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
