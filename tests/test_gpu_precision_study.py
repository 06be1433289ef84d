"""Precision study: FP32 logits (the new path) against BF16 logits (the legacy
path) and what each does to the cross entropy, measured with the HIP kernels
against the FP64 oracle.

The pages state the effect but print no error table: the output-layer GEMM's
FP32 accumulator is kept as FP32 logits instead of being rounded to BF16
(Megatron-LM "Add mixed-precision (FP32) LM output logits", "What does this
PR do?"), and with integer operands the FP32 logits are exact (same page,
"Tests", the integer construction at 16 x K activations and 32,768 x K
weights).  This test builds that table over K = 512 ... 16384 for two input
kinds and checks the claims it rests on:

  integer operands in [-8, 8]   FP32 logits exact; BF16 logits wrong in a
                                large fraction of entries, by up to half a
                                BF16 ulp of the logit;
  x ~ N(0, 1), W ~ N(0, 0.02^2) FP32 logits within 1e-5 S of FP64 (the
                                parity bar); BF16 logits >= 100x further off
                                in median;
  cross entropy on either       loss and FP32 gradient against the oracle run
                                on the FP64 logits rounded to FP32: the BF16
                                logits' loss error is >= 10x the FP32 logits'.

Both logit kinds feed the FP32 backward in that table.  A second table
(test_precision_study_bf16_backward) sets the FP32 backward against the old
fused kernel's BF16 backward as Transformer Engine issue "[Pytorch] change
fused cross entropy backward grad to fp32 ..." describes it ("Description":
the backward ran in BF16 for BF16 input; discussion: the gradients were
stored over the BF16 input): softmax minus one-hot stored in BF16, then
scaled by the upstream gradient in BF16.  Checked claims: the FP32 backward
keeps each gradient row summing to zero; the BF16 one is within half a BF16
ulp of it elementwise, >= 100x further from the FP64 gradient, and its rows
no longer sum to zero (the target entry -(1 - p_y) rounds to -1).  Run with
-s to see the tables."""
import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import dev_bf16, dev_f32, dev_i32, host_bits, host_f32

pytestmark = pytest.mark.gpu

KS = (512, 1024, 2048, 4096, 8192, 16384)
M, V = 16, 32768


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _ce(z32_dev, t_dev, dloss):
    loss, st = lmh.lmhead_xent_fwd(z32_dev, t_dev)
    g = lmh.lmhead_xent_bwd(z32_dev, st, t_dev, torch.full((1,), dloss, device="cuda"))
    torch.cuda.synchronize()
    return host_f32(loss).astype(np.float64), host_f32(g).astype(np.float64)


def _study(kind, K):
    if kind == "integer":
        inp = workloads.integer_gemm(M, K, V, seed=workloads.SEED)
    else:
        inp = workloads.normal_gemm(M, K, V, 0.02, seed=workloads.SEED + K)
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    l32 = lmh.lmhead_logits(x, W, out_dtype="fp32")
    l16 = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    exact, S = oracle.logits(inp.x, inp.W)
    f32 = host_f32(l32).astype(np.float64)
    b16 = oracle.bf16_bits_to_f64(host_bits(l16))
    e32, e16 = np.abs(f32 - exact), np.abs(b16 - exact)
    # cross entropy on each kind of logits (the BF16 ones widened exactly)
    t = dev_i32(inp.target)
    dl = 1.0 / M
    loss32, g32 = _ce(l32, t, dl)
    loss16, g16 = _ce(dev_f32(b16.astype(np.float32)), t, dl)
    truth_z = exact.astype(np.float32)  # FP64 logits rounded once to FP32
    ref = oracle.xent_fwd(truth_z, inp.target)
    gref = oracle.xent_bwd(truth_z, inp.target, -100, dl)
    return {
        "kind": kind, "K": K,
        "f32_max_err": float(e32.max()), "f32_med_err": float(np.median(e32)),
        "f32_max_rel_S": float((e32 / np.maximum(S, 1e-300)).max()),
        "bf16_max_err": float(e16.max()), "bf16_med_err": float(np.median(e16)),
        "bf16_frac_inexact": float((e16 > 0).mean()),
        "loss_err_f32": float(np.abs(loss32 - ref[:, 3]).max()),
        "loss_err_bf16": float(np.abs(loss16 - ref[:, 3]).max()),
        "grad_err_f32": float(np.abs(g32 - gref).max()),
        "grad_err_bf16": float(np.abs(g16 - gref).max()),
        "logit_scale": float(np.abs(exact).max()),
    }


def _print_table(rows):
    cols = ("kind", "K", "f32_max_err", "bf16_max_err", "bf16_med_err", "bf16_frac_inexact",
            "loss_err_f32", "loss_err_bf16", "grad_err_f32", "grad_err_bf16", "logit_scale")
    print("\n" + " | ".join(cols))
    for r in rows:
        print(" | ".join(f"{r[c]:.3g}" if isinstance(r[c], float) else str(r[c]) for c in cols))


def test_precision_study_integer_operands():
    rows = [_study("integer", K) for K in KS]
    _print_table(rows)
    for r in rows:
        assert r["f32_max_err"] == 0.0                      # FP32 logits exact
        assert r["bf16_frac_inexact"] > 0.3                 # most logits need > 8 bits
        # RNE to BF16 is off by at most half an ulp: 2^-8 relative at most
        assert r["bf16_max_err"] <= r["logit_scale"] * 2.0 ** -8
        assert r["loss_err_bf16"] >= 10.0 * max(r["loss_err_f32"], 1e-6)
    # the error of the rounded logits grows with the logit magnitude (with K)
    assert rows[-1]["bf16_max_err"] > rows[0]["bf16_max_err"]


def test_precision_study_normal_operands():
    rows = [_study("normal", K) for K in KS]
    _print_table(rows)
    for r in rows:
        assert r["f32_max_rel_S"] <= 1e-5                   # the FP32 parity bar
        assert r["bf16_med_err"] >= 100.0 * max(r["f32_med_err"], 1e-12)
        assert r["loss_err_f32"] <= 1e-5 * max(1.0, r["logit_scale"])
        assert r["loss_err_bf16"] >= 10.0 * max(r["loss_err_f32"], 1e-7)
        assert r["grad_err_f32"] <= 1e-6


def _old_style_grad(z32_dev, t_dev, dl):
    """The old kernel's gradient: softmax - one-hot from lmhead_xent_bwd with
    unit upstream gradient, stored in BF16 (its BF16 output), then scaled by
    the upstream gradient in BF16 arithmetic -- the exact product of two BF16
    values rounded to nearest-even BF16 by the oracle's rounding helper."""
    _, st = lmh.lmhead_xent_fwd(z32_dev, t_dev)
    g = lmh.lmhead_xent_bwd(z32_dev, st, t_dev, torch.ones(1, device="cuda"), grad_dtype="bf16")
    torch.cuda.synchronize()
    g16 = oracle.bf16_bits_to_f64(host_bits(g))
    dl16 = oracle.bf16_bits_to_f64(oracle.round_bf16(np.array([dl])))[0]
    return oracle.bf16_bits_to_f64(oracle.round_bf16(g16 * dl16))


def _grad_metrics(g, gref):
    err = np.abs(g - gref)
    rel = np.linalg.norm(g - gref, axis=1) / np.linalg.norm(gref, axis=1)
    return float(err.max()), float(np.median(rel)), float(np.abs(g.sum(axis=1)).max())


@pytest.mark.parametrize("K", (512, 4096, 16384))
def test_precision_study_bf16_backward(K):
    inp = workloads.normal_gemm(M, K, V, 0.02, seed=workloads.SEED + K)
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    l32 = lmh.lmhead_logits(x, W, out_dtype="fp32")
    l16 = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    exact, _ = oracle.logits(inp.x, inp.W)
    t = dev_i32(inp.target)
    dl = 1.0 / M
    gref = oracle.xent_bwd(exact.astype(np.float32), inp.target, -100, dl)
    _, g_new = _ce(l32, t, dl)                                   # FP32 logits, FP32 backward
    g_old_bwd = _old_style_grad(l32, t, dl)                       # FP32 logits, BF16 backward
    b16 = oracle.bf16_bits_to_f64(host_bits(l16)).astype(np.float32)
    g_old = _old_style_grad(dev_f32(b16), t, dl)                  # BF16 logits, BF16 backward
    rows = {"fp32 logits + fp32 bwd": _grad_metrics(g_new, gref),
            "fp32 logits + bf16 bwd": _grad_metrics(g_old_bwd, gref),
            "bf16 logits + bf16 bwd": _grad_metrics(g_old, gref)}
    print(f"\nK={K}: path | max |err| | median row rel L2 err | max |row sum|  (dloss = {dl})")
    for k, (mx, rel, rs) in rows.items():
        print(f"  {k} | {mx:.3g} | {rel:.3g} | {rs:.3g}")
    new, old = rows["fp32 logits + fp32 bwd"], rows["fp32 logits + bf16 bwd"]
    assert new[0] <= 1e-6                                        # the FP32 gradient bar
    assert new[2] <= 1e-5 * dl                                   # rows sum to zero
    # BF16 storage of softmax - one-hot: at most half an ulp, 2^-8 relative
    # (8-bit significand); dl is a power of two, so the BF16 scaling adds no
    # rounding
    assert np.all(np.abs(g_old_bwd - g_new) <= 2.0 ** -8 * np.abs(g_new) * (1 + 1e-6) + 1e-30)
    assert old[1] >= 100.0 * max(new[1], 1e-12)
    assert old[2] >= 100.0 * max(new[2], 1e-15)
