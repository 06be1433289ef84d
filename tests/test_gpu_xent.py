"""GPU parity of the fused cross-entropy (forward stats, mean, backward)
against the FP64 oracle, through the C ABI (via the thin binding).

Bars: m and X_y bit-exact (selections); d and loss within 1e-5 relative
(loss with an absolute floor below |loss| = 1); FP32 dlogits within 1e-6
absolute; BF16 dlogits bit-identical to round-to-nearest-even of the FP32
dlogits of the same kernel; in-place bit-identical to out-of-place; two runs
bit-identical.  The n_rows x 4 record and the FP32 backward follow
Transformer Engine "[Pytorch] change fused cross entropy backward grad to
fp32 and reduce one read/..." (discussion; sections "Description",
"Changes")."""
import math

import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import (assert_loss_close, dev_bf16, dev_f32, dev_i32, host_f32, padded_out,
                      padding_untouched)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _say(*a):
    print(*a, flush=True)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _check_stats(st_gpu, st_ref, what=""):
    """m, X bit-exact; d within 1e-5 rel; loss within 1e-5 rel (floor 1)."""
    assert np.array_equal(_bits(st_gpu[:, 0]), _bits(st_ref[:, 0].astype(np.float32))), what + " m"
    assert np.array_equal(_bits(st_gpu[:, 2]), _bits(st_ref[:, 2].astype(np.float32))), what + " X"
    assert np.all(np.abs(st_gpu[:, 1] - st_ref[:, 1]) <= 1e-5 * st_ref[:, 1]), what + " d"
    assert_loss_close(st_gpu[:, 3], st_ref[:, 3], 1e-5, what + " loss")


def _check_grad(g_gpu, g_ref, tol=1e-6, what="dlogits"):
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: max err {err[i]} at {i} gpu={g_gpu[i]} ref={g_ref[i]}")


def _run_chain(z_dev, t_dev, ignore, grad_dtype="fp32"):
    loss, st = lmh.lmhead_xent_fwd(z_dev, t_dev, ignore)
    mean, inv = lmh.lmhead_xent_mean(loss, t_dev, ignore)
    g = lmh.lmhead_xent_bwd(z_dev, st, t_dev, inv, ignore, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return loss, st, mean, inv, g


# ------------------------------------------------------------ tiny exact

def test_tiny_exact_chain():
    """x [16 x 512] . W [1024 x 512]^T integers -> FP32 logits (bit-exact) ->
    CE fwd -> mean (dloss = 1/16) -> FP32 bwd; the oracle runs its own chain."""
    inp = workloads.tiny_exact()
    _say("tiny_exact chain")
    logits = lmh.lmhead_logits(dev_bf16(inp.x), dev_bf16(inp.W), out_dtype="fp32")
    t = dev_i32(inp.target)
    loss, st, mean, inv, g = _run_chain(logits, t, -100)
    L, _ = oracle.logits(inp.x, inp.W)
    z = L.astype(np.float32)                      # exact: integer logits < 2^24
    assert np.array_equal(_bits(host_f32(logits)), _bits(z))
    st_ref = oracle.xent_fwd(z, inp.target, -100)
    _check_stats(host_f32(st), st_ref, "tiny")
    assert np.array_equal(_bits(host_f32(loss)), _bits(host_f32(st)[:, 3]))
    m_ref, inv_ref, nv = oracle.xent_mean(st_ref[:, 3], inp.target, -100)
    assert nv == 16 and host_f32(inv)[0] == np.float32(1.0 / 16)
    assert_loss_close(host_f32(mean), [m_ref], 1e-5, "mean")
    g_ref = oracle.xent_bwd(z, inp.target, -100, inv_ref)
    _check_grad(host_f32(g), g_ref)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("V", [1024, 32768, 131072])
@pytest.mark.parametrize("c", [0.0, 7.25])
def test_uniform_logits_closed_form(V, c):
    """All logits equal: m = c, d = V exactly, loss = ln V; with dloss = 1/16
    the gradient is exactly dloss/V off target and dloss/V - dloss on it."""
    n = 4
    _say(f"uniform V={V} c={c}")
    z = torch.full((n, V), c, dtype=torch.float32, device="cuda")
    tgt = np.array([0, V - 1, 3, V // 2], dtype=np.int32)
    t = dev_i32(tgt)
    loss, st = lmh.lmhead_xent_fwd(z, t)
    dl = torch.full((1,), 1.0 / 16, device="cuda")
    g = lmh.lmhead_xent_bwd(z, st, t, dl)
    torch.cuda.synchronize()
    s = host_f32(st)
    assert np.all(s[:, 0] == np.float32(c)) and np.all(s[:, 2] == np.float32(c))
    assert np.all(s[:, 1] == np.float32(V))
    assert np.allclose(s[:, 3], math.log(V), rtol=1e-6, atol=0)
    gh = host_f32(g)
    for i, y in enumerate(tgt):
        expect = np.full(V, np.float32(1.0 / 16 / V))
        expect[y] = np.float32(1.0 / 16 / V - 1.0 / 16)
        assert np.array_equal(_bits(gh[i]), _bits(expect))


def test_vocab_one_and_two():
    """V = 1: loss 0, gradient 0.  V = 2: loss = log1p(exp(z_o - z_y)) and
    grad_y = -dloss * sigmoid(z_o - z_y) = -grad_o (closed forms)."""
    z1 = dev_f32(np.array([[3.5], [-2.0], [0.0]], np.float32), ld=4)
    t1 = dev_i32(np.array([0, 0, -100]))
    loss, st = lmh.lmhead_xent_fwd(z1, t1)
    g = lmh.lmhead_xent_bwd(z1, st, t1, torch.full((1,), 0.5, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(host_f32(loss) == 0) and np.all(host_f32(g) == 0)
    zz = np.array([[1.25, -0.5], [4.0, 4.5], [-3.0, 9.0]], np.float32)
    tt = np.array([0, 1, 0], np.int32)
    z2 = dev_f32(zz, ld=4)
    loss, st = lmh.lmhead_xent_fwd(z2, dev_i32(tt))
    g = lmh.lmhead_xent_bwd(z2, st, dev_i32(tt), torch.full((1,), 0.25, device="cuda"))
    torch.cuda.synchronize()
    lh, gh = host_f32(loss), host_f32(g)
    for i, y in enumerate(tt):
        o = 1 - y
        delta = float(zz[i, o]) - float(zz[i, y])
        assert math.isclose(lh[i], math.log1p(math.exp(delta)), rel_tol=1e-5, abs_tol=1e-6)
        sig = 1.0 / (1.0 + math.exp(-delta))
        assert abs(gh[i, y] + 0.25 * sig) <= 1e-6 and abs(gh[i, o] - 0.25 * sig) <= 1e-6


# ------------------------------------------------------------ edge shapes

@pytest.mark.parametrize("n,V", [(1, 1), (3, 2), (5, 3), (17, 5), (4, 63), (9, 64), (33, 65),
                                 (2, 1023), (600, 257), (700, 4097), (3, 40000)])
@pytest.mark.parametrize("dloss_mode", ["scalar", "per_row"])
def test_edge_shapes_random(n, V, dloss_mode):
    """Ragged V (tails of 1-3 columns, one partial block), both launch
    shapes (n < 512 and n >= 512), padded ld with untouched padding, ignored
    rows, a custom ignore value, scalar and per-row dloss."""
    rng = np.random.default_rng(n * 7919 + V)
    inp = workloads.xent_logits(n, V, sigma=2.0, spike_frac=0.1, spike=30.0, ignore_frac=0.2,
                                seed=n * 31 + V)
    ignore = -100 if V % 2 else 7777
    tgt = inp.target.copy()
    tgt[tgt == -100] = ignore
    _say(f"edge n={n} V={V} {dloss_mode} ignore={ignore}")
    ld = (V + 3) // 4 * 4 + 4
    z = dev_f32(inp.logits, ld)
    t = dev_i32(tgt)
    loss, st = lmh.lmhead_xent_fwd(z, t, ignore)
    if dloss_mode == "scalar":
        dl_host = np.float32(0.375)
        dl = torch.full((1,), float(dl_host), device="cuda")
        dl_ref = float(dl_host)
    else:
        dl_host = rng.uniform(-1, 1, n).astype(np.float32)
        dl = torch.from_numpy(dl_host).cuda()
        dl_ref = dl_host.astype(np.float64)
    g = padded_out(n, V, ld + 4, torch.float32)
    lmh.lmhead_xent_bwd(z, st, t, dl, ignore, dlogits=g)
    gb = padded_out(n, V, (V + 7) // 8 * 8 + 8, torch.bfloat16)
    lmh.lmhead_xent_bwd(z, st, t, dl, ignore, dlogits=gb, grad_dtype="bf16")
    torch.cuda.synchronize()
    st_ref = oracle.xent_fwd(inp.logits, tgt, ignore)
    _check_stats(host_f32(st), st_ref, f"n={n} V={V}")
    g_ref = oracle.xent_bwd(inp.logits, tgt, ignore, dl_ref)
    _check_grad(host_f32(g), g_ref)
    assert torch.equal(gb.view(torch.int16), g.to(torch.bfloat16).view(torch.int16))
    assert padding_untouched(g) and padding_untouched(gb)
    # gradient rows sum to zero
    rs = np.abs(host_f32(g).astype(np.float64).sum(axis=1))
    scale = np.abs(np.broadcast_to(dl_ref, (n,)))
    assert np.all(rs <= 1e-5 * scale + 1e-7)


@pytest.mark.parametrize("V", [9 * 1024 + 3, 32768, 40001, 65536])
def test_target_lane_every_residue(V):
    """The one-hot term lands on the target column whatever its position in
    its 16-byte group (target mod 4 = 0..3), in the first, middle and last
    block of a row and in the ragged tail, for the backward and for the
    one-read kernel's forms (8 and 16 float4 per thread, whole rows and ragged
    ones).  With dloss > 0 the target column is the only negative entry of its
    gradient row (softmax minus one-hot, scaled), so its position is checked
    exactly, then every value against the oracle."""
    mid = (V // 2) & ~3
    cols = [0, 1, 2, 3, 1020, 1021, 1022, 1023, 4100, 4101, 4102, 4103,
            mid, mid + 1, mid + 2, mid + 3, V - 7, V - 6, V - 5, V - 4, V - 3, V - 2, V - 1]
    n = len(cols) * 2
    tgt = np.array(cols + cols, dtype=np.int32)
    rng = np.random.default_rng(4242 + V)
    logits = rng.normal(0.0, 1.5, (n, V)).astype(np.float32)
    dl_host = rng.uniform(0.25, 2.0, n).astype(np.float32)
    _say(f"target lanes n={n} V={V}")
    z, t = dev_f32(logits, (V + 3) // 4 * 4), dev_i32(tgt)
    dl = torch.from_numpy(dl_host).cuda()
    _, st = lmh.lmhead_xent_fwd(z, t)
    g = lmh.lmhead_xent_bwd(z, st, t, dl)
    gb = lmh.lmhead_xent_bwd(z, st, t, dl, grad_dtype="bf16")
    _, _, gf = lmh.lmhead_xent_fused(z, t, dl)                       # one-read kernel
    _, _, gfb = lmh.lmhead_xent_fused(z, t, dl, grad_dtype="bf16")
    torch.cuda.synchronize()
    g_ref = oracle.xent_bwd(logits, tgt, -100, dl_host.astype(np.float64))
    for name, gg, gg16 in (("bwd", g, gb), ("fused", gf, gfb)):
        gh = host_f32(gg)
        neg = [np.flatnonzero(gh[r] < 0).tolist() for r in range(n)]
        assert neg == [[int(y)] for y in tgt], name
        _check_grad(gh, g_ref, what=name)
        assert torch.equal(gg16.view(torch.int16), gg.to(torch.bfloat16).view(torch.int16)), name


def test_all_rows_ignored_and_bad_target():
    V = 100
    z = dev_f32(np.random.default_rng(1).normal(0, 1, (6, V)).astype(np.float32))
    t = dev_i32(np.full(6, -100))
    loss, st = lmh.lmhead_xent_fwd(z, t)
    mean, inv = lmh.lmhead_xent_mean(loss, t)
    g = lmh.lmhead_xent_bwd(z, st, t, inv)
    torch.cuda.synchronize()
    assert host_f32(mean)[0] == 0 and host_f32(inv)[0] == 0
    assert np.all(host_f32(g) == 0) and np.all(host_f32(loss) == 0)
    # a target outside [0, V) that is not ignore_index yields a NaN row only
    tb = dev_i32(np.array([1, V, 2, -5, 3, 4]))
    loss, st = lmh.lmhead_xent_fwd(z, tb)
    g = lmh.lmhead_xent_bwd(z, st, tb, torch.full((1,), 1.0, device="cuda"))
    torch.cuda.synchronize()
    lh, gh = host_f32(loss), host_f32(g)
    assert np.isnan(lh[[1, 3]]).all() and np.isfinite(lh[[0, 2, 4, 5]]).all()
    assert np.isnan(gh[[1, 3]]).all() and np.isfinite(gh[[0, 2, 4, 5]]).all()


def test_empty_rows_noop():
    z = torch.empty((0, 16), device="cuda")
    t = torch.empty((0,), dtype=torch.int32, device="cuda")
    loss, st = lmh.lmhead_xent_fwd(z, t)
    mean, inv = lmh.lmhead_xent_mean(loss, t)
    torch.cuda.synchronize()
    assert host_f32(mean)[0] == 0 and host_f32(inv)[0] == 0


# ------------------------------------------------- benchmark-shaped rows

def test_xent_1024x32768_bf16_grads_and_determinism():
    """n=1024, V=32768 (the CE launch shape of the M=1024 step), BF16 grads:
    stats and FP32 grads on sampled rows vs the oracle; BF16 == RNE(FP32);
    two runs bit-identical."""
    inp = workloads.xent_logits(1024, 32768, sigma=1.8, spike_frac=0.0, ignore_frac=0.0,
                                seed=workloads.SEED + 5)
    _say("xent 1024x32768")
    z, t = dev_f32(inp.logits), dev_i32(inp.target)
    loss, st, mean, inv, gb = _run_chain(z, t, -100, "bf16")
    g = lmh.lmhead_xent_bwd(z, st, t, inv)
    loss2, st2, mean2, inv2, gb2 = _run_chain(z, t, -100, "bf16")
    assert torch.equal(st.view(torch.int32), st2.view(torch.int32))
    assert torch.equal(gb.view(torch.int16), gb2.view(torch.int16))
    assert torch.equal(mean.view(torch.int32), mean2.view(torch.int32))
    assert torch.equal(gb.view(torch.int16), g.to(torch.bfloat16).view(torch.int16))
    rows = np.array([0, 1, 255, 256, 511, 777, 1023])
    st_ref = oracle.xent_fwd(inp.logits, inp.target, -100, rows=rows)
    _check_stats(host_f32(st)[rows], st_ref)
    ref_all = oracle.xent_fwd(inp.logits, inp.target, -100)
    m_ref, inv_ref, _ = oracle.xent_mean(ref_all[:, 3], inp.target, -100)
    assert_loss_close(host_f32(mean), [m_ref], 1e-5, "mean")
    g_ref = oracle.xent_bwd(inp.logits, inp.target, -100, inv_ref, rows=rows)
    _check_grad(host_f32(g)[rows], g_ref)


def test_xent_131k_spikes_inplace():
    """logits FP32 [8192 x 131072] ~ N(0, 3^2), 1% rows with a +30 spike, 2%
    ignored: no inf/NaN anywhere; spike rows' m is the spike value; sampled
    rows match the oracle; FP32 in-place == out-of-place bitwise; BF16 ==
    RNE(FP32)."""
    inp = workloads.xent_131k()
    n, V = inp.logits.shape
    _say("xent 8192x131072 spikes")
    z = dev_f32(inp.logits)
    t = dev_i32(inp.target)
    loss, st, mean, inv, g = _run_chain(z, t, -100, "fp32")
    sh = host_f32(st)
    assert np.isfinite(sh).all() and np.isfinite(host_f32(loss)).all()
    assert not torch.isnan(g).any().item() and not torch.isinf(g).any().item()
    assert np.array_equal(_bits(sh[inp.spike_rows, 0]),
                          _bits(inp.logits[inp.spike_rows, inp.spike_cols]))
    ign = inp.meta["ignored_rows"]
    rows = np.unique(np.concatenate([inp.spike_rows[:6], ign[:4], [0, 1, 4095, 4096, 8191]]))
    st_ref = oracle.xent_fwd(inp.logits, inp.target, -100, rows=rows)
    _check_stats(sh[rows], st_ref, "131k")
    # mean over every row: oracle losses for all rows (FP64, one pass each)
    ref_all = oracle.xent_fwd(inp.logits, inp.target, -100)
    m_ref, inv_ref, nv = oracle.xent_mean(ref_all[:, 3], inp.target, -100)
    assert nv == n - ign.size
    assert_loss_close(host_f32(mean), [m_ref], 1e-5, "mean")
    g_ref = oracle.xent_bwd(inp.logits, inp.target, -100, inv_ref, rows=rows)
    gh = host_f32(g[torch.from_numpy(rows).cuda()])
    _check_grad(gh, g_ref)
    rs = np.abs(gh.astype(np.float64).sum(axis=1))
    assert np.all(rs <= 1e-5 * float(host_f32(inv)[0]) + 1e-9)
    gb = lmh.lmhead_xent_bwd(z, st, t, inv, grad_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(gb.view(torch.int16), g.to(torch.bfloat16).view(torch.int16))
    del gb
    del g
    # split-vocabulary forward (32 blocks of 4096 columns) at the same size:
    # m and X_y equal the one-pass forward bitwise, d within 1e-5 relative,
    # and the sampled rows match the oracle
    part = lmh.lmhead_xent_partial(z, t, block_cols=4096)
    loss_s, st_s = lmh.lmhead_xent_merge(part, t, V)
    torch.cuda.synchronize()
    ss = host_f32(st_s)
    assert np.array_equal(_bits(ss[:, 0]), _bits(sh[:, 0]))
    assert np.array_equal(_bits(ss[:, 2]), _bits(sh[:, 2]))
    assert np.all(np.abs(ss[:, 1] - sh[:, 1]) <= 1e-5 * sh[:, 1])
    _check_stats(ss[rows], st_ref, "131k split")
    del part, loss_s, st_s
    # 64-column blocks: 2048 x 8192 = 2^24 workgroups, more than one launch
    # may hold (2^32 work-items), so the library splits the call into row
    # ranges; the merged statistics are those of the one-pass forward
    part = lmh.lmhead_xent_partial(z, t, block_cols=64)
    loss_s, st_s = lmh.lmhead_xent_merge(part, t, V)
    torch.cuda.synchronize()
    ss = host_f32(st_s)
    assert np.array_equal(_bits(ss[:, 0]), _bits(sh[:, 0]))
    assert np.array_equal(_bits(ss[:, 2]), _bits(sh[:, 2]))
    assert np.all(np.abs(ss[:, 1] - sh[:, 1]) <= 1e-5 * sh[:, 1])
    del part, loss_s, st_s
    # in place over the logits (the copy keeps z for nothing else)
    g = lmh.lmhead_xent_bwd(z, st, t, inv)
    zc = z.clone()
    lmh.lmhead_xent_bwd(zc, st, t, inv, in_place=True)
    torch.cuda.synchronize()
    assert torch.equal(zc.view(torch.int32), g.view(torch.int32))
    del zc
    # The same backward with unit upstream gradient: its largest entries are
    # near 1 (p_y - 1), so the 1e-6 absolute bar is a tight relative check
    # (with dloss = 1/8028 above it allowed ~1 % of the largest gradient).
    one = torch.ones((1,), dtype=torch.float32, device="cuda")
    g1 = lmh.lmhead_xent_bwd(z, st, t, one, dlogits=g)
    torch.cuda.synchronize()
    g1_ref = oracle.xent_bwd(inp.logits, inp.target, -100, 1.0, rows=rows)
    gh1 = host_f32(g1[torch.from_numpy(rows).cuda()])
    assert np.abs(g1_ref).max() > 0.5
    _check_grad(gh1, g1_ref, 1e-6, "dlogits, dloss = 1")


# ---------------------------------------------------- masked (-inf) logits

def _masked_logits(n, V, seed):
    """Rows with -inf (masked) columns: leading 4096 columns masked, all but
    the 3 tail columns masked, trailing columns masked, none masked."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 3.0, (n, V)).astype(np.float32)
    t = np.empty(n, dtype=np.int32)
    for i in range(n):
        kind = i % 4
        if kind == 0:
            z[i, :4096] = -np.inf
            t[i] = rng.integers(4096, V)
        elif kind == 1:
            z[i, :V - 3] = -np.inf
            t[i] = V - 1 - (i % 3)
        elif kind == 2:
            z[i, 5000:] = -np.inf
            t[i] = rng.integers(0, 5000)
        else:
            t[i] = rng.integers(0, V)
    t[5::7] = -100
    return z, t


@pytest.mark.parametrize("n", [9, 520])
def test_masked_columns_forward_split_fused_backward(n):
    """Logits of -inf contribute nothing (exp(-inf) = 0): whole 4-value groups,
    whole column blocks and rows masked up to their ragged tail.  The one-pass
    forward (1024- and 256-thread forms), the split forward in 64- and
    4096-column blocks (masked blocks report the empty pair m = -inf, d = 0),
    the fused single-read kernel and the backward all match the oracle, with
    exact zeros at the masked columns."""
    V = 4096 + 3000 + 3
    z_h, t_h = _masked_logits(n, V, seed=n)
    _say(f"masked logits n={n} V={V}")
    z, t = dev_f32(z_h, V + 1), dev_i32(t_h)        # rows padded to a multiple of 4
    loss, st = lmh.lmhead_xent_fwd(z, t)
    dl = torch.full((1,), 0.5, device="cuda")
    g = lmh.lmhead_xent_bwd(z, st, t, dl)
    lf, sf, gf = lmh.lmhead_xent_fused(z, t, dl)
    parts = {bc: lmh.lmhead_xent_partial(z, t, block_cols=bc) for bc in (64, 4096)}
    merged = {bc: lmh.lmhead_xent_merge(p, t, V)[1] for bc, p in parts.items()}
    torch.cuda.synchronize()
    ref = oracle.xent_fwd(z_h, t_h, -100)
    assert np.isfinite(ref).all()
    _check_stats(host_f32(st), ref, "fwd")
    _check_stats(host_f32(sf), ref, "fused")
    for bc in parts:
        _check_part(host_f32(parts[bc]), oracle.xent_partial(z_h, t_h, block_cols=bc),
                    f"part {bc}")
        _check_stats(host_f32(merged[bc]), ref, f"merge {bc}")
    g_ref = oracle.xent_bwd(z_h, t_h, -100, 0.5)
    _check_grad(host_f32(g), g_ref, 1e-6, "bwd")
    _check_grad(host_f32(gf), g_ref, 1e-6, "fused")
    masked = np.isneginf(z_h)
    assert np.all(host_f32(g)[masked] == 0.0) and np.all(host_f32(gf)[masked] == 0.0)


def test_fully_masked_row():
    """A row of -inf logits has no softmax: m = -inf, d = 0 and a NaN loss, as
    in the oracle; an ignored such row has loss 0; other rows are unaffected."""
    z_h = np.random.default_rng(3).normal(0, 1, (3, 40)).astype(np.float32)
    z_h[0] = -np.inf
    z_h[1] = -np.inf
    t_h = np.array([7, -100, 7], dtype=np.int32)
    loss, st = lmh.lmhead_xent_fwd(dev_f32(z_h), dev_i32(t_h))
    _, sf, gf = lmh.lmhead_xent_fused(dev_f32(z_h), dev_i32(t_h), torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.xent_fwd(z_h, t_h, -100)
    for name, sh in (("fwd", host_f32(st)), ("fused", host_f32(sf))):
        assert np.all(sh[:2, 0] == -np.inf) and np.all(sh[:2, 1] == 0.0), name
        assert np.isnan(sh[0, 3]) and np.isnan(ref[0, 3]), name
        assert sh[1, 3] == 0.0 and ref[1, 3] == 0.0, name
        _check_stats(sh[2:], ref[2:], name + " unmasked row")
    gh = host_f32(gf)
    assert np.all(gh[1] == 0.0)                      # ignored: zero gradient
    _check_grad(gh[2:], oracle.xent_bwd(z_h[2:], t_h[2:], -100, 1.0), what="fused unmasked row")


def test_bf16_grads_of_subnormal_size_round_like_torch():
    """Gradients far below the row maximum (exp(z - m) down to FP32's
    subnormal range and to zero): the BF16 gradients of the backward and the
    fused kernel equal torch's nearest-even rounding of the same kernels'
    FP32 gradients bit for bit, subnormals included."""
    V = 4096 + 8
    rng = np.random.default_rng(777)
    z_h = rng.uniform(-110.0, 0.0, (6, V)).astype(np.float32)   # e = exp(z - m) from 1 down to 0
    z_h[:, 5] = 0.0
    t_h = np.array([5, 17, V - 1, 0, 4096, 3], dtype=np.int32)
    z, t = dev_f32(z_h), dev_i32(t_h)
    dl = torch.full((1,), 1.0, device="cuda")
    _, st = lmh.lmhead_xent_fwd(z, t)
    out = {}
    out["bwd"] = (lmh.lmhead_xent_bwd(z, st, t, dl), lmh.lmhead_xent_bwd(z, st, t, dl, grad_dtype="bf16"))
    out["fused"] = (lmh.lmhead_xent_fused(z, t, dl)[2],
                    lmh.lmhead_xent_fused(z, t, dl, grad_dtype="bf16")[2])
    torch.cuda.synchronize()
    for name, (g, gb) in out.items():
        gh = host_f32(g)
        sub = (gh != 0) & (np.abs(gh) < np.finfo(np.float32).tiny)
        assert sub.sum() > 100, name                     # the case is exercised
        assert torch.equal(gb.view(torch.int16), g.to(torch.bfloat16).view(torch.int16)), name


# ------------------------------------ calls longer than one launch can hold

def test_many_rows_split_into_several_launches():
    """2^25 + 3 rows of 4 columns: the forward (256 work-items per row), the
    backward (128 per row), the fused kernel (1024 per row), the split forward
    and the merge all need more than 2^31 work-items, so the library runs each
    as several launches over row ranges.  Rows on both sides of every range
    boundary, and others, match the oracle; nothing is left unwritten."""
    n, V = (1 << 25) + 3, 4
    rng = np.random.default_rng(workloads.SEED + 25)
    z_h = rng.standard_normal((n, V), dtype=np.float32) * np.float32(3.0)
    t_h = rng.integers(0, V, n).astype(np.int32)
    t_h[rng.choice(n, n // 50, replace=False)] = -100
    _say(f"many rows n={n} V={V}")
    z, t = dev_f32(z_h), dev_i32(t_h)
    dl = torch.full((1,), 0.25, device="cuda")
    loss, st = lmh.lmhead_xent_fwd(z, t)
    g = lmh.lmhead_xent_bwd(z, st, t, dl)
    lf, sf, gf = lmh.lmhead_xent_fused(z, t, dl)
    part = lmh.lmhead_xent_partial(z, t, block_cols=4)
    lm, sm = lmh.lmhead_xent_merge(part, t, V)
    _, inv = lmh.lmhead_xent_mean(None, t)
    torch.cuda.synchronize()
    for name, a in (("fwd", st), ("fused", sf), ("merge", sm)):
        assert torch.isfinite(a[:, :2]).all().item(), name
        assert torch.isfinite(a[:, 3]).all().item(), name
    assert torch.isfinite(g).all().item() and torch.isfinite(gf).all().item()
    edges = np.arange(1, 17) << 21
    rows = np.unique(np.concatenate([(edges[:, None] + np.arange(-2, 2)[None, :]).ravel(),
                                     rng.integers(0, n, 300), [0, n - 1]]))
    rows = rows[(rows >= 0) & (rows < n)]
    rt = torch.from_numpy(rows).cuda()
    ref = oracle.xent_fwd(z_h, t_h, -100, rows=rows)
    for name, a in (("fwd", st), ("fused", sf), ("merge", sm)):
        _check_stats(host_f32(a[rt]), ref, name)
    g_ref = oracle.xent_bwd(z_h, t_h, -100, 0.25, rows=rows)
    _check_grad(host_f32(g[rt]), g_ref, 1e-6, "bwd")
    _check_grad(host_f32(gf[rt]), g_ref, 1e-6, "fused")
    nv = int((t_h != -100).sum())
    assert float(host_f32(inv)[0]) == np.float32(1.0 / nv)


# ------------------------------------------------ split-vocabulary forward

def _check_part(p_gpu, p_ref, what=""):
    """m_b, X_b bit-exact; own_b exact; d_b within 1e-5 relative."""
    p_gpu = p_gpu.reshape(p_ref.shape)
    assert np.array_equal(_bits(p_gpu[..., 0]), _bits(p_ref[..., 0].astype(np.float32))), what + " m"
    assert np.array_equal(_bits(p_gpu[..., 2]), _bits(p_ref[..., 2].astype(np.float32))), what + " X"
    assert np.array_equal(p_gpu[..., 3], p_ref[..., 3].astype(np.float32)), what + " own"
    assert np.all(np.abs(p_gpu[..., 1] - p_ref[..., 1]) <= 1e-5 * p_ref[..., 1]), what + " d"


@pytest.mark.parametrize("n,V,bc", [(1, 1, 4), (3, 7, 4), (37, 10000, 1000), (37, 10000, 4096),
                                    (5, 4099, 4096), (128, 32768, 4096), (600, 3000, 512),
                                    (2, 64, 8192)])
def test_split_partial_and_merge(n, V, bc):
    """Per-block records against the oracle's (ragged last block, one-block
    rows, tails of 1-3 columns, a block wider than the row, padded ld); the
    merge against the oracle's full-row statistics and the one-pass forward;
    the backward on the merged statistics against the oracle."""
    inp = workloads.xent_logits(n, V, sigma=2.5, spike_frac=0.05, spike=30.0, ignore_frac=0.1,
                                seed=n * 13 + V + bc)
    _say(f"split n={n} V={V} bc={bc}")
    ld = (V + 3) // 4 * 4 + 8
    z, t = dev_f32(inp.logits, ld), dev_i32(inp.target)
    part = lmh.lmhead_xent_partial(z, t, block_cols=bc)
    loss, st = lmh.lmhead_xent_merge(part, t, V)
    _, st1 = lmh.lmhead_xent_fwd(z, t)
    dl = torch.full((1,), 0.125, device="cuda")
    g = lmh.lmhead_xent_bwd(z, st, t, dl)
    torch.cuda.synchronize()
    _check_part(host_f32(part), oracle.xent_partial(inp.logits, inp.target, block_cols=bc), "part")
    st_ref = oracle.xent_fwd(inp.logits, inp.target, -100)
    _check_stats(host_f32(st), st_ref, "merge")
    assert np.array_equal(_bits(host_f32(loss)), _bits(host_f32(st)[:, 3]))
    one = host_f32(st1)
    assert np.array_equal(_bits(host_f32(st)[:, 0]), _bits(one[:, 0]))
    assert np.array_equal(_bits(host_f32(st)[:, 2]), _bits(one[:, 2]))
    _check_grad(host_f32(g), oracle.xent_bwd(inp.logits, inp.target, -100, 0.125))


def test_split_two_shards_with_offset_and_stride():
    """Two vocabulary shards (global columns [0, 6144) and [6144, 10000)),
    each reduced with its own col0 into one strided parts buffer, merge to
    the oracle's full-row statistics; two runs are bit-identical."""
    n, V, a = 45, 10000, 6144
    inp = workloads.xent_logits(n, V, sigma=2.0, spike_frac=0.1, ignore_frac=0.1, seed=77)
    _say("split two shards")
    z0 = dev_f32(np.ascontiguousarray(inp.logits[:, :a]))
    z1 = dev_f32(np.ascontiguousarray(inp.logits[:, a:]))
    t = dev_i32(inp.target)
    nb0, nb1 = a // 2048, -(-(V - a) // 2048)
    buf = torch.full((nb0 + nb1, n + 3, 4), float("nan"), device="cuda")  # stride 4 (n + 3)
    parts = buf[:, :n, :]
    lmh.lmhead_xent_partial(z0, t, col0=0, block_cols=2048, part=parts[:nb0])
    lmh.lmhead_xent_partial(z1, t, col0=a, block_cols=2048, part=parts[nb0:])
    loss, st = lmh.lmhead_xent_merge(parts, t, V)
    loss2, st2 = lmh.lmhead_xent_merge(parts, t, V)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:, n:, :]).all().item()       # padding rows never written
    assert torch.equal(st.view(torch.int32), st2.view(torch.int32))
    ph = host_f32(parts)
    assert np.array_equal(ph[:, :, 3].sum(axis=0), np.where(inp.target == -100, 0, 1).astype(np.float32))
    _check_stats(host_f32(st), oracle.xent_fwd(inp.logits, inp.target, -100), "shards")


def test_split_merge_nan_rows():
    """A target outside [0, vocab) or one that no supplied part owns gives
    NaN X_y and loss (m, d finite); ignored rows give 0."""
    V = 300
    rng = np.random.default_rng(12)
    zh = rng.normal(0, 1, (4, V)).astype(np.float32)
    tgt = np.array([-100, 310, 20, 250], dtype=np.int32)
    z, t = dev_f32(np.ascontiguousarray(zh[:, :200])), dev_i32(tgt)   # columns 200.. not supplied
    part = lmh.lmhead_xent_partial(z, t, block_cols=64)
    loss, st = lmh.lmhead_xent_merge(part, t, V)
    torch.cuda.synchronize()
    sh, lh = host_f32(st), host_f32(loss)
    assert sh[0, 2] == 0 and lh[0] == 0
    assert np.isnan(lh[1]) and np.isnan(sh[1, 2])
    assert np.isfinite(lh[2]) and sh[2, 2] == zh[2, 20]
    assert np.isnan(lh[3]) and np.isnan(sh[3, 2])
    assert np.isfinite(sh[:, :2]).all()
    ref = oracle.xent_merge(oracle.xent_partial(zh[:, :200], tgt, block_cols=64), tgt, V)
    assert np.array_equal(np.isnan(ref[:, 3]), np.isnan(lh))


# ------------------------------------------- single-read fused forward+backward

@pytest.mark.parametrize("n,V,mode", [(1, 1, "scalar"), (3, 5, "per_row"), (33, 65, "scalar"),
                                      (600, 4097, "per_row"), (128, 32768, "scalar"),
                                      (5, 40001, "per_row"), (7, 65536, "scalar"),
                                      (3, 65537, "per_row"),
                                      # one element either side of the whole-row forms
                                      (4, 32767, "scalar"), (4, 32769, "per_row"),
                                      (4, 65535, "scalar"),
                                      # several rounds of workgroups per CU
                                      (600, 32768, "per_row"), (520, 16384, "scalar"),
                                      (1024, 32768, "scalar")])
def test_fused_matches_oracle(n, V, mode):
    """Stats and gradients of the one-read kernel against the oracle: 8 and 16
    float4 per thread, ragged tails, ignored rows, scalar and per-row dloss,
    rows past 65536 columns (the two-kernel path), 520 - 1024 rows of 16384
    and 32768 columns; BF16 == RNE(FP32); in place == out of place bitwise;
    agrees with fwd + bwd to rounding."""
    inp = workloads.xent_logits(n, V, sigma=2.5, spike_frac=0.1, spike=30.0, ignore_frac=0.15,
                                seed=n * 7 + V)
    _say(f"fused n={n} V={V} {mode}")
    rng = np.random.default_rng(V)
    if mode == "scalar":
        dl_host = np.float32(0.0625)
        dl = torch.full((1,), float(dl_host), device="cuda")
        dl_ref = float(dl_host)
    else:
        dl_host = rng.uniform(0.1, 1.0, n).astype(np.float32)
        dl = torch.from_numpy(dl_host).cuda()
        dl_ref = dl_host.astype(np.float64)
    ld = (V + 3) // 4 * 4
    z, t = dev_f32(inp.logits, ld), dev_i32(inp.target)
    g = padded_out(n, V, ld + 8, torch.float32)
    loss, st, _ = lmh.lmhead_xent_fused(z, t, dl, dlogits=g)
    _, st16, g16 = lmh.lmhead_xent_fused(z, t, dl, grad_dtype="bf16")
    _, st2 = lmh.lmhead_xent_fwd(z, t)
    g2 = lmh.lmhead_xent_bwd(z, st2, t, dl)
    zc = dev_f32(inp.logits, ld)  # a second padded copy for the in-place run
    _, _, gi = lmh.lmhead_xent_fused(zc, t, dl, in_place=True)
    torch.cuda.synchronize()
    st_ref = oracle.xent_fwd(inp.logits, inp.target, -100)
    _check_stats(host_f32(st), st_ref, "fused")
    assert np.array_equal(_bits(host_f32(loss)), _bits(host_f32(st)[:, 3]))
    assert torch.equal(st.view(torch.int32), st16.view(torch.int32))
    g_ref = oracle.xent_bwd(inp.logits, inp.target, -100, dl_ref)
    _check_grad(host_f32(g), g_ref)
    assert padding_untouched(g)
    assert torch.equal(g16.view(torch.int16), g.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(gi.view(torch.int32), g.view(torch.int32))
    assert np.array_equal(_bits(host_f32(st)[:, 0]), _bits(host_f32(st2)[:, 0]))
    _check_grad(host_f32(g), host_f32(g2).astype(np.float64), tol=1e-6, what="fused vs fwd+bwd")


def test_fused_mean_chain_with_targets_only_inverse():
    """The mean-loss chain in one logits read: 1/n_valid from the targets
    alone (no loss yet), the fused kernel with it as dloss, then the mean of
    the losses: equal to the two-read chain's mean and inverse bitwise; the
    all-ignored and bad-target rows behave as in the forward."""
    n, V = 1024, 32768
    inp = workloads.xent_logits(n, V, sigma=1.8, spike_frac=0.0, ignore_frac=0.05,
                                seed=workloads.SEED + 9)
    tgt = inp.target.copy()
    tgt[3] = V + 5                                     # bad target: NaN row only
    _say("fused mean chain")
    z, t = dev_f32(inp.logits), dev_i32(tgt)
    _, inv0 = lmh.lmhead_xent_mean(None, t)
    loss, st, gb = lmh.lmhead_xent_fused(z, t, inv0, grad_dtype="bf16")
    mean, inv = lmh.lmhead_xent_mean(loss, t)
    loss2, st2 = lmh.lmhead_xent_fwd(z, t)
    mean2, inv2 = lmh.lmhead_xent_mean(loss2, t)
    torch.cuda.synchronize()
    assert host_f32(inv0)[0] == host_f32(inv2)[0] == np.float32(1.0 / (tgt != -100).sum())
    assert host_f32(inv)[0] == host_f32(inv0)[0]
    lh = host_f32(loss)
    assert np.isnan(lh[3]) and np.isnan(host_f32(mean)[0])  # a NaN loss poisons the mean
    assert torch.isnan(gb[3].float()).all().item()
    ok = np.ones(n, bool)
    ok[3] = False
    assert torch.isfinite(gb[torch.from_numpy(ok).cuda()].float()).all().item()
    rows = np.array([0, 1, 2, 4, 500, 1023])
    st_ref = oracle.xent_fwd(inp.logits, inp.target, -100, rows=rows)
    _check_stats(host_f32(st)[rows], st_ref, "fused chain")
