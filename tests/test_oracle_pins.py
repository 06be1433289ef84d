"""Pins for the FP64 oracle: each check comes from something other than the
oracle itself -- integer arithmetic, closed forms, brute force without the
max shift, finite differences, numpy/torch library routines, or the values the
pages print (tests/golden).  A dropped term, a wrong sign or index, or a
transposed operand anywhere in the oracle fails at least one of them."""
import math

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _ints_bf16(rng, shape, lo=-8, hi=8):
    v = rng.integers(lo, hi + 1, shape)
    return v, workloads.int_to_bf16_bits(v)


def _padded(bits, ld):
    """Place a [r, c] uint16 array in a wider [r, ld] buffer (garbage padding)."""
    r, c = bits.shape
    buf = np.full((r, ld), 0x7FC0, dtype=np.uint16)  # NaN padding must never be read
    buf[:, :c] = bits
    return buf[:, :c]


# ----------------------------------------------------------------- GEMM pins

@pytest.mark.parametrize("M,K,V", [(5, 37, 11), (1, 8, 1), (16, 64, 33), (3, 129, 7)])
def test_logits_integer_exact_vs_int64(M, K, V):
    """Pin (a): integer operands make the sum exact; compare with int64 math
    (non-square shapes catch a transposed operand, padding catches ld bugs)."""
    rng = np.random.default_rng(7 + M + K + V)
    xi, xb = _ints_bf16(rng, (M, K))
    wi, wb = _ints_bf16(rng, (V, K))
    L, S = oracle.logits(_padded(xb, K + 8), _padded(wb, K + 5))
    assert np.array_equal(L, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(S, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))
    rows = np.array([M - 1, 0], dtype=np.int64)
    Lr, _ = oracle.logits(xb, wb, rows=rows)
    assert np.array_equal(Lr, (xi[rows] @ wi.T).astype(np.float64))


def test_logits_random_vs_numpy_matmul():
    """Random BF16 operands: the plain FP64 sum agrees with numpy's FP64
    matmul (a library routine) to FP64 rounding."""
    rng = np.random.default_rng(11)
    xb = workloads.normal_bf16(rng, (9, 300), 1.0)
    wb = workloads.normal_bf16(rng, (40, 300), 0.02)
    L, S = oracle.logits(xb, wb)
    ref = oracle.bf16_bits_to_f64(xb) @ oracle.bf16_bits_to_f64(wb).T
    assert np.all(np.abs(L - ref) <= 1e-13 * S + 1e-300)
    refS = np.abs(oracle.bf16_bits_to_f64(xb)) @ np.abs(oracle.bf16_bits_to_f64(wb)).T
    assert np.allclose(S, refS, rtol=1e-13, atol=0)


def test_logits_empty_k_is_zero():
    xb = np.zeros((3, 0), np.uint16)
    wb = np.zeros((4, 0), np.uint16)
    L, S = oracle.logits(xb, wb)
    assert L.shape == (3, 4) and np.all(L == 0) and np.all(S == 0)


@pytest.mark.parametrize("M,K,V", [(6, 24, 10), (4, 8, 33)])
def test_dgrad_wgrad_integer_exact(M, K, V):
    """dX = dl . W and dW = dl^T . x against int64 matmul, including row
    subsets and padded leading dimensions."""
    rng = np.random.default_rng(100 + M)
    dli, dlb = _ints_bf16(rng, (M, V))
    wi, wb = _ints_bf16(rng, (V, K))
    xi, xb = _ints_bf16(rng, (M, K))
    dX, SX = oracle.dgrad(_padded(dlb, V + 3), _padded(wb, K + 8))
    assert np.array_equal(dX, (dli @ wi).astype(np.float64))
    assert np.array_equal(SX, (np.abs(dli) @ np.abs(wi)).astype(np.float64))
    dW, SW = oracle.wgrad(_padded(dlb, V + 1), _padded(xb, K + 16))
    assert np.array_equal(dW, (dli.T @ xi).astype(np.float64))
    assert np.array_equal(SW, (np.abs(dli).T @ np.abs(xi)).astype(np.float64))
    rows = np.array([V - 1, 2], dtype=np.int64)
    dWr, _ = oracle.wgrad(dlb, xb, rows=rows)
    assert np.array_equal(dWr, (dli.T @ xi)[rows].astype(np.float64))
    rows = np.array([M - 1], dtype=np.int64)
    dXr, _ = oracle.dgrad(dlb, wb, rows=rows)
    assert np.array_equal(dXr, (dli @ wi)[rows].astype(np.float64))


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(3)
    xb = workloads.normal_bf16(rng, (13, 200), 1.0)
    wb = workloads.normal_bf16(rng, (50, 200), 0.02)
    a, _ = oracle.logits(xb, wb, nthreads=1)
    b, _ = oracle.logits(xb, wb, nthreads=5)
    assert np.array_equal(a, b)


def test_pages_integer_construction(golden):
    """The pages' integer construction: operands in [-8, 8]; K * 8^2 < 2^24
    for every width of the sweep (example: K=512 gives 32,768)."""
    g = golden("pages_integer_exactness.txt")
    assert g["example_k"] * g["operand_max"] ** 2 == g["example_k_times_max_sq"]
    assert g["exact_bound"] == 2 ** 24
    assert tuple(g["k_widths"]) == workloads.INT_SWEEP_K
    for k in g["k_widths"]:
        assert k * max(abs(g["operand_min"]), g["operand_max"]) ** 2 < g["exact_bound"]
    assert g["seed"] == workloads.SEED
    inp = workloads.tiny_exact()
    xv = oracle.bf16_bits_to_f64(inp.x)
    assert xv.min() >= g["operand_min"] and xv.max() <= g["operand_max"]
    assert np.all(xv == np.round(xv))
    # both ends of the inclusive range occur in the draw
    assert xv.min() == g["operand_min"] and xv.max() == g["operand_max"]


def test_pages_integer_sweep_exact_worst_case(golden):
    """At every sweep width the all-(+8)/all-(-8) worst case is exact in FP32:
    the oracle's sum equals K * 64 and that integer round-trips through FP32."""
    g = golden("pages_integer_exactness.txt")
    for k in g["k_widths"]:
        x = workloads.int_to_bf16_bits(np.full((1, k), 8))
        w = workloads.int_to_bf16_bits(np.full((2, k), -8))
        L, _ = oracle.logits(x, w)
        assert L[0, 0] == -64.0 * k
        assert float(np.float32(L[0, 0])) == L[0, 0]


def test_pages_gemm_grid(golden):
    g = golden("pages_gemm_grid.txt")
    assert tuple(g["m_values"]) == workloads.GEMM_GRID_M
    assert tuple(g["k_values"]) == workloads.GEMM_GRID_K
    assert g["n_vocab"] == workloads.GEMM_GRID_V
    assert len(g["m_values"]) * len(g["k_values"]) == g["n_shapes"]


# ----------------------------------------------------------- CE forward pins

def _logsumexp_bruteforce(row):
    """log sum_j exp(z_j) with no max shift, summed exactly by math.fsum."""
    return math.log(math.fsum(math.exp(float(v)) for v in row))


@pytest.mark.parametrize("V", [1024, 32768, 131072])
@pytest.mark.parametrize("c", [0.0, 7.25])
def test_xent_uniform_logits_closed_form(V, c):
    """Pin (b): all logits equal => m = c, d = V exactly, loss = ln V."""
    z = np.full((2, V), c, dtype=np.float32)
    t = np.array([0, V - 1], dtype=np.int32)
    st = oracle.xent_fwd(z, t, -100)
    assert np.all(st[:, 0] == c)
    assert np.all(st[:, 1] == V)
    assert np.all(st[:, 2] == c)
    assert np.allclose(st[:, 3], math.log(V), rtol=1e-14, atol=0)


@pytest.mark.parametrize("V", [2, 3, 5, 8])
def test_xent_bruteforce_small_vocab(V):
    """Pin (d): brute force log-sum-exp without the max shift, every target."""
    rng = np.random.default_rng(V)
    z = rng.uniform(-6, 6, (V, V)).astype(np.float32)
    t = np.arange(V, dtype=np.int32)  # row i targets column i
    st = oracle.xent_fwd(z, t, -100)
    for i in range(V):
        lse = _logsumexp_bruteforce(z[i])
        assert math.isclose(st[i, 3], lse - float(z[i, i]), rel_tol=1e-13, abs_tol=1e-14)
        assert st[i, 0] == float(z[i].max())
        assert st[i, 2] == float(z[i, i])
        assert math.isclose(st[i, 1], math.fsum(math.exp(float(v) - float(z[i].max())) for v in z[i]),
                            rel_tol=1e-14)


def test_xent_vocab_one_and_two_closed_forms():
    z1 = np.array([[3.5], [-2.0]], dtype=np.float32)
    st = oracle.xent_fwd(z1, np.zeros(2, np.int32), -100)
    assert np.all(st[:, 3] == 0.0) and np.all(st[:, 1] == 1.0)
    g = oracle.xent_bwd(z1, np.zeros(2, np.int32), -100, 0.5)
    assert np.all(g == 0.0)
    # V = 2: loss = log1p(exp(z_o - z_y)); grad_y = -dloss * sigmoid(z_o - z_y) = -grad_o
    z2 = np.array([[1.25, -0.5], [4.0, 4.5]], dtype=np.float32)
    t2 = np.array([0, 1], dtype=np.int32)
    st = oracle.xent_fwd(z2, t2, -100)
    g = oracle.xent_bwd(z2, t2, -100, 0.25)
    for i, y in enumerate(t2):
        o = 1 - y
        delta = float(z2[i, o]) - float(z2[i, y])
        assert math.isclose(st[i, 3], math.log1p(math.exp(delta)), rel_tol=1e-14)
        sig = 1.0 / (1.0 + math.exp(-delta))
        assert math.isclose(g[i, y], -0.25 * sig, rel_tol=1e-13)
        assert math.isclose(g[i, o], 0.25 * sig, rel_tol=1e-13)


def test_xent_shift_invariance():
    rng = np.random.default_rng(5)
    z = (rng.integers(-64, 64, (4, 50)) / 8.0).astype(np.float32)
    t = rng.integers(0, 50, 4).astype(np.int32)
    a = oracle.xent_fwd(z, t, -100)
    b = oracle.xent_fwd(z + np.float32(16.0), t, -100)  # exact shift in FP32
    assert np.allclose(a[:, 1], b[:, 1], rtol=1e-14, atol=0)
    assert np.allclose(a[:, 3], b[:, 3], rtol=1e-13, atol=1e-14)
    ga = oracle.xent_bwd(z, t, -100, 1.0)
    gb = oracle.xent_bwd(z + np.float32(16.0), t, -100, 1.0)
    assert np.allclose(ga, gb, rtol=0, atol=1e-15)


def test_xent_ignore_and_out_of_range():
    z = np.arange(12, dtype=np.float32).reshape(3, 4)
    t = np.array([-100, 2, -100], dtype=np.int32)
    st = oracle.xent_fwd(z, t, -100)
    assert np.all(st[[0, 2], 2] == 0) and np.all(st[[0, 2], 3] == 0)
    assert st[0, 0] == 3.0 and st[2, 0] == 11.0          # m, d still computed
    assert math.isclose(st[0, 1], sum(math.exp(-k) for k in range(4)), rel_tol=1e-15)
    g = oracle.xent_bwd(z, t, -100, 1.0)
    assert np.all(g[[0, 2]] == 0.0)
    with pytest.raises(ValueError):
        oracle.xent_fwd(z, np.array([0, 4, 0], np.int32), -100)
    with pytest.raises(ValueError):
        oracle.xent_bwd(z, np.array([0, -1, 0], np.int32), -100, 1.0)
    # a custom ignore value is honoured and -100 is then an invalid target
    st = oracle.xent_fwd(z, np.array([7, 1, 7], np.int32), 7)
    assert np.all(st[[0, 2], 3] == 0)
    with pytest.raises(ValueError):
        oracle.xent_fwd(z, np.array([-100, 1, 0], np.int32), 7)


def test_xent_padded_rows_and_subset():
    rng = np.random.default_rng(9)
    buf = np.full((5, 24), np.nan, dtype=np.float32)  # NaN padding must never be read
    buf[:, :21] = rng.normal(0, 2, (5, 21))
    z = buf[:, :21]
    t = rng.integers(0, 21, 5).astype(np.int32)
    full = oracle.xent_fwd(z, t, -100)
    assert np.all(np.isfinite(full))
    sub = oracle.xent_fwd(z, t, -100, rows=[4, 1])
    assert np.array_equal(sub, full[[4, 1]])
    g = oracle.xent_bwd(z, t, -100, 1.0, rows=[3])
    assert np.all(np.isfinite(g))


# ---------------------------------------------------------- CE backward pins

def test_xent_bwd_finite_differences():
    """The softmax-minus-one-hot gradient equals the central difference of the
    oracle's own forward loss (FP32-exact perturbations, FP64 losses)."""
    rng = np.random.default_rng(21)
    V, n = 7, 4
    z = (rng.integers(-40, 40, (n, V)) / 16.0).astype(np.float32)
    t = rng.integers(0, V, n).astype(np.int32)
    dl = np.array([1.0, 0.5, -2.0, 0.125])
    g = oracle.xent_bwd(z, t, -100, dl)
    h = 2.0 ** -12
    for i in range(n):
        for j in range(V):
            zp = z.copy(); zp[i, j] += np.float32(h)
            zm = z.copy(); zm[i, j] -= np.float32(h)
            lp = oracle.xent_fwd(zp, t, -100, rows=[i])[0, 3]
            lm = oracle.xent_fwd(zm, t, -100, rows=[i])[0, 3]
            fd = dl[i] * (lp - lm) / (2 * h)
            assert abs(fd - g[i, j]) < 1e-7, (i, j, fd, g[i, j])


def test_xent_bwd_row_sums_zero():
    """Pin (c): every gradient row sums to zero."""
    rng = np.random.default_rng(4)
    z = rng.normal(0, 3, (6, 1000)).astype(np.float32)
    t = rng.integers(0, 1000, 6).astype(np.int32)
    g = oracle.xent_bwd(z, t, -100, 0.75)
    for row in g:
        assert abs(math.fsum(row)) < 1e-14


def test_xent_bwd_uniform_power_of_two():
    """Uniform logits, dloss = 1/16, V = 1024: g = 2^-14 off target and
    2^-14 - 2^-4 on target, exactly."""
    V = 1024
    z = np.zeros((3, V), np.float32)
    t = np.array([0, 5, 1023], np.int32)
    g = oracle.xent_bwd(z, t, -100, 1.0 / 16)
    for i, y in enumerate(t):
        assert g[i, y] == 2.0 ** -14 - 2.0 ** -4
        mask = np.ones(V, bool); mask[y] = False
        assert np.all(g[i, mask] == 2.0 ** -14)


def test_xent_bwd_per_row_vs_scalar_dloss():
    rng = np.random.default_rng(8)
    z = rng.normal(0, 1, (3, 16)).astype(np.float32)
    t = np.array([1, 2, 3], np.int32)
    g1 = oracle.xent_bwd(z, t, -100, 0.5)
    g2 = oracle.xent_bwd(z, t, -100, np.array([0.5, 0.5, 0.5]))
    assert np.array_equal(g1, g2)
    g3 = oracle.xent_bwd(z, t, -100, np.array([0.5, 1.0, 0.0]))
    assert np.array_equal(g3[0], g1[0]) and np.allclose(g3[1], 2 * g1[1]) and np.all(g3[2] == 0)


# ----------------------------------------------------------------- mean pins

# ------------------------------------------------ split-vocabulary CE pins

def _split_inputs(n, V, seed, ignore_frac=0.2):
    rng = np.random.default_rng(seed)
    z = (rng.normal(0.0, 2.0, (n, V)) + rng.choice([0.0, 25.0], (n, V), p=[0.97, 0.03]))
    z = z.astype(np.float32)
    t = rng.integers(0, V, n).astype(np.int32)
    t[rng.random(n) < ignore_frac] = -100
    return z, t


@pytest.mark.parametrize("V,bc", [(1, 4), (7, 1), (37, 4), (100, 32), (257, 64), (1000, 999),
                                  (1000, 1000), (64, 4096)])
def test_split_merge_equals_full_row(V, bc):
    """Invariant: the merge of the per-block records equals the full-row
    statistics of the (separately pinned) forward, for ragged last blocks,
    one-column blocks and a single block wider than the row."""
    z, t = _split_inputs(9, V, seed=V * 31 + bc)
    part = oracle.xent_partial(z, t, -100, col0=0, block_cols=bc)
    assert part.shape == (-(-V // bc), 9, 4)
    st = oracle.xent_merge(part, t, V, -100)
    ref = oracle.xent_fwd(z, t, -100)
    assert np.array_equal(st[:, 0], ref[:, 0])          # max of maxima is exact
    assert np.array_equal(st[:, 2], ref[:, 2])          # X_y copied, not computed
    np.testing.assert_allclose(st[:, 1], ref[:, 1], rtol=1e-13, atol=0)
    np.testing.assert_allclose(st[:, 3], ref[:, 3], rtol=1e-12, atol=1e-12)


def test_split_slices_with_column_offset():
    """Two slices of the vocabulary (global columns [0, a) and [a, V)), each
    reduced with its own col0 and targets given as global columns, merge to
    the full-row statistics; each valid target is owned by exactly one slice."""
    V, a = 300, 128
    z, t = _split_inputs(11, V, seed=5)
    p0 = oracle.xent_partial(np.ascontiguousarray(z[:, :a]), t, -100, col0=0, block_cols=64)
    p1 = oracle.xent_partial(np.ascontiguousarray(z[:, a:]), t, -100, col0=a, block_cols=48)
    part = np.concatenate([p0, p1])
    owners = part[:, :, 3].sum(axis=0)
    assert np.array_equal(owners, np.where(t == -100, 0.0, 1.0))
    st = oracle.xent_merge(part, t, V, -100)
    ref = oracle.xent_fwd(z, t, -100)
    assert np.array_equal(st[:, 0], ref[:, 0]) and np.array_equal(st[:, 2], ref[:, 2])
    np.testing.assert_allclose(st[:, 1], ref[:, 1], rtol=1e-13, atol=0)
    # merge order does not change the statistics (m exactly)
    st_rev = oracle.xent_merge(part[::-1].copy(), t, V, -100)
    assert np.array_equal(st_rev[:, 0], st[:, 0]) and np.array_equal(st_rev[:, 2], st[:, 2])
    np.testing.assert_allclose(st_rev[:, 1], st[:, 1], rtol=1e-14, atol=0)


@pytest.mark.parametrize("c", [0.0, -3.5, 11.25])
def test_split_uniform_closed_form(c):
    """All logits equal: m_b = c and d_b = the block's width exactly; the
    owning block is (y - col0) // block_cols."""
    V, bc = 1000, 96
    z = np.full((4, V), c, dtype=np.float32)
    t = np.array([0, 999, 96, -100], dtype=np.int32)
    part = oracle.xent_partial(z, t, -100, block_cols=bc)
    widths = np.minimum(bc, V - bc * np.arange(part.shape[0]))
    assert np.all(part[:, :, 0] == c)
    assert np.array_equal(part[:, :, 1], np.repeat(widths[:, None].astype(np.float64), 4, axis=1))
    own = part[:, :, 3]
    for r, y in enumerate(t):
        expect = np.zeros(part.shape[0])
        if y != -100:
            expect[y // bc] = 1.0
        assert np.array_equal(own[:, r], expect)
        assert np.all(part[:, r, 2] == (c if y != -100 else 0.0) * own[:, r])


def test_split_single_column_blocks_and_unshifted_sum():
    """One-column blocks: m_b = z_j, d_b = 1 exactly.  Wider blocks of small
    logits: d_b * exp(m_b) equals the unshifted sum of exp(z_j) (brute force
    without the max shift)."""
    rng = np.random.default_rng(3)
    z = rng.uniform(-4, 4, (3, 10)).astype(np.float32)
    t = np.array([2, 9, 0], dtype=np.int32)
    p1 = oracle.xent_partial(z, t, -100, block_cols=1)
    assert np.array_equal(p1[:, :, 0].T, z.astype(np.float64))
    assert np.all(p1[:, :, 1] == 1.0)
    p4 = oracle.xent_partial(z, t, -100, block_cols=4)
    for b in range(3):
        blk = z[:, 4 * b:4 * b + 4].astype(np.float64)
        brute = np.array([sum(math.exp(v) for v in row) for row in blk])
        np.testing.assert_allclose(p4[b, :, 1] * np.exp(p4[b, :, 0]), brute, rtol=1e-14)


def test_split_merge_bad_and_unowned_targets():
    """Ignored rows: X = loss = 0.  A target outside [0, vocab), or one that no
    supplied part owns, gives NaN X and loss while m and d stay finite."""
    V = 50
    z, _ = _split_inputs(4, V, seed=9, ignore_frac=0.0)
    t = np.array([-100, 60, 10, 45], dtype=np.int32)
    part = oracle.xent_partial(np.ascontiguousarray(z[:, :40]), t, -100, block_cols=16)
    st = oracle.xent_merge(part, t, V, -100)            # columns 40..49 not supplied
    assert st[0, 2] == 0.0 and st[0, 3] == 0.0
    assert np.isnan(st[1, 2]) and np.isnan(st[1, 3])    # 60 >= vocab
    assert np.isfinite(st[2, 3]) and st[2, 2] == np.float64(z[2, 10])
    assert np.isnan(st[3, 2]) and np.isnan(st[3, 3])    # 45 owned by no part
    assert np.all(np.isfinite(st[:, :2]))


def test_masked_columns_carry_no_probability():
    """Logits of -inf (masked columns) contribute exp(-inf) = 0: a row padded
    with -inf columns on both sides has the statistics of its finite part
    (m, X and the sequential d bitwise, since adding 0 is exact), its loss is
    the unshifted brute-force log-sum-exp over the finite part minus z_y,
    and its gradient is 0 at every masked column."""
    rng = np.random.default_rng(17)
    core = rng.normal(0, 3, (3, 40)).astype(np.float32)
    t_core = np.array([0, 17, 39], dtype=np.int32)
    a, b = 4096, 5
    z = np.full((3, a + 40 + b), -np.inf, dtype=np.float32)
    z[:, a:a + 40] = core
    t = t_core + a
    st = oracle.xent_fwd(z, t, -100)
    ref = oracle.xent_fwd(core, t_core, -100)
    assert np.array_equal(st, ref)
    for i in range(3):
        lse = _logsumexp_bruteforce(core[i])
        assert math.isclose(st[i, 3], lse - float(core[i, t_core[i]]), rel_tol=1e-13)
    g = oracle.xent_bwd(z, t, -100, 0.5)
    assert np.all(g[:, :a] == 0.0) and np.all(g[:, a + 40:] == 0.0)
    assert np.array_equal(g[:, a:a + 40], oracle.xent_bwd(core, t_core, -100, 0.5))


@pytest.mark.parametrize("bc", [4, 64, 4096])
def test_split_masked_blocks_are_empty(bc):
    """A column block whose logits are all -inf reports the empty pair
    (m_b = -inf, d_b = 0), which the merge skips: the merged statistics of a
    row whose first 4096 columns are masked equal the full-row forward's."""
    rng = np.random.default_rng(bc)
    V = 4096 + 300
    z = rng.normal(0, 3, (4, V)).astype(np.float32)
    z[:, :4096] = -np.inf
    t = np.array([4096, V - 1, 4200, -100], dtype=np.int32)
    part = oracle.xent_partial(z, t, -100, block_cols=bc)
    nmasked = 4096 // bc
    assert np.all(part[:nmasked, :, 0] == -np.inf) and np.all(part[:nmasked, :, 1] == 0.0)
    st = oracle.xent_merge(part, t, V, -100)
    ref = oracle.xent_fwd(z, t, -100)
    assert np.all(np.isfinite(st[:3])) and np.array_equal(st[:, 0], ref[:, 0])
    assert np.array_equal(st[:, 2], ref[:, 2])
    np.testing.assert_allclose(st[:, 1], ref[:, 1], rtol=1e-13, atol=0)
    np.testing.assert_allclose(st[:, 3], ref[:, 3], rtol=1e-12, atol=1e-12)


def test_fully_masked_row_has_no_loss():
    """A row whose logits are all -inf has no softmax: m = -inf, d = 0 (the
    empty sum) and a NaN loss; an ignored such row still has loss 0."""
    z = np.full((2, 9), -np.inf, dtype=np.float32)
    st = oracle.xent_fwd(z, np.array([3, -100], dtype=np.int32), -100)
    assert np.all(st[:, 0] == -np.inf) and np.all(st[:, 1] == 0.0)
    assert np.isnan(st[0, 3]) and st[1, 3] == 0.0


def test_xent_mean():
    loss = np.array([1.5, 9.0, 2.25, 4.0, 0.5])
    t = np.array([3, -100, 1, -100, 0], np.int32)
    mean, inv, nv = oracle.xent_mean(loss, t, -100)
    assert nv == 3 and inv == 1.0 / 3
    assert mean == math.fsum([1.5, 2.25, 0.5]) / 3
    mean, inv, nv = oracle.xent_mean(loss, np.full(5, -100, np.int32), -100)
    assert (mean, inv, nv) == (0.0, 0.0, 0)
    mean, inv, nv = oracle.xent_mean(np.zeros(0), np.zeros(0, np.int32), -100)
    assert (mean, inv, nv) == (0.0, 0.0, 0)


# ------------------------------------------------------- BF16 rounding pins

def _torch_bf16_bits(f32):
    import torch
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_round_bf16_hand_values():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2 ** -8, 0x3F80),              # tie -> even (1.0)
        (1.0 + 3 * 2 ** -8, 0x3F82),          # tie -> even (1 + 2^-6)
        (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),   # just above the tie
        (-2.0, 0xC000),
        (65535.0, 0x4780),                    # rounds up into the next binade
        (2039.0, 0x44FF),                     # 2039 -> 2040 (spacing 8)
        (float(np.finfo(np.float32).max), 0x7F80),  # past the largest BF16 -> inf
        (2.0 ** -133, 0x0001),                # smallest BF16 subnormal
        (2.0 ** -134, 0x0000),                # tie with zero -> even (zero)
        (3 * 2.0 ** -134, 0x0002),            # tie -> even
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    vals = np.array([v for v, _ in cases], dtype=np.float64)
    got = oracle.round_bf16(vals)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
    assert int(oracle.round_bf16(np.array([np.nan]))[0]) == 0x7FC0


def test_round_bf16_matches_torch_on_fp32_inputs():
    """Every FP32 input class (normals, subnormals, exact ties, huge values)
    rounds as torch's CPU cast does."""
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties, ties | 0x10000])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, _torch_bf16_bits(f))


# ------------------------------------------------------ generator sanity

def test_generator_deterministic_and_in_range():
    a = workloads.tiny_exact()
    b = workloads.tiny_exact()
    assert np.array_equal(a.x, b.x) and np.array_equal(a.W, b.W) and np.array_equal(a.target, b.target)
    assert a.x.shape == (16, 512) and a.W.shape == (1024, 512)
    assert a.target.min() >= 0 and a.target.max() < 1024
    z = workloads.xent_logits(64, 500, spike_frac=0.05, ignore_frac=0.1, seed=3)
    assert z.logits.shape == (64, 500) and z.spike_rows.size == 3
    assert np.sum(z.target == -100) == 6
    for r, c in zip(z.spike_rows, z.spike_cols):
        assert z.logits[r, c] > 10.0
