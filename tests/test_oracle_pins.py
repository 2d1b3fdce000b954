"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test reaches the expected value by a route that does not go through the
oracle function it checks: a library routine (scipy's Hadamard, numpy's QR,
torch's bfloat16 rounding), a closed form, an explicit permutation-matrix
construction, or an invariant (orthogonality, exact inverse, norm
preservation).  Citations name the page and section the property comes from:
[TS] is the HARP technical summary (gist.science, paper 2605.29843), [ABS] the
arXiv abstract of that paper, [RHT] the abstract of "Quantizing With
Randomized Hadamard Transforms: Efficient Heuristic Now Proven".
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import harp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _recursive_sylvester(n):
    """H_1 = [1], H_2n = [[H, H], [H, -H]] (unnormalised)."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ---------------------------------------------------------------- P1 Sylvester
@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32])
def test_sylvester_matches_recursive_construction(b):
    # [TS §2.2]: normalised Sylvester Hadamard base mixer.
    want = _recursive_sylvester(b) / np.sqrt(b)
    np.testing.assert_array_equal(O.sylvester(b), want)
    np.testing.assert_allclose(O.sylvester(b) @ O.sylvester(b).T, np.eye(b), atol=1e-15)


def test_sylvester_matches_scipy():
    np.testing.assert_array_equal(O.sylvester(64) * 8.0, scipy.linalg.hadamard(64).astype(float))


# ---------------------------------------------------------------- P2 QR fallback
@pytest.mark.parametrize("b", [3, 5, 6, 7, 12])
def test_qr_fallback_unique_factor(b):
    # [TS §2.1/§2.2]: QR of a fixed Gaussian matrix; diag(R) > 0 makes Q unique,
    # so Householder (LAPACK) and modified Gram-Schmidt must agree.
    z = RNG.standard_normal((b, b))
    q = O.qr_fallback(z)
    q2, r2 = O.mgs_qr(z)
    assert np.all(np.diag(r2) > 0)
    np.testing.assert_allclose(q, q2, atol=1e-13)
    r = q.T @ z
    assert np.all(np.diag(r) > 0)
    np.testing.assert_allclose(np.tril(r, -1), 0.0, atol=1e-13)
    np.testing.assert_allclose(q @ r, z, atol=1e-14 * np.abs(z).max() * b)
    np.testing.assert_allclose(q.T @ q, np.eye(b), atol=1e-14)


# ---------------------------------------------------------------- P3 Cayley
def test_cayley_zero_is_identity():
    for b in (3, 5, 8, 16):
        np.testing.assert_array_equal(O.cayley(np.zeros(b * (b - 1) // 2), b), np.eye(b))


@pytest.mark.parametrize("b", [3, 4, 5, 8, 16])
def test_cayley_orthogonal_special_and_odd(b):
    p = RNG.standard_normal(b * (b - 1) // 2) * 0.3
    q = O.cayley(p, b)
    np.testing.assert_allclose(q.T @ q, np.eye(b), atol=1e-14)
    assert abs(np.linalg.det(q) - 1.0) < 1e-12
    np.testing.assert_allclose(O.cayley(-p, b), q.T, atol=1e-14)


def test_cayley_2x2_closed_form():
    for a in (0.0, 0.1, -0.7, 2.5):
        want = np.array([[1 - a * a, -2 * a], [2 * a, 1 - a * a]]) / (1 + a * a)
        np.testing.assert_allclose(O.cayley(np.array([a]), 2), want, atol=1e-15)


def test_cayley_3x3_rodrigues_closed_form():
    # For 3x3 skew A with |w|^2 = sum of its parameters squared,
    # (I - A)(I + A)^-1 = I + 2(A^2 - A) / (1 + |w|^2).
    p = np.array([0.3, -0.2, 0.5])
    a = np.array([[0, p[0], p[1]], [-p[0], 0, p[2]], [-p[1], -p[2], 0]])
    want = np.eye(3) + 2 * (a @ a - a) / (1 + p @ p)
    np.testing.assert_allclose(O.cayley(p, 3), want, atol=1e-15)


# ---------------------------------------------------------------- P4 Givens
def test_givens_closed_form():
    np.testing.assert_array_equal(O.givens(0.0), np.eye(2))
    t = 0.37
    g = O.givens(t)
    np.testing.assert_allclose(g @ np.array([1.0, 0.0]), [np.cos(t), np.sin(t)], atol=1e-16)
    np.testing.assert_allclose(g @ O.givens(-t), np.eye(2), atol=1e-16)


# ---------------------------------------------------------------- P5 Theta = 0 is the RHT
def _zero_blocks(schedule):
    d = int(np.prod(schedule))
    th = np.zeros(sum(O.theta_counts(schedule, d)))
    gs = np.concatenate([RNG.standard_normal(b * b) for b in schedule if not O.is_pow2(b)] or [np.zeros(0)])
    return O.materialize_blocks(schedule, d, th, gs)


@pytest.mark.parametrize("schedule", [(2,) * 6, (4, 16), (8, 8), (64,), (16, 4), (2, 8, 4)])
def test_theta_zero_equals_sylvester_times_signs_d64(schedule):
    # [TS §2.2] / [ABS]: at Theta = 0 every block is G_b and HARP equals the
    # fixed RHT H_d D_s; with Sylvester radices this holds for any schedule.
    d = 64
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    m = O.dense_operator(schedule, _zero_blocks(schedule), s)
    want = scipy.linalg.hadamard(d).astype(float) / np.sqrt(d) * s[None, :]
    np.testing.assert_allclose(m, want, atol=1e-15)


@pytest.mark.slow
def test_theta_zero_equals_sylvester_d4096():
    schedule = (8, 8, 8, 8)
    d = 4096
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    m = O.dense_operator(schedule, _zero_blocks(schedule), s)
    want = scipy.linalg.hadamard(d).astype(float) / 64.0 * s[None, :]
    assert np.abs(m - want).max() <= 1e-15


def test_theta_zero_equals_sylvester_d8192_columns():
    schedule = (8, 8, 8, 16)
    d = 8192
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    h = scipy.linalg.hadamard(d, dtype=np.int8)
    cols = RNG.choice(d, 48, replace=False)
    e = np.zeros((cols.size, d))
    e[np.arange(cols.size), cols] = 1.0
    y = O.apply(e, schedule, _zero_blocks(schedule), s)   # rows = M e_j
    want = h[:, cols].T.astype(float) / np.sqrt(d) * s[cols][:, None]
    assert np.abs(y - want).max() <= 1e-15


# ---------------------------------------------------------------- P6/P7 Kronecker routes
def _kron_all(mats):
    out = np.ones((1, 1))
    for mm in mats:
        out = np.kron(out, mm)
    return out


@pytest.mark.parametrize("schedule", [(8, 8, 8, 5, 2), (2, 3, 5), (3, 3, 3), (5, 2, 6), (8, 8, 3, 3)])
def test_theta_zero_mixed_radix_is_kronecker(schedule):
    # Index digits in C order (reading R1): stage t's base mixer acts on digit
    # t, so at Theta = 0 the operator is the Kronecker product of the base
    # mixers, in stage order, times D_s.
    d = int(np.prod(schedule))
    gs_list = {b: RNG.standard_normal((b, b)) for b in set(schedule) if not O.is_pow2(b)}
    gauss = np.concatenate([gs_list[b].ravel() for b in schedule if not O.is_pow2(b)] or [np.zeros(0)])
    blocks = O.materialize_blocks(schedule, d, np.zeros(sum(O.theta_counts(schedule, d))), gauss)
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    g = [scipy.linalg.hadamard(b) / np.sqrt(b) if O.is_pow2(b) else np.linalg.qr(gs_list[b])[0]
         * np.sign(np.diag(np.linalg.qr(gs_list[b])[1]))[None, :] for b in schedule]
    want = _kron_all(g) * s[None, :]
    if d <= 2048:
        np.testing.assert_allclose(O.dense_operator(schedule, blocks, s), want, atol=1e-13)
    else:
        cols = RNG.choice(d, 32, replace=False)
        e = np.zeros((cols.size, d))
        e[np.arange(cols.size), cols] = 1.0
        np.testing.assert_allclose(O.apply(e, schedule, blocks, s), want[:, cols].T, atol=1e-13)


@pytest.mark.parametrize("schedule", [(2, 3, 5), (4, 3, 2), (8, 5)])
def test_shared_blocks_are_kronecker(schedule):
    # With one block per stage (shared by all groups) the stages act on
    # different digits and the operator is the Kronecker product of the blocks.
    d = int(np.prod(schedule))
    per_stage = [np.linalg.qr(RNG.standard_normal((b, b)))[0] for b in schedule]
    blocks = [np.repeat(bt[None], d // b, axis=0) for bt, b in zip(per_stage, schedule)]
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    np.testing.assert_allclose(O.dense_operator(schedule, blocks, s), _kron_all(per_stage) * s[None, :], atol=1e-13)


# ---------------------------------------------------------------- P8 brute force
def _perm_route(schedule, blocks, signs):
    """M = prod_t P_t^T (block_diag_c B_{t,c}) P_t D_s, built from explicit
    permutation matrices (pure-Python loops, tiny d only)."""
    d = int(np.prod(schedule))
    m = np.diag(signs.astype(float))
    for t, b in enumerate(schedule):
        p = np.zeros((d, d))
        for i in range(d):
            digits = np.unravel_index(i, schedule)
            other = tuple(dg for u, dg in enumerate(digits) if u != t)
            other_shape = tuple(bb for u, bb in enumerate(schedule) if u != t)
            c = int(np.ravel_multi_index(other, other_shape)) if other else 0
            p[c * b + digits[t], i] = 1.0
        bd = scipy.linalg.block_diag(*blocks[t])
        m = p.T @ bd @ p @ m
    return m


@pytest.mark.parametrize("schedule", [(2, 3), (3, 2, 2), (2, 3, 5), (5, 2, 4), (3, 4, 5), (2, 2, 2, 2, 2, 2), (6, 5)])
def test_brute_force_permutation_route(schedule):
    # [TS §2.1]: stages of block-diagonal orthogonal matrices on coordinate
    # groups separated by stride permutations.
    d = int(np.prod(schedule))
    th = RNG.standard_normal(sum(O.theta_counts(schedule, d))) * 0.4
    gauss = np.concatenate([RNG.standard_normal(b * b) for b in schedule if not O.is_pow2(b)] or [np.zeros(0)])
    blocks = O.materialize_blocks(schedule, d, th, gauss)
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    np.testing.assert_allclose(O.dense_operator(schedule, blocks, s), _perm_route(schedule, blocks, s), atol=1e-13)
    x = RNG.standard_normal((5, d))
    np.testing.assert_allclose(O.apply(x, schedule, blocks, s), x @ _perm_route(schedule, blocks, s).T, atol=1e-13)


def test_block_definition_q_times_g():
    # [TS §2.2]: B_{t,c} = Q_{t,c}(theta) G_{b_t}; check one group of each kind.
    schedule = (2, 5, 8)
    d = 80
    th = RNG.standard_normal(sum(O.theta_counts(schedule, d))) * 0.2
    z5 = RNG.standard_normal((5, 5))
    blocks = O.materialize_blocks(schedule, d, th, z5.ravel())
    counts = O.theta_counts(schedule, d)
    # stage 0 (radix 2), group 7: one Givens angle
    ang = th[7]
    np.testing.assert_allclose(blocks[0][7], O.givens(ang) @ (scipy.linalg.hadamard(2) / np.sqrt(2)), atol=1e-15)
    # stage 1 (radix 5), group 3: 10 Cayley params after stage 0's
    p = th[counts[0] + 3 * 10: counts[0] + 4 * 10]
    a = np.zeros((5, 5))
    a[np.triu_indices(5, 1)] = p
    a = a - a.T
    q = np.linalg.inv(np.eye(5) + a) @ (np.eye(5) - a)
    qr_q, qr_r = np.linalg.qr(z5)
    g5 = qr_q * np.sign(np.diag(qr_r))[None, :]
    np.testing.assert_allclose(blocks[1][3], q @ g5, atol=1e-14)


# ---------------------------------------------------------------- P9/P10 orthogonality, inverse
CONFIG_SCHEDULES = [(2,) * 6, (8, 8, 8, 8), (8, 8, 8, 5, 2), (8, 8, 8, 3, 3, 3), (8, 8, 8, 16)]


@pytest.mark.parametrize("schedule", [(2,) * 6, (8, 8, 8, 5, 2), (8, 8), (3, 5, 7)])
def test_dense_orthogonal(schedule):
    d = int(np.prod(schedule))
    th = RNG.standard_normal(sum(O.theta_counts(schedule, d))) * 0.05
    gauss = np.concatenate([RNG.standard_normal(b * b) for b in schedule if not O.is_pow2(b)] or [np.zeros(0)])
    blocks = O.materialize_blocks(schedule, d, th, gauss)
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    m = O.dense_operator(schedule, blocks, s)
    assert np.abs(m.T @ m - np.eye(d)).max() <= 1e-12


@pytest.mark.parametrize("schedule", CONFIG_SCHEDULES)
def test_inverse_roundtrip_and_norm(schedule):
    # Exact change of basis [TS §5; ABS]: apply_inverse(apply(x)) = x and
    # ||Mx|| = ||x|| for every row.
    d = int(np.prod(schedule))
    th = RNG.standard_normal(sum(O.theta_counts(schedule, d))) * 0.05
    gauss = np.concatenate([RNG.standard_normal(b * b) for b in schedule if not O.is_pow2(b)] or [np.zeros(0)])
    blocks = O.materialize_blocks(schedule, d, th, gauss)
    s = np.where(RNG.integers(0, 2, d) == 1, 1.0, -1.0)
    x = RNG.standard_t(3, size=(4, d))
    y = O.apply(x, schedule, blocks, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert O.row_rel_l2(O.apply_inverse(y, schedule, blocks, s), x).max() <= 1e-12


def test_stage_order_matters_and_is_stage0_first():
    # Reading R3: M = S_1 S_0 D_s for a two-stage schedule; build the two
    # stage operators separately (single-stage schedules on the same digits).
    schedule = (3, 4)
    d = 12
    th = RNG.standard_normal(sum(O.theta_counts(schedule, d))) * 0.5
    blocks = O.materialize_blocks(schedule, d, th, RNG.standard_normal(9))
    s = np.ones(d)
    ident = [np.repeat(np.eye(3)[None], 4, axis=0), np.repeat(np.eye(4)[None], 3, axis=0)]
    s0 = O.dense_operator(schedule, [blocks[0], ident[1]], s)
    s1 = O.dense_operator(schedule, [ident[0], blocks[1]], s)
    m = O.dense_operator(schedule, blocks, s)
    np.testing.assert_allclose(m, s1 @ s0, atol=1e-14)
    assert np.abs(m - s0 @ s1).max() > 1e-3


# ---------------------------------------------------------------- P11 RHT composition
def test_rht_identities():
    # [RHT]: y = H D_k ... H D_1 x.  With all-ones signs H^2 = I.
    d = 256
    x = RNG.standard_normal((3, d))
    ones = np.ones((1, d))
    h = scipy.linalg.hadamard(d) / np.sqrt(d)
    np.testing.assert_allclose(O.rht_compose(x, np.repeat(ones, 2, 0)), x, atol=1e-13)
    np.testing.assert_allclose(O.rht_compose(x, np.repeat(ones, 3, 0)), x @ h.T, atol=1e-13)


def test_rht_one_hot_flat():
    d = 8192
    s = np.where(RNG.integers(0, 2, (1, d)) == 1, 1.0, -1.0)
    e = np.zeros((1, d))
    e[0, 1234] = 1.0
    y = O.rht_compose(e, s)
    np.testing.assert_allclose(np.abs(y), 1.0 / np.sqrt(d), atol=1e-16)


def test_rht_equals_sequential_harp_at_theta_zero():
    schedule = (8, 8, 8, 16)
    d = 8192
    signs = np.where(RNG.integers(0, 2, (3, d)) == 1, 1.0, -1.0)
    x = RNG.standard_normal((4, d))
    blocks = _zero_blocks(schedule)
    want = x
    for s in signs:
        want = O.apply(want, schedule, blocks, s)
    np.testing.assert_allclose(O.rht_compose(x, signs), want, atol=1e-13)
    np.testing.assert_allclose(O.rht_compose(want, signs, inverse=True), x, atol=1e-12)


# ---------------------------------------------------------------- P12 two-sided
def test_two_sided_small_dense():
    # [TS §3, ABS]: two-sided processor W~ = M_U W M_V^T, exact change of basis.
    su, sv = (2, 3), (5, 2)
    du, dv = 6, 10
    thu = RNG.standard_normal(sum(O.theta_counts(su, du))) * 0.3
    thv = RNG.standard_normal(sum(O.theta_counts(sv, dv))) * 0.3
    bu = O.materialize_blocks(su, du, thu, RNG.standard_normal(9))
    bv = O.materialize_blocks(sv, dv, thv, RNG.standard_normal(25))
    sgu = np.where(RNG.integers(0, 2, du) == 1, 1.0, -1.0)
    sgv = np.where(RNG.integers(0, 2, dv) == 1, 1.0, -1.0)
    w = RNG.standard_normal((du, dv))
    mu = _perm_route(su, bu, sgu)
    mv = _perm_route(sv, bv, sgv)
    wt = O.rotate_weight(w, su, bu, sgu, sv, bv, sgv)
    np.testing.assert_allclose(wt, mu @ w @ mv.T, atol=1e-13)
    assert abs(np.linalg.norm(wt) - np.linalg.norm(w)) <= 1e-13 * np.linalg.norm(w)
    np.testing.assert_allclose(O.rotate_weight(wt, su, bu, sgu, sv, bv, sgv, inverse=True), w, atol=1e-13)


def test_two_sided_theta_zero_hadamard():
    su, sv = (4, 2), (2, 8)
    w = RNG.standard_normal((8, 16))
    bu, bv = _zero_blocks(su), _zero_blocks(sv)
    hm = scipy.linalg.hadamard(8) / np.sqrt(8)
    hn = scipy.linalg.hadamard(16) / 4.0
    np.testing.assert_allclose(O.rotate_weight(w, su, bu, np.ones(8), sv, bv, np.ones(16)), hm @ w @ hn, atol=1e-14)


# ---------------------------------------------------------------- storage formats
def test_round_bf16_matches_torch_on_fp32_values():
    v = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(v.astype(np.float64)), want)


def test_round_bf16_nearest_from_fp64():
    v = RNG.standard_normal(20000) * np.exp(RNG.uniform(-10, 10, 20000))
    r = O.round_bf16(v)
    # representable: the low 16 bits of the fp32 pattern are zero
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # nearest: error at most half a unit in the 8th significant bit
    ulp = np.ldexp(1.0, np.frexp(v)[1] - 8)
    assert np.all(np.abs(r - v) <= ulp / 2)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert O.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_quantize_i8_bounds():
    bt = RNG.standard_normal((50, 8, 8)) * 0.3
    code, scale = O.quantize_i8(bt)
    assert code.dtype == np.int8 and np.all(np.abs(code.astype(int)) <= 127)
    deq = code.astype(float) * scale.astype(float)[:, None, None]
    assert np.all(np.abs(deq - bt) <= scale.astype(float)[:, None, None] * 0.5 + 1e-12)
    assert np.all(np.abs(code.reshape(50, -1)).max(axis=1) >= 126)


def test_bf16x2_storage_error():
    bt = [RNG.standard_normal((10, 8, 8)) * 0.3]
    st = O.stored_blocks(bt, "bf16x2")[0]
    assert np.all(np.abs(st - bt[0]) <= np.abs(bt[0]) * 2.0 ** -16)


# ---------------------------------------------------------------- facts the pages print
def test_pages_facts_fixture():
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)
    # [TS §2.1] example: d = 5120 with the mixed-radix schedule (8, 8, 8, 5, 2)
    ex = facts["mixed_radix_example"]
    assert int(np.prod(ex["schedule"])) == ex["d"]
    sch = tuple(ex["schedule"])
    blocks = _zero_blocks(sch)
    assert [bt.shape for bt in blocks] == [(ex["d"] // b, b, b) for b in sch]
    # [TS §4] int8 parameters raise bits per parameter from 2.00 to 2.05 on a
    # 2-bit model; per-group Cayley parameters on a two-sided (8,8,8,8)
    # processor of a 4096 x 4096 layer give that overhead, a per-stage
    # sharing would not (reading R10).
    bpp = facts["bits_per_param"]
    d = 4096
    n_params = 2 * sum(O.theta_counts((8, 8, 8, 8), d))
    overhead = n_params * 8 / (d * d)
    assert round(bpp["base"] + overhead, 2) == bpp["with_harp_int8"]
    per_stage = 2 * 4 * 28
    assert round(bpp["base"] + per_stage * 8 / (d * d), 2) != bpp["with_harp_int8"]


def test_golden_small_cases_regression():
    # Stored by tests/golden/make_golden.py, which calls only the oracle.
    with open(os.path.join(GOLDEN, "small_cases.json")) as f:
        cases = json.load(f)
    for case in cases:
        sch = tuple(case["schedule"])
        d = case["d"]
        blocks = O.materialize_blocks(sch, d, np.array(case["theta"]), np.array(case["gauss"]))
        y = O.apply(np.array(case["x"]), sch, blocks, np.array(case["signs"], dtype=float))
        np.testing.assert_allclose(y, np.array(case["y"]), atol=1e-14)


# ------------------------------------------------------------------ int8 parameter storage
def test_theta_i8_hand_example():
    # [TS §2.4] parameters may be stored in int8; the per-stage scale is
    # reading R11.  The fixture was worked out by hand: a per-group scale, a
    # wrong stage split or a dropped rounding all give other codes.
    with open(os.path.join(GOLDEN, "theta_i8_hand.json")) as f:
        case = json.load(f)
    sch, d = tuple(case["schedule"]), case["d"]
    codes, scales = O.quantize_theta(sch, d, np.array(case["theta"]))
    assert codes.dtype == np.int8 and scales.dtype == np.float32
    np.testing.assert_array_equal(codes.astype(int), case["codes"])
    want = np.array([np.float32(n / q) for n, q in case["scale_quotients"]], dtype=np.float32)
    np.testing.assert_array_equal(scales, want)
    back = O.dequantize_theta(sch, d, codes, scales)
    np.testing.assert_array_equal(back, np.array(case["codes"], dtype=float) *
                                  np.repeat(want.astype(float), [6, 12, 6]))


def test_theta_i8_scale_granularity_matches_bits_per_param():
    # [TS §4] int8 HARP parameters raise bits per parameter from 2.00 to 2.05
    # (2-bit model).  On a two-sided (8,8,8,8) processor of a 4096 x 4096
    # layer, per-stage fp32 scales keep that figure; per-group fp32 scales
    # would add 0.008 bits and give 2.06 (reading R11).
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        bpp = json.load(f)["bits_per_param"]
    d, sch = 4096, (8, 8, 8, 8)
    codes_bits = 2 * sum(O.theta_counts(sch, d)) * 8
    per_stage = codes_bits + 2 * len(sch) * 32
    per_group = codes_bits + 2 * sum(d // b for b in sch) * 32
    assert round(bpp["base"] + per_stage / d ** 2, 2) == bpp["with_harp_int8"]
    assert round(bpp["base"] + per_group / d ** 2, 2) != bpp["with_harp_int8"]


@pytest.mark.parametrize("sch,d", [((8, 8), 64), ((2, 5, 4), 40), ((16, 2, 3), 96)])
def test_theta_i8_properties(sch, d):
    # Symmetric rounding to the nearest code: the error per parameter is at
    # most half its stage's scale, each stage's largest magnitude maps to
    # +-127, negation commutes with quantisation, and dequantisation returns
    # the exact product code * scale.
    n = sum(O.theta_counts(sch, d))
    theta = RNG.standard_normal(n) * 0.3
    codes, scales = O.quantize_theta(sch, d, theta)
    assert codes.size == n and scales.size == len(sch)
    back = O.dequantize_theta(sch, d, codes, scales)
    counts = O.theta_counts(sch, d)
    sscale = np.repeat(scales.astype(np.float64), counts)
    assert np.all(np.abs(back - theta) <= 0.5 * sscale * (1 + 1e-12))
    lo = 0
    for n_t in counts:
        assert np.abs(codes[lo:lo + n_t].astype(int)).max() == 127
        lo += n_t
    nc, ns = O.quantize_theta(sch, d, -theta)
    np.testing.assert_array_equal(nc, -codes)
    np.testing.assert_array_equal(ns, scales)
    np.testing.assert_array_equal(back, codes.astype(np.float64) * sscale)


def test_theta_i8_zero_and_cayley_lipschitz():
    # All-zero parameters quantise to zero codes and scales, so the blocks are
    # the base mixers G [TS §2.2].  For skew A, ||(I + A)^-1||_2 <= 1, so the
    # Cayley factor moves by at most 2 ||dA||_2 + O(dA^2) when the parameters
    # are rounded to int8.
    sch, d = (8, 4), 32
    n = sum(O.theta_counts(sch, d))
    codes, scales = O.quantize_theta(sch, d, np.zeros(n))
    assert not codes.any() and not scales.any()
    theta = RNG.standard_normal(n) * 0.2
    codes, scales = O.quantize_theta(sch, d, theta)
    back = O.dequantize_theta(sch, d, codes, scales)
    b0 = O.materialize_blocks(sch, d, theta, None)
    b1 = O.materialize_blocks(sch, d, back, None)
    pos = 0
    for t, b in enumerate(sch):
        per = b * (b - 1) // 2
        for c in range(d // b):
            da = O.skew_from_params(back[pos:pos + per], b) - O.skew_from_params(theta[pos:pos + per], b)
            pos += per
            bound = 2 * np.linalg.norm(da, 2)
            assert np.linalg.norm(b1[t][c] - b0[t][c], 2) <= bound * 1.05 + 1e-15


# ------------------------------------------------------------------ reverse mode (calibration gradients)
def _vjp_case(sch, d, rows, seed, sigma=0.2):
    rng = np.random.default_rng(seed)
    theta = rng.standard_normal(sum(O.theta_counts(sch, d))) * sigma
    gl = O.gauss_stage_list(sch)
    gauss = np.concatenate([rng.standard_normal(sch[t] ** 2) for t in gl]) if gl else None
    signs = rng.choice([-1.0, 1.0], d)
    x = rng.standard_normal((rows, d))
    dy = rng.standard_normal((rows, d))
    return theta, gauss, signs, x, dy


@pytest.mark.parametrize("sch,d", [((2, 3, 4), 24), ((8, 8), 64), ((5, 2), 10)])
def test_vjp_dx_is_transpose_apply(sch, d):
    # dL/dx = M^T dy; M is orthogonal [TS §2.1], so this is also the inverse
    # transform and the dense operator's transpose times dy.
    theta, gauss, signs, x, dy = _vjp_case(sch, d, 3, 11)
    blocks = O.materialize_blocks(sch, d, theta, gauss)
    dx, _ = O.apply_vjp(x, sch, blocks, signs, dy)
    m = O.dense_operator(sch, blocks, signs)
    np.testing.assert_allclose(dx, dy @ m, atol=1e-12)
    np.testing.assert_allclose(dx, O.apply_inverse(dy, sch, blocks, signs), atol=1e-12)


@pytest.mark.parametrize("sch,d", [((2, 3, 4), 24), ((3, 2), 6)])
def test_vjp_dblocks_central_differences(sch, d):
    # y is linear in each single block entry, so a central difference of
    # L = sum <dy, y> in that entry is exact up to rounding.
    theta, gauss, signs, x, dy = _vjp_case(sch, d, 4, 12)
    blocks = O.materialize_blocks(sch, d, theta, gauss)
    _, dblocks = O.apply_vjp(x, sch, blocks, signs, dy)
    h = 0.5
    for t in range(len(sch)):
        for idx in np.ndindex(blocks[t].shape):
            bp = [b.copy() for b in blocks]
            bm = [b.copy() for b in blocks]
            bp[t][idx] += h
            bm[t][idx] -= h
            fd = (np.sum(dy * O.apply(x, sch, bp, signs)) - np.sum(dy * O.apply(x, sch, bm, signs))) / (2 * h)
            assert abs(fd - dblocks[t][idx]) <= 1e-11 * max(1.0, abs(fd)), (t, idx)


@pytest.mark.parametrize("sch,d", [((2, 3, 4), 24), ((5, 2), 10), ((4, 4), 16)])
def test_theta_vjp_central_differences(sch, d):
    # The whole chain theta -> blocks -> y against central differences of the
    # oracle forward: O(h^2) truncation, h = 1e-5.
    theta, gauss, signs, x, dy = _vjp_case(sch, d, 3, 13)
    blocks = O.materialize_blocks(sch, d, theta, gauss)
    _, dblocks = O.apply_vjp(x, sch, blocks, signs, dy)
    dtheta = O.theta_vjp(sch, d, theta, gauss, dblocks)

    def loss(th):
        return np.sum(dy * O.apply(x, sch, O.materialize_blocks(sch, d, th, gauss), signs))
    h = 1e-5
    for i in range(theta.size):
        tp, tm = theta.copy(), theta.copy()
        tp[i] += h
        tm[i] -= h
        fd = (loss(tp) - loss(tm)) / (2 * h)
        assert abs(fd - dtheta[i]) <= 1e-7 * max(1.0, abs(fd)), i


def test_theta_vjp_matches_torch_autograd():
    # The theta -> block map differentiated by torch's autograd (fp64, CPU):
    # Cayley by a linear solve, Givens by cos/sin, times the same base G.
    sch, d = (4, 2, 3), 24
    theta, gauss, _, _, _ = _vjp_case(sch, d, 1, 14)
    rng = np.random.default_rng(15)
    dblocks = [rng.standard_normal((d // b, b, b)) for b in sch]
    want = O.theta_vjp(sch, d, theta, gauss, dblocks)
    th = torch.tensor(theta, dtype=torch.float64, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    pos = gpos = 0
    for t, b in enumerate(sch):
        if O.is_pow2(b):
            g = torch.tensor(O.sylvester(b))
        else:
            g = torch.tensor(O.qr_fallback(gauss[gpos:gpos + b * b].reshape(b, b)))
            gpos += b * b
        per = 1 if b == 2 else b * (b - 1) // 2
        for c in range(d // b):
            p = th[pos + c * per: pos + (c + 1) * per]
            if b == 2:
                cs, sn = torch.cos(p[0]), torch.sin(p[0])
                q = torch.stack([torch.stack([cs, -sn]), torch.stack([sn, cs])])
            else:
                u = torch.zeros(b, b, dtype=torch.float64)
                iu = torch.triu_indices(b, b, 1)
                u = u.index_put((iu[0], iu[1]), p)
                a = u - u.T
                eye = torch.eye(b, dtype=torch.float64)
                q = torch.linalg.solve(eye + a, eye - a)
            loss = loss + torch.sum(torch.tensor(dblocks[t][c]) * (q @ g))
        pos += (d // b) * per
    loss.backward()
    np.testing.assert_allclose(want, th.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_theta_vjp_at_zero_closed_form():
    # At theta = 0: Q = I and M = I, so dL/dA = -2 dL/dQ and
    # dtheta_(r,k) = -2 (dQ[r,k] - dQ[k,r]) for Cayley; for Givens
    # dtheta = dQ[1,0] - dQ[0,1]; dQ = dB G^T.
    sch, d = (4, 2), 8
    rng = np.random.default_rng(16)
    dblocks = [rng.standard_normal((d // b, b, b)) for b in sch]
    dt = O.theta_vjp(sch, d, np.zeros(sum(O.theta_counts(sch, d))), None, dblocks)
    g4 = scipy.linalg.hadamard(4) / 2.0
    g2 = scipy.linalg.hadamard(2) / np.sqrt(2.0)
    pos = 0
    for c in range(2):
        gq = dblocks[0][c] @ g4.T
        for r in range(4):
            for k in range(r + 1, 4):
                assert abs(dt[pos] - (-2.0) * (gq[r, k] - gq[k, r])) < 1e-12
                pos += 1
    for c in range(4):
        gq = dblocks[1][c] @ g2.T
        assert abs(dt[pos] - (gq[1, 0] - gq[0, 1])) < 1e-12
        pos += 1


def test_rht_one_hot_marginals_diagnostic():
    # [RHT]: composing randomized Hadamard transforms makes the coordinates of
    # any input close to Gaussian.  For the one-hot rows of the d = 8192, k = 3
    # workload, sqrt(d) * y / ||y|| is exactly two-point (+-1) after one RHT,
    # and its pooled per-coordinate marginal after two and three RHTs is
    # compared with N(0, 1) by the Kolmogorov distance (a diagnostic; the bound
    # below only guards against a broken transform: the values sit on a
    # lattice of spacing 2 / sqrt(d), which alone keeps the distance near
    # 0.2 * 2 / sqrt(d) ~ 0.004).
    import scipy.stats
    from structured_rotations_amd import workloads as W
    w = W.make("rht3_8192_bf16", rows=256)
    x = w["x"].astype(np.float64)
    d = w["d"]
    one_hot = x[(np.count_nonzero(x, axis=1) == 1)][:16]
    assert one_hot.shape[0] >= 8
    signs = w["signs"].astype(float)
    dist = {}
    for k in (1, 2, 3):
        y = O.rht_compose(one_hot, signs[:k])
        z = np.sqrt(d) * y / np.linalg.norm(y, axis=1, keepdims=True)
        if k == 1:
            np.testing.assert_allclose(np.abs(z), 1.0, atol=1e-12)
            continue
        dist[k] = scipy.stats.kstest(z.ravel(), "norm").statistic
    print(f"Kolmogorov distance to N(0,1): k=2 {dist[2]:.4f}, k=3 {dist[3]:.4f}")
    assert dist[2] < 0.02 and dist[3] < 0.02


# ---------------------------------------------------------------- parity metric
def test_row_rel_l2_hand_example():
    # The per-row relative l2 error every parity bound is stated for, against
    # values worked out by hand (tests/golden/row_rel_l2_hand.json): a divisor
    # of ||y|| instead of ||ref||, a sum instead of a difference, a squared
    # ratio, a max over columns, a zero reference row or one global ratio over
    # the batch would each give other numbers.
    with open(os.path.join(GOLDEN, "row_rel_l2_hand.json")) as f:
        fx = json.load(f)
    got = O.row_rel_l2(np.array(fx["y"], dtype=float), np.array(fx["ref"], dtype=float))
    assert got.shape == (len(fx["ref"]),)
    np.testing.assert_allclose(got, fx["per_row"], rtol=1e-15, atol=0)


def test_row_rel_l2_scale_and_single_row():
    # Invariants that need no arithmetic of the metric: a common factor on both
    # arguments leaves it unchanged, equal rows give exactly zero, and a 1-D row
    # is treated as one row.
    y = np.array([[1.0, -2.0, 0.5], [0.0, 3.0, 4.0]])
    ref = np.array([[1.0, -2.5, 0.0], [0.0, 3.0, 4.0]])
    np.testing.assert_allclose(O.row_rel_l2(7.0 * y, 7.0 * ref), O.row_rel_l2(y, ref), rtol=1e-15)
    assert O.row_rel_l2(ref, ref).tolist() == [0.0, 0.0]
    assert O.row_rel_l2(y[0], ref[0]).shape == (1,)
