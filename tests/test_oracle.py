"""Pins for the CPU oracle, against things other than the oracle itself.

Each test names what fixes the expected value: a closed form, an integer
special case checked with numpy int64 matmul (exact), a library conversion,
brute force over the candidate integers, a value worked by hand, or an
invariant.  Together they are chosen so that a plausible slip in the oracle (a
field read from the wrong bits, a swapped nibble, a transposed operand, a
dropped min term, a wrong rounding) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from tests import fmt_helpers as fh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- scalars

def test_half_to_double_all_bit_patterns(orc):
    """Every fp16 bit pattern decodes to what numpy's float16 conversion gives."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_to_double_matches_torch(orc):
    import torch
    g = np.random.default_rng(7)
    bits = np.concatenate([g.integers(0, 65536, 4000), [0, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x0080]])
    bits = bits.astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_silu_closed_forms(orc):
    assert orc.silu(0.0) == 0.0
    for z in [1e-3, 0.5, 1.0, 3.0, 17.0, 40.0]:
        # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
        assert abs((orc.silu(z) - orc.silu(-z)) - z) <= 1e-15 * max(1.0, z)
    assert abs(orc.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert orc.silu(800.0) == 800.0
    assert orc.silu(-800.0) == 0.0


# ---------------------------------------------------------------- activation quantization

def test_quantize_hand_block_ties_to_even(orc):
    """amax = 127 makes the scale exactly 1, so q is x rounded half to even (worked by hand)."""
    x = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5, 126.5, -126.5, 0.25, 0.75, -3.5, 4.5, 5.5, -5.5,
         100.49, 100.51, 0.0, -0.0, 1.0, -1.0, 64.0, -64.0, 10.5, 11.5, 12.5, 13.5, -10.5, -11.5, -12.5, -13.5]
    want = [127, 2, 4, -2, 0, 2, 0, -2, 126, -126, 0, 1, -4, 4, 6, -6,
            100, 101, 0, 0, 1, -1, 64, -64, 10, 12, 12, 14, -10, -12, -12, -14]
    qx, dx, sx = orc.quantize_act_q8(np.array([x], np.float32))
    assert dx[0, 0] == 1.0
    assert qx[0].tolist() == want
    assert sx[0, 0] == sum(want)


def test_quantize_zero_and_single_spike(orc):
    x = np.zeros((1, 64), np.float32)
    x[0, 40] = -3.7
    qx, dx, sx = orc.quantize_act_q8(x)
    assert dx[0, 0] == 0.0 and not qx[0, :32].any() and sx[0, 0] == 0
    assert qx[0, 40] == -127 and sx[0, 1] == -127
    assert np.count_nonzero(qx[0, 32:]) == 1
    # scale is the correctly rounded fp32 quotient: within half an ulp of 3.7f/127
    d = float(dx[0, 1])
    exact = float(np.float32(3.7)) / 127.0
    assert abs(d - exact) <= 0.5 * float(np.spacing(np.float32(d)))


def _nearest_int_brute(r: np.ndarray) -> np.ndarray:
    """Nearest integer in [-127, 127] to each r by exhaustive search, ties to the even one."""
    cand = np.arange(-127, 128, dtype=np.float64)
    dist = np.abs(r.astype(np.float64)[..., None] - cand)
    best = dist.min(axis=-1, keepdims=True)
    hit = dist == best
    # among equally near candidates prefer the even one
    even = (np.abs(cand) % 2 == 0)
    pick_even = hit & even
    use = np.where(pick_even.any(axis=-1, keepdims=True), pick_even, hit)
    return cand[np.argmax(use, axis=-1)].astype(np.int64)


def test_quantize_brute_force_nearest(orc):
    """q is the nearest integer (ties even, clamped) to the fp32 quotient x/d, found by search."""
    g = np.random.default_rng(11)
    scales = 10.0 ** g.uniform(-6, 4, size=(300, 1))
    x = (g.standard_normal((300, 32)) * scales).astype(np.float32)
    x[::7, ::5] = 0.0
    qx, dx, sx = orc.quantize_act_q8(x.reshape(1, -1))
    qx = qx.reshape(300, 32)
    dx = dx.reshape(300)
    r = (x / dx[:, None].astype(np.float32)).astype(np.float32)  # IEEE fp32 quotient
    assert np.array_equal(qx.astype(np.int64), _nearest_int_brute(r))
    assert np.array_equal(sx.reshape(300), qx.astype(np.int64).sum(axis=1))
    # the scale: fp32 value within half an ulp of amax/127 (exact quotient in fp64)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    err = np.abs(dx.astype(np.float64) - amax / 127.0)
    assert np.all(err <= 0.5 * np.spacing(dx).astype(np.float64))


def test_quantize_invariants(orc):
    g = np.random.default_rng(12)
    x = g.standard_normal((4, 2048)).astype(np.float32)
    qx, dx, sx = orc.quantize_act_q8(x)
    q = qx.astype(np.int64).reshape(4, 64, 32)
    d = dx.astype(np.float64)
    xb = x.astype(np.float64).reshape(4, 64, 32)
    # the element of largest magnitude quantizes to +-127
    am = np.abs(xb).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(q, am[..., None], 2)) == 127)
    assert np.all(np.abs(q) <= 127)
    # reconstruction is within half a step (plus the fp32 quotient's rounding)
    assert np.all(np.abs(xb - d[..., None] * q) <= d[..., None] * (0.5 + 128 * 2.0 ** -23))
    # sign follows x
    assert np.all(np.sign(q) * np.sign(xb) >= 0)
    # negation and exact power-of-two scaling
    qn, dn, sn = orc.quantize_act_q8(-x)
    assert np.array_equal(qn, -qx) and np.array_equal(dn, dx) and np.array_equal(sn, -sx)
    for k in (-9, -1, 3, 12):
        qs, ds, ss = orc.quantize_act_q8(x * np.float32(2.0 ** k))
        assert np.array_equal(qs, qx) and np.array_equal(ss, sx)
        assert np.array_equal(ds, dx * np.float32(2.0 ** k))


def test_quantize_subnormal_scale_clamps(orc):
    """Worked by hand in units u = 2^-149 (the smallest fp32 subnormal): amax = 143u gives
    d = fl32(143u/127) = 1u (1.126u rounds down), so 143u/d = 143 and -140u/d = -140 must be
    clamped to +-127, while 100u/d = 100 is kept."""
    u = np.float32(2.0 ** -149)
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = np.array([143, -140, 100, 3], np.float32) * u
    qx, dx, sx = orc.quantize_act_q8(x)
    assert dx[0, 0] == u
    assert qx[0, :4].tolist() == [127, -127, 100, 3] and not qx[0, 4:].any()
    assert sx[0, 0] == 103


# ---------------------------------------------------------------- Q8_0

def test_q8_0_integer_special_case_is_exact_int_matmul(orc):
    """d = 1 and an integer activation whose blocks reach +-127 (scale 1, quants = x):
    the GEMV is an integer matmul, exact in int64."""
    g = np.random.default_rng(21)
    N, K, M = 37, 1024, 3
    q = g.integers(-127, 128, size=(N, K // 32, 32)).astype(np.int8)
    W = synth.q8_0_from_parts(np.ones((N, K // 32), np.float16), q)
    x = fh.integer_activation(g, M, K)
    qx, dx, sx = orc.quantize_act_q8(x)
    assert np.all(dx == 1.0) and np.array_equal(qx.astype(np.float32), x)
    y, bound = orc.gemv(orc.FMT_Q8_0, W, N, K, qx, dx)
    Wi = q.reshape(N, K).astype(np.int64)
    xi = x.astype(np.int64)
    assert np.array_equal(y, (xi @ Wi.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(xi) @ np.abs(Wi).T).astype(np.float64))


def test_q8_0_hand_block(orc):
    """N=1, K=32, d=0.5, q_i = i-16, qx_i = 2, dx = 0.25 -> y = -4, bound = 64 (by hand)."""
    q = (np.arange(32) - 16).astype(np.int8).reshape(1, 1, 32)
    W = synth.q8_0_from_parts(np.array([[0.5]], np.float16), q)
    assert W[0, 0] == 0x00 and W[0, 1] == 0x38  # fp16 0.5 = 0x3800, little endian
    y, bound = orc.gemv(orc.FMT_Q8_0, W, 1, 32, np.full((1, 32), 2, np.int8), np.array([[0.25]], np.float32))
    assert y[0, 0] == -4.0 and bound[0, 0] == 64.0


def test_q8_0_block_isums_exact(orc):
    g = np.random.default_rng(22)
    N, K, M = 9, 512, 2
    W = synth.q8_0_weight(g, N, K)
    qx, _, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    _, qw = fh.unpack_q8_0(W, N, K)
    ref = np.einsum("nbi,mbi->mnb", qw, qx.astype(np.int64).reshape(M, K // 32, 32))
    assert np.array_equal(orc.block_isums(orc.FMT_Q8_0, W, N, K, qx).astype(np.int64), ref)


def test_q8_0_general_vs_numpy_matmul(orc):
    g = np.random.default_rng(23)
    N, K, M = 45, 768, 3
    W = synth.q8_0_weight(g, N, K)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    Wd = fh.numpy_dequant_q8_0(W, N, K)
    assert np.array_equal(orc.dequant(orc.FMT_Q8_0, W, N, K), Wd)
    a = dx.astype(np.float64).repeat(32, axis=1) * qx.astype(np.float64)
    y, bound = orc.gemv(orc.FMT_Q8_0, W, N, K, qx, dx)
    assert np.all(np.abs(y - a @ Wd.T) <= 1e-12 * (np.abs(a) @ np.abs(Wd).T))
    assert np.allclose(bound, np.abs(a) @ np.abs(Wd).T, rtol=1e-13)


def test_gemv_fx_integer_special_case_is_exact_int_matmul(orc):
    """fp32 activation, no quantization: d = 1 and integer x (any magnitude that stays
    exact) make the product an int64 matmul."""
    g = np.random.default_rng(24)
    N, K, M = 29, 512, 3
    q = g.integers(-127, 128, size=(N, K // 32, 32)).astype(np.int8)
    W = synth.q8_0_from_parts(np.ones((N, K // 32), np.float16), q)
    xi = g.integers(-1000, 1001, size=(M, K))
    y, bound = orc.gemv_fx(orc.FMT_Q8_0, W, N, K, xi.astype(np.float32))
    Wi = q.reshape(N, K).astype(np.int64)
    assert np.array_equal(y, (xi @ Wi.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(xi) @ np.abs(Wi).T).astype(np.float64))


def test_gemv_fx_hand_block(orc):
    """N=1, K=32, d=0.5, q_i = i-16, x_i = 0.25*i -> y = 0.5*0.25*sum (i-16)*i = 0.125*2480 = 310."""
    q = (np.arange(32) - 16).astype(np.int8).reshape(1, 1, 32)
    W = synth.q8_0_from_parts(np.array([[0.5]], np.float16), q)
    x = (0.25 * np.arange(32)).astype(np.float32).reshape(1, 32)
    y, bound = orc.gemv_fx(orc.FMT_Q8_0, W, 1, 32, x)
    assert y[0, 0] == 310.0
    assert bound[0, 0] == 0.125 * float(np.sum(np.abs(np.arange(32) - 16) * np.arange(32)))


def test_gemv_fx_equals_gemv_on_a_representable_activation(orc):
    """x = dx*qx with power-of-two scales is exact in fp32, so the fp32-activation product
    equals the Q8-activation product term for term (both fp64)."""
    g = np.random.default_rng(25)
    N, K, M = 31, 1024, 2
    W = synth.q8_0_weight(g, N, K)
    qx = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    dx = (2.0 ** g.integers(-6, 3, size=(M, K // 32))).astype(np.float32)
    x = (dx.repeat(32, axis=1) * qx.astype(np.float32)).astype(np.float32)
    y1, b1 = orc.gemv_fx(orc.FMT_Q8_0, W, N, K, x)
    y2, b2 = orc.gemv(orc.FMT_Q8_0, W, N, K, qx, dx)
    assert np.all(np.abs(y1 - y2) <= 1e-13 * b2)
    assert np.allclose(b1, b2, rtol=1e-14, atol=0)


def test_gemv_fx_general_vs_numpy_matmul(orc):
    g = np.random.default_rng(26)
    N, K, M = 40, 768, 3
    W = synth.q8_0_weight(g, N, K)
    x = synth.activations(g, M, K)
    Wd = fh.numpy_dequant_q8_0(W, N, K)
    y, bound = orc.gemv_fx(orc.FMT_Q8_0, W, N, K, x)
    a = x.astype(np.float64)
    assert np.all(np.abs(y - a @ Wd.T) <= 1e-12 * (np.abs(a) @ np.abs(Wd).T))
    assert np.allclose(bound, np.abs(a) @ np.abs(Wd).T, rtol=1e-13)


def test_gemv_threads_do_not_change_result(orc):
    g = np.random.default_rng(24)
    N, K = 64, 512
    W = synth.q8_0_weight(g, N, K)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, 2, K))
    y1, b1 = orc.gemv(orc.FMT_Q8_0, W, N, K, qx, dx, nthreads=1)
    y4, b4 = orc.gemv(orc.FMT_Q8_0, W, N, K, qx, dx, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(b1, b4)


# ---------------------------------------------------------------- Q4_K

def _rand_fields(g, N, S):
    sc = g.integers(0, 64, size=(N, S, 8))
    m = g.integers(0, 64, size=(N, S, 8))
    q = g.integers(0, 16, size=(N, S, 8, 32))
    return sc, m, q


def test_q4k_nibble_order(orc):
    """d = 1, dmin = 0, every sub-scale 1: the weights are the nibbles themselves."""
    g = np.random.default_rng(31)
    N, S = 3, 2
    sc, m, q = _rand_fields(g, N, S)
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.zeros((N, S)), np.ones_like(sc), m, q)
    assert np.array_equal(orc.dequant(orc.FMT_Q4K, W, N, 256 * S), q.reshape(N, 256 * S).astype(np.float64))


def test_q4k_scale_and_min_fields(orc):
    """Every quant 1, d = 1, dmin = 0 reads back sc_j; d = 0, dmin = 1 reads back -m_j."""
    g = np.random.default_rng(32)
    N, S = 5, 3
    sc, m, _ = _rand_fields(g, N, S)
    ones = np.ones((N, S, 8, 32), np.int64)
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.zeros((N, S)), sc, m, ones)
    w = orc.dequant(orc.FMT_Q4K, W, N, 256 * S).reshape(N, S, 8, 32)
    assert np.array_equal(w, np.broadcast_to(sc[..., None], w.shape).astype(np.float64))
    W = fh.pack_q4k_matrix(np.zeros((N, S)), np.ones((N, S)), sc, m, ones)
    w = orc.dequant(orc.FMT_Q4K, W, N, 256 * S).reshape(N, S, 8, 32)
    assert np.array_equal(w, -np.broadcast_to(m[..., None], w.shape).astype(np.float64))


def test_q4k_minus_ones_closed_form(orc):
    """d = 0, dmin = 1, all mins 1: W = -1, so y = -sum_k dx*qx."""
    g = np.random.default_rng(33)
    N, S, M = 4, 4, 2
    sc, _, q = _rand_fields(g, N, S)
    W = fh.pack_q4k_matrix(np.zeros((N, S)), np.ones((N, S)), sc, np.ones((N, S, 8), int), q)
    K = 256 * S
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    y, _ = orc.gemv(orc.FMT_Q4K, W, N, K, qx, dx)
    a = (dx.astype(np.float64).repeat(32, axis=1) * qx).sum(axis=1)
    assert np.allclose(y, -a[:, None], rtol=1e-14, atol=0)


def test_q4k_integer_special_case_is_exact_int_matmul(orc):
    """d = 1, dmin = 0: W = sc*q is an integer matrix; with scale-1 activations y is exact."""
    g = np.random.default_rng(34)
    N, S, M = 6, 4, 3
    K = 256 * S
    sc, m, q = _rand_fields(g, N, S)
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.zeros((N, S)), sc, m, q)
    x = fh.integer_activation(g, M, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    y, _ = orc.gemv(orc.FMT_Q4K, W, N, K, qx, dx)
    Wi = (sc[..., None] * q).reshape(N, K).astype(np.int64)
    assert np.array_equal(y, (x.astype(np.int64) @ Wi.T).astype(np.float64))


def test_q4k_min_term_has_its_own_sign(orc):
    """Both terms at once: d = 1, dmin = 1 gives W = sc*q - m exactly (integers)."""
    g = np.random.default_rng(35)
    N, S = 4, 2
    sc, m, q = _rand_fields(g, N, S)
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.ones((N, S)), sc, m, q)
    want = (sc[..., None] * q - m[..., None]).reshape(N, 256 * S).astype(np.float64)
    assert np.array_equal(orc.dequant(orc.FMT_Q4K, W, N, 256 * S), want)


def test_q4k_block_isums_exact(orc):
    g = np.random.default_rng(36)
    N, K, M = 7, 1024, 2
    W = synth.q4k_weight(g, N, K)
    qx, _, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    _, _, _, _, q = fh.unpack_q4k_fields(W, N, K)
    ref = np.einsum("nbi,mbi->mnb", q.reshape(N, K // 32, 32), qx.astype(np.int64).reshape(M, K // 32, 32))
    assert np.array_equal(orc.block_isums(orc.FMT_Q4K, W, N, K, qx).astype(np.int64), ref)


def test_q4k_general_vs_numpy_matmul(orc):
    g = np.random.default_rng(37)
    N, K, M = 33, 1280, 2
    W = synth.q4k_weight(g, N, K)
    Wd = fh.numpy_dequant_q4k(W, N, K)
    assert np.allclose(orc.dequant(orc.FMT_Q4K, W, N, K), Wd, rtol=1e-15, atol=1e-18)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    a = dx.astype(np.float64).repeat(32, axis=1) * qx.astype(np.float64)
    y, bound = orc.gemv(orc.FMT_Q4K, W, N, K, qx, dx)
    ref = a @ Wd.T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(a) @ np.abs(Wd).T))
    assert np.allclose(bound, np.abs(a) @ np.abs(Wd).T, rtol=1e-12)


# ---------------------------------------------------------------- MoE table

def test_moe_table_matches_numpy_unique(orc):
    g = np.random.default_rng(41)
    for T, topk, E in [(1, 6, 256), (8, 6, 256), (64, 6, 384), (5, 3, 4), (9, 2, 7)]:
        ids = g.integers(0, E, size=(T, topk)).astype(np.int32)  # duplicates allowed
        tab = orc.moe_table(ids, E)
        uniq, inv = np.unique(ids.ravel(), return_inverse=True)
        assert tab["status"] == 0
        assert np.array_equal(tab["uniq"], uniq) and tab["n_uniq"] == len(uniq)
        assert np.array_equal(tab["slot"].ravel(), inv)
        order = np.argsort(inv, kind="stable")
        assert np.array_equal(tab["pairs"], order)
        counts = np.bincount(inv, minlength=len(uniq))
        assert np.array_equal(np.diff(tab["pair_off"]), counts) and tab["pair_off"][0] == 0


def test_moe_table_invalid_ids(orc):
    ids = np.array([[3, -1, 5], [7, 3, 1 << 30], [8, 0, 7]], np.int32)
    tab = orc.moe_table(ids, 8)
    assert tab["status"] == orc.BAD_EXPERT
    assert tab["uniq"].tolist() == [0, 3, 5, 7]
    assert tab["slot"].tolist() == [[1, -1, 2], [3, 1, -1], [-1, 0, 3]]
    assert tab["pairs"].tolist() == [7, 0, 4, 2, 3, 8]
    assert tab["pair_off"].tolist() == [0, 1, 3, 4, 6]


# ---------------------------------------------------------------- MoE end to end

def _small_moe(seed, T=5, topk=3, E=6, D=256, F=256):
    g = np.random.default_rng(seed)
    gate, up, down = synth.moe_experts(g, E, D, F)
    ids = synth.moe_ids_uniform(g, T, E, topk)
    rw = synth.routing_weights(g, T, topk)
    x = synth.activations(g, T, D)
    return gate, up, down, ids, rw, x


def test_moe_routed_single_expert_composition(orc):
    """T=1, top-1, weight 1: y = down . Q8(silu(gate . x) * (up . x)) of the chosen expert."""
    gate, up, down, _, _, x = _small_moe(51, T=1)
    D = F = 256
    qx, dx, _ = orc.quantize_act_q8(x)
    for e in (0, 4):
        y, _, st = orc.moe_routed(qx, dx, np.array([[e]]), np.ones((1, 1), np.float32), gate, up, down, D, F)
        gg, _ = orc.gemv(orc.FMT_Q4K, gate[e], F, D, qx, dx)
        vv, _ = orc.gemv(orc.FMT_Q4K, up[e], F, D, qx, dx)
        h = np.array([orc.silu(a) for a in gg[0]]) * vv[0]
        hq, hd, _ = orc.quantize_act_q8(h.astype(np.float32)[None])
        o, _ = orc.gemv(orc.FMT_Q4K, down[e], D, F, hq, hd)
        assert st == 0 and np.array_equal(y, o)


def test_moe_routed_weights_follow_their_slot(orc):
    """Two experts with weights 0.25 and 0.75: y = 0.25 o(e0) + 0.75 o(e1), where o(e) is the
    single-expert result (pinned above); a weight applied to the wrong slot fails this."""
    gate, up, down, _, _, x = _small_moe(54, T=1)
    D = F = 256
    qx, dx, _ = orc.quantize_act_q8(x)
    one = np.ones((1, 1), np.float32)
    o0, b0, _ = orc.moe_routed(qx, dx, np.array([[1]]), one, gate, up, down, D, F)
    o1, b1, _ = orc.moe_routed(qx, dx, np.array([[4]]), one, gate, up, down, D, F)
    y, _, st = orc.moe_routed(qx, dx, np.array([[1, 4]]), np.array([[0.25, 0.75]], np.float32),
                              gate, up, down, D, F)
    assert st == 0
    assert np.all(np.abs(y - (0.25 * o0 + 0.75 * o1)) <= 1e-14 * (b0 + b1))
    assert np.max(np.abs(y - (0.75 * o0 + 0.25 * o1))) > 1e-3 * np.max(b0 + b1) / D


def test_moe_routed_invariants(orc):
    gate, up, down, ids, rw, x = _small_moe(52)
    D = F = 256
    T = ids.shape[0]
    qx, dx, _ = orc.quantize_act_q8(x)
    y, bound, st = orc.moe_routed(qx, dx, ids, rw, gate, up, down, D, F)
    assert st == 0 and np.all(bound >= np.abs(y))
    # token permutation permutes rows exactly
    perm = np.array([3, 0, 4, 1, 2])
    yp, _, _ = orc.moe_routed(qx[perm], dx[perm], ids[perm], rw[perm], gate, up, down, D, F)
    assert np.array_equal(yp, y[perm])
    # relabelling the experts (ids and pointer tables together) changes nothing
    lab = np.array([5, 2, 0, 4, 1, 3])          # new id of old expert e is lab[e]
    inv = np.argsort(lab)
    yl, _, _ = orc.moe_routed(qx, dx, lab[ids], rw, [gate[i] for i in inv], [up[i] for i in inv],
                              [down[i] for i in inv], D, F)
    assert np.array_equal(yl, y)
    # doubling the routing weights doubles y exactly
    y2, _, _ = orc.moe_routed(qx, dx, ids, rw * 2, gate, up, down, D, F)
    assert np.array_equal(y2, 2 * y)
    # identical tokens give identical rows
    yd, _, _ = orc.moe_routed(np.repeat(qx[:1], 2, 0), np.repeat(dx[:1], 2, 0), np.repeat(ids[:1], 2, 0),
                              np.repeat(rw[:1], 2, 0), gate, up, down, D, F)
    assert np.array_equal(yd[0], yd[1]) and np.array_equal(yd[0], y[0])
    # the routing weights sum to one per token
    assert np.allclose(rw.sum(axis=1), 1.0, atol=1e-6)


def test_moe_routed_invalid_id_contributes_nothing(orc):
    gate, up, down, ids, rw, x = _small_moe(53)
    D = F = 256
    qx, dx, _ = orc.quantize_act_q8(x)
    bad = ids.copy()
    bad[2, 1] = -1
    y, _, st = orc.moe_routed(qx, dx, bad, rw, gate, up, down, D, F)
    assert st == orc.BAD_EXPERT
    rw0 = rw.copy()
    rw0[2, 1] = 0.0
    yz, _, st0 = orc.moe_routed(qx, dx, ids, rw0, gate, up, down, D, F)
    assert st0 == 0 and np.array_equal(y, yz)


# ---------------------------------------------------------------- prefill

def test_prefill_integer_special_case(orc):
    """d = 1, dmin = 0 and small-integer bf16 activations: Y is an exact integer matmul."""
    import torch
    g = np.random.default_rng(61)
    N, S, M = 5, 2, 4
    K = 256 * S
    sc, m, q = _rand_fields(g, N, S)
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.zeros((N, S)), sc, m, q)
    xi = g.integers(-100, 101, size=(M, K))
    xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Y, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb)
    Wi = (sc[..., None] * q).reshape(N, K).astype(np.int64)
    assert np.array_equal(Y, (xi @ Wi.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(xi) @ np.abs(Wi).T).astype(np.float64))


def test_prefill_general_vs_numpy_matmul(orc):
    import torch
    g = np.random.default_rng(62)
    N, K, M = 17, 768, 6
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    Wd = fh.numpy_dequant_q4k(W, N, K)
    Y, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb)
    assert np.all(np.abs(Y - x @ Wd.T) <= 1e-12 * (np.abs(x) @ np.abs(Wd).T))
    Y1, _ = orc.prefill(orc.FMT_Q4K, W, N, K, xb[2:3])
    assert np.array_equal(Y1[0], Y[2])


# ---------------------------------------------------------------- facts printed on the pages

def test_golden_q4k_expert_bytes(orc):
    """The pages give 13.50 MiB per Q4_K routed expert; with 144-byte superblocks of 256
    weights, gate + up (2048 x 4096) and down (4096 x 2048) come to exactly that."""
    with open(os.path.join(GOLDEN, "q4k_expert_bytes.json")) as f:
        fact = json.load(f)
    D, F = fact["hidden"], fact["expert_ffn"]
    total = 2 * F * orc.row_bytes(orc.FMT_Q4K, D) + D * orc.row_bytes(orc.FMT_Q4K, F)
    assert total == round(fact["MiB_per_expert"] * 2 ** 20)


def test_golden_expert_id_range(orc):
    """The pages show a decode with 256 experts failing on an expert id of -1, out of the range 0..256."""
    with open(os.path.join(GOLDEN, "expert_id_range.json")) as f:
        fact = json.load(f)
    E = fact["experts"]
    for bad in fact["invalid_ids"]:
        assert orc.moe_table(np.array([[bad, 0]], np.int32), E)["status"] == orc.BAD_EXPERT
    for ok in fact["valid_ids"]:
        assert orc.moe_table(np.array([[ok, 0]], np.int32), E)["status"] == 0


# ---------------------------------------------------------------- FP8 E4M3 / FP4 E2M1 expert formats

def _ocp():
    with open(os.path.join(GOLDEN, "ocp_fp8_fp4_values.json")) as f:
        return json.load(f)


def test_e4m3_all_codes_match_torch(orc):
    """Every E4M3 code decodes to what torch's float8_e4m3fn conversion gives (signed zeros too)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_and_ue8m0_landmarks_golden(orc):
    o = _ocp()
    for k, v in o["e4m3_landmarks"].items():
        assert orc.e4m3_to_double(int(k, 16)) == v, k
    for k in o["e4m3_nan_codes"]:
        assert math.isnan(orc.e4m3_to_double(int(k, 16)))
    for k, v in o["ue8m0_landmarks"].items():
        assert orc.ue8m0_to_double(int(k, 16)) == v, k
    for k in o["ue8m0_nan_codes"]:
        assert math.isnan(orc.ue8m0_to_double(int(k, 16)))


def test_e2m1_table_golden(orc):
    """The sixteen E2M1 codes decode to the MX specification's element values."""
    ref = _ocp()["e2m1_values_by_code"]
    for c in range(16):
        got = orc.e2m1_to_double(c)
        assert got == ref[c] and math.copysign(1.0, got) == math.copysign(1.0, ref[c]), c
    # only the low nibble is read
    assert orc.e2m1_to_double(0xF7) == 6.0


def test_ue8m0_all_codes_match_torch(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([orc.ue8m0_to_double(int(c)) for c in codes])
    assert np.array_equal(got, ref, equal_nan=True)


def _torch_decode_fp8(W, N, K):
    """Test-side decode of an FP8 E4M3 / 128 x 128 buffer through torch's float8 dtypes."""
    import torch
    codes = W[:N * K].reshape(N, K)
    off = (N * K + 255) // 256 * 256
    sc = W[off:off + (N + 127) // 128 * (K // 128)].reshape((N + 127) // 128, K // 128)
    v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = torch.from_numpy(sc.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return v * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:N]


def _table_decode_fp4(W, N, K):
    """Test-side decode of an FP4 E2M1 / 1 x 32 buffer through the MX value table."""
    import torch
    lut = np.array(_ocp()["e2m1_values_by_code"])
    codes = W[:N * K // 2].reshape(N, K // 2)
    off = (N * K // 2 + 255) // 256 * 256
    sc = W[off:off + N * (K // 32)].reshape(N, K // 32)
    nib = np.empty((N, K), np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    s = torch.from_numpy(sc.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return lut[nib] * np.repeat(s, 32, axis=1)


@pytest.mark.parametrize("fmt", [2, 3])
def test_scaled_formats_general_vs_independent_decode(orc, fmt):
    """Ragged rows (N not a multiple of 128), several scale blocks: the oracle's dequantized
    matrix equals the test-side decode exactly, and its GEMV equals numpy's matmul."""
    g = np.random.default_rng(60 + fmt)
    N, K, M = 300, 512, 3
    W = synth.weight(fmt, g, N, K)
    assert W.size == orc.matrix_bytes(fmt, N, K)
    ref = _torch_decode_fp8(W, N, K) if fmt == 2 else _table_decode_fp4(W, N, K)
    assert np.array_equal(orc.dequant(fmt, W, N, K), ref)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    a = dx.astype(np.float64).repeat(32, axis=1) * qx.astype(np.float64)
    y, bound = orc.gemv(fmt, W, N, K, qx, dx)
    assert np.all(np.abs(y - a @ ref.T) <= 1e-12 * (np.abs(a) @ np.abs(ref).T))
    assert np.allclose(bound, np.abs(a) @ np.abs(ref).T, rtol=1e-13)


def test_fp8_scale_blocks_are_row_by_column(orc):
    """Every code 1.0 (0x38) and every scale 2^0 except block (row block 1, column block 2) at
    2^3: exactly rows 128..255 x columns 256..383 read 8 (a transposed scale index fails)."""
    N, K = 300, 512
    codes = np.full((N, K), 0x38, np.uint8)
    sc = np.full((3, 4), 127, np.uint8)
    sc[1, 2] = 130
    w = orc.dequant(2, synth.fp8_from_parts(codes, sc), N, K)
    expect = np.ones((N, K))
    expect[128:256, 256:384] = 8.0
    assert np.array_equal(w, expect)


def test_fp4_nibble_order_and_scale_per_32(orc):
    """Byte 0x21 holds element 0 = code 1 (0.5) in its low nibble and element 1 = code 2 (1.0)
    in its high nibble; scale byte (row 1, block 1) = 2^2 multiplies exactly that block."""
    N, K = 2, 64
    codes = np.zeros((N, K // 2), np.uint8)
    codes[0, 0] = 0x21
    codes[1, 16] = 0x9F   # row 1, elements 32 (code 15: -6) and 33 (code 9: -0.5)
    sc = np.full((N, 2), 127, np.uint8)
    sc[1, 1] = 129
    w = orc.dequant(3, synth.fp4_from_parts(codes, sc), N, K)
    expect = np.zeros((N, K))
    expect[0, 0], expect[0, 1] = 0.5, 1.0
    expect[1, 32], expect[1, 33] = -24.0, -2.0
    assert np.array_equal(w, expect)


def test_scaled_formats_integer_case_is_exact(orc):
    """Codes whose values are integers (FP8: 1, 2, 4; FP4: 1, 2, 4, 6), scale 2^0, integer
    activation with dx = 1: the GEMV is an int64 matmul."""
    g = np.random.default_rng(64)
    N, K, M = 130, 256, 2
    x = fh.integer_activation(g, M, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    assert np.all(dx == 1.0)
    xi = x.astype(np.int64)
    # FP8: 0x38 = 1, 0x40 = 2, 0x48 = 4, and their negatives with the sign bit
    pick = g.integers(0, 6, size=(N, K))
    fp8_codes = np.array([0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], np.uint8)[pick]
    fp8_vals = np.array([1, 2, 4, -1, -2, -4], np.int64)[pick]
    W8 = synth.fp8_from_parts(fp8_codes, np.full((2, 2), 127, np.uint8))
    y8, _ = orc.gemv(2, W8, N, K, qx, dx)
    assert np.array_equal(y8, (xi @ fp8_vals.T).astype(np.float64))
    # FP4: codes 2 (1), 4 (2), 6 (4), 7 (6), 10 (-1), 15 (-6)
    pick = g.integers(0, 6, size=(N, K))
    nib = np.array([2, 4, 6, 7, 10, 15], np.uint8)[pick]
    fp4_vals = np.array([1, 2, 4, 6, -1, -6], np.int64)[pick]
    W4 = synth.fp4_from_parts((nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8),
                              np.full((N, K // 32), 127, np.uint8))
    y4, _ = orc.gemv(3, W4, N, K, qx, dx)
    assert np.array_equal(y4, (xi @ fp4_vals.T).astype(np.float64))


@pytest.mark.parametrize("fmt", [2, 3])
def test_moe_routed_scaled_format_composition(orc, fmt):
    """The routed MoE on FP8 / FP4 experts composes like the Q4_K one: top-1 with weight 1
    gives down . Q8(silu(gate . x) * (up . x)) of the chosen expert in that format."""
    g = np.random.default_rng(70 + fmt)
    E, D, F = 4, 256, 512
    gate, up, down = synth.moe_experts(g, E, D, F, fmt=fmt)
    x = synth.activations(g, 1, D)
    qx, dx, _ = orc.quantize_act_q8(x)
    e = 2
    y, _, st = orc.moe_routed(qx, dx, np.array([[e]]), np.ones((1, 1), np.float32), gate, up, down, D, F,
                              fmt=fmt)
    gg, _ = orc.gemv(fmt, gate[e], F, D, qx, dx)
    vv, _ = orc.gemv(fmt, up[e], F, D, qx, dx)
    h = np.array([orc.silu(a) for a in gg[0]]) * vv[0]
    hq, hd, _ = orc.quantize_act_q8(h.astype(np.float32)[None])
    o, _ = orc.gemv(fmt, down[e], D, F, hq, hd)
    assert st == 0 and np.array_equal(y, o)
