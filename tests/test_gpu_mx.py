"""GPU parity of the block-scaled expert formats -- FP8 E4M3 with 128 x 128 UE8M0
block scales and FP4 E2M1 with 1 x 32 UE8M0 scales -- as a dense mat-vec (qgemv_mx)
and on the routed-MoE path (moe_routed_qgemv_fmt), called through the C ABI.

Expected values come from the CPU oracle on the same seeded inputs.  fp32
outputs: |y - y_oracle| <= 1e-5 * sum_k |w_k x_k|; cases whose exact result is
representable (integer activations with scale 1, one code or one scale per
row) are compared exactly.
"""
import numpy as np
import pytest

import synth
from tests import fmt_helpers as fh
from tests.gpu_util import assert_within_bound, dev, empty, host, oracle_threads, progress, sentinel
from tests.test_gpu_moe import ONE_TOKEN_CASES, MoeProblem, check_staged, one_token_table_case

pytestmark = pytest.mark.gpu

FMTS = [2, 3]  # FP8 E4M3 128x128, FP4 E2M1 1x32


@pytest.fixture(scope="module")
def qg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_moe_matvec_amd as qg
    return qg


def _run(qg, fmt, W, N, K, qx, dx, M):
    import torch
    y = sentinel((M, N), torch.float32, 4321.0)
    qg.qgemv_mx(fmt, W, N, K, qx, dx, M, y)
    return host(y)


MX_CASES = [
    # N, K, M: one chunk per lane or fewer (masked lanes), ragged 128-row scale
    # blocks, the expert shapes, a row length whose chunks do not fill the last
    # load (7168), the largest K, the largest batch (tokens staged in chunks)
    (37, 256, 1),
    (129, 1280, 4),
    (300, 512, 3),
    (2048, 4096, 1),
    (4096, 2048, 2),
    (130, 7168, 2),
    (64, 16384, 5),
    (1000, 2048, 32),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", MX_CASES)
def test_mx_parity(qg, orc, fmt, N, K, M):
    progress("mx fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))
    g = np.random.default_rng(5000 + 10 * fmt + N + K + M)
    W = synth.weight(fmt, g, N, K)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    y = _run(qg, fmt, dev(W), N, K, dev(qx), dev(dx), M)
    ref, bound = orc.gemv(fmt, W, N, K, qx, dx, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="mx fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))


def test_mx_every_fp8_code_decodes_exactly(qg, orc):
    """Row r holds code r everywhere (NaN codes left out), scale 2^0, an integer activation
    with unit Q8 scale: y[r] = e4m3(r) * sum(x) exactly (the device reads OCP E4M3)."""
    K = 512
    codes = np.array([c for c in range(256) if c not in synth.E4M3_NAN_CODES], np.uint8)
    N = codes.size
    W = synth.fp8_from_parts(np.repeat(codes[:, None], K, axis=1), np.full(((N + 127) // 128, K // 128), 127,
                                                                                np.uint8))
    x = fh.integer_activation(np.random.default_rng(81), 2, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    assert np.all(dx == 1.0)
    y = _run(qg, 2, dev(W), N, K, dev(qx), dev(dx), 2)
    vals = np.array([orc.e4m3_to_double(int(c)) for c in codes])
    ref = vals[None, :] * x.astype(np.float64).sum(axis=1)[:, None]
    assert np.array_equal(y.astype(np.float64), ref)


def test_mx_every_fp4_code_decodes_exactly(qg, orc):
    """Row r holds nibble r in both halves of every byte, scale 2^0: y[r] = e2m1(r) * sum(x)."""
    K = 512
    N = 16
    codes = np.repeat((np.arange(16, dtype=np.uint8) * 17)[:, None], K // 2, axis=1)
    W = synth.fp4_from_parts(codes, np.full((N, K // 32), 127, np.uint8))
    x = fh.integer_activation(np.random.default_rng(82), 3, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    y = _run(qg, 3, dev(W), N, K, dev(qx), dev(dx), 3)
    vals = np.array([orc.e2m1_to_double(c) for c in range(16)])
    assert np.array_equal(y.astype(np.float64), vals[None, :] * x.astype(np.float64).sum(axis=1)[:, None])


def test_mx_nibble_order_on_device(qg, orc):
    """Only element 0 of each 32-block is 0.5 (low nibble of its first byte): a swapped
    nibble order would multiply element 1 of the activation instead."""
    N, K = 8, 256
    codes = np.zeros((N, K // 2), np.uint8)
    codes[:, ::16] = 0x01
    W = synth.fp4_from_parts(codes, np.full((N, K // 32), 127, np.uint8))
    x = fh.integer_activation(np.random.default_rng(83), 1, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    y = _run(qg, 3, dev(W), N, K, dev(qx), dev(dx), 1)
    assert np.all(y[0] == 0.5 * x[0, ::32].astype(np.float64).sum())


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_scale_structure_exact(qg, orc, fmt):
    """Every code 1.0, a different power-of-two scale per block (per 128 x 128 for FP8, per
    row and 32 columns for FP4), integer activation: the result is exact, so it must equal
    the oracle bit for bit (a transposed or shifted scale index fails)."""
    g = np.random.default_rng(90 + fmt)
    N, K, M = 300, 1024, 2
    if fmt == 2:
        W = synth.fp8_from_parts(np.full((N, K), 0x38, np.uint8),
                                 g.integers(124, 131, size=((N + 127) // 128, K // 128)).astype(np.uint8))
    else:
        W = synth.fp4_from_parts(np.full((N, K // 2), 0x22, np.uint8),
                                 g.integers(124, 131, size=(N, K // 32)).astype(np.uint8))
    x = fh.integer_activation(g, M, K)
    qx, dx, _ = orc.quantize_act_q8(x)
    y = _run(qg, fmt, dev(W), N, K, dev(qx), dev(dx), M)
    ref, _ = orc.gemv(fmt, W, N, K, qx, dx)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_wide_scale_range(qg, orc, fmt):
    """Scales across 2^-67 .. 2^63 and activations across 2^-20 .. 2^20 per token."""
    g = np.random.default_rng(95 + fmt)
    N, K, M = 500, 2048, 3
    W = synth.fp8_weight(g, N, K, 60, 190) if fmt == 2 else synth.fp4_weight(g, N, K, 60, 190)
    x = synth.activations(g, M, K) * np.array([2.0 ** -20, 1.0, 2.0 ** 20], np.float32)[:, None]
    qx, dx, _ = orc.quantize_act_q8(x)
    y = _run(qg, fmt, dev(W), N, K, dev(qx), dev(dx), M)
    ref, bound = orc.gemv(fmt, W, N, K, qx, dx)
    assert np.all(np.isfinite(ref))
    assert_within_bound(y, ref, bound, what="mx wide scales fmt=%d" % fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_batch_rows_equal_single_token_calls(qg, orc, fmt):
    g = np.random.default_rng(97 + fmt)
    N, K, M = 700, 4096, 9
    Wd = dev(synth.weight(fmt, g, N, K))
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    qxd, dxd = dev(qx), dev(dx)
    y = _run(qg, fmt, Wd, N, K, qxd, dxd, M)
    for t in range(M):
        one = _run(qg, fmt, Wd, N, K, qxd[t:t + 1], dxd[t:t + 1], 1)
        assert np.array_equal(y[t].view(np.uint32), one[0].view(np.uint32)), t


def test_mx_errors_leave_outputs_untouched(qg):
    import torch
    W = dev(synth.fp4_weight(np.random.default_rng(1), 16, 512))
    qx = dev(np.zeros((1, 512), np.int8))
    dx = dev(np.ones((1, 16), np.float32))
    y = sentinel((1, 16), torch.float32, 5.0)
    c = qg._c_mx
    assert c(1, W.data_ptr(), 16, 512, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None) == -4
    assert c(3, W.data_ptr(), 16, 500, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None) == -2
    assert c(3, W.data_ptr(), 16, 512, None, dx.data_ptr(), 1, y.data_ptr(), None) == -1
    assert c(3, W.data_ptr() + 8, 16, 512, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None) == -3
    torch.cuda.synchronize()
    assert np.all(host(y) == 5.0)


# ---------------------------------------------------------------- routed MoE

@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_small_staged_and_end_to_end(qg, orc, fmt):
    for (E, D, F, T, topk, seed) in [(16, 512, 256, 1, 6, 1), (16, 512, 256, 3, 6, 2), (10, 768, 512, 8, 4, 3),
                                     (8, 256, 256, 9, 8, 4)]:
        progress("moe mx fmt=%d E=%d D=%d F=%d T=%d topk=%d" % (fmt, E, D, F, T, topk))
        pb = MoeProblem(qg, E, D, F, T, topk, seed, fmt=fmt)
        y, ws, st = pb.run()
        assert st == 0
        check_staged(qg, orc, pb, y, ws)
        ye, be, ste = orc.moe_routed(host(pb.qx), host(pb.dx), pb.ids, pb.rw, pb.gate, pb.up, pb.down, D, F,
                                     nthreads=oracle_threads(), fmt=fmt)
        assert ste == 0
        assert_within_bound(y, ye, be, rel=1e-3, what="end-to-end fmt=%d" % fmt)


@pytest.mark.parametrize("name", ["moe_fp8_e256_t1", "moe_fp4_e384_t1"])
def test_moe_mx_full_size_t1(qg, orc, name):
    """The expert-format workloads at full size (gate/up 4096 -> 2048, down 2048 -> 4096),
    top-6 of 256 (FP8) or 384 (FP4) experts, one token; unselected experts are NULL."""
    w = synth.WORKLOADS[name]
    progress("moe mx full %s" % name)
    pb = MoeProblem(qg, w["E"], w["D"], w["F"], w["T"], w["topk"], w["seed"], only_selected=True, fmt=w["fmt"])
    y, ws, st = pb.run()
    assert st == 0
    check_staged(qg, orc, pb, y, ws)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ONE_TOKEN_CASES)
def test_moe_mx_one_token_table_and_status(qg, orc, fmt, case):
    """The expert formats with one token (the table built in the gate/up launch): table, status
    and dropped pairs as for Q4_K experts."""
    one_token_table_case(qg, orc, case, fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_gate_equals_dense_call(qg, fmt):
    """The routed gate GEMV and qgemv_mx share one engine: g is bit-equal to the dense call."""
    import torch
    pb = MoeProblem(qg, 12, 1024, 512, 4, 3, 7, fmt=fmt)
    y, ws, st = pb.run()
    assert st == 0
    R = pb.regions(ws)
    for p in range(pb.T * pb.topk):
        t, e = p // pb.topk, int(pb.ids.ravel()[p])
        out = torch.empty(1, pb.F, dtype=torch.float32, device="cuda")
        qg.qgemv_mx(fmt, pb.dgate[e], pb.F, pb.D, pb.qx[t:t + 1], pb.dx[t:t + 1], 1, out)
        assert np.array_equal(host(out)[0].view(np.uint32), R["g"][p].view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_invalid_id(qg, fmt):
    pb = MoeProblem(qg, 16, 512, 256, 4, 6, 13, fmt=fmt)
    base, _, st0 = pb.run()
    assert st0 == 0
    ids = pb.ids.copy()
    ids[2, 3] = -1
    y, ws, st = pb.run(ids=ids)
    assert st == qg.DEV_BAD_EXPERT
    rw0 = pb.rw.copy()
    rw0[2, 3] = 0.0
    yz, _, _ = pb.run(rw=rw0)
    assert np.array_equal(y[2], yz[2])
    for t in (0, 1, 3):
        assert np.array_equal(y[t], base[t])
