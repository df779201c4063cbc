"""GPU parity of the activation quantizer and the dense decode mat-vecs.

The HIP library is called through its C ABI (the ctypes binding); expected
values come only from the CPU oracle on the same seeded inputs.
Bit-exact: qx/dx/sx and the per-block integer sums.  fp32 outputs:
|y - y_oracle| <= 1e-5 * sum_k |w_k x_k| per output.
"""
import numpy as np
import pytest

import synth
from tests import fmt_helpers as fh
from tests.gpu_util import assert_within_bound, dev, empty, host, oracle_threads, progress, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_moe_matvec_amd as qg
    return qg


def gpu_quantize(qg, x: np.ndarray):
    import torch
    M, K = x.shape
    xd = dev(x.astype(np.float32))
    qx = empty((M, K), torch.int8)
    dx = empty((M, K // 32), torch.float32)
    sx = empty((M, K // 32), torch.int32)
    qg.quantize_act_q8(xd, M, K, qx, dx, sx)
    return qx, dx, sx


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("M,K", [(1, 32), (1, 1024), (3, 4096), (8, 8192), (5, 2080)])
def test_quantize_bit_exact(qg, orc, M, K):
    progress("quantize M=%d K=%d" % (M, K))
    g = np.random.default_rng(100 + M * 7 + K)
    x = synth.activations(g, M, K) * np.float32(10.0) ** g.integers(-3, 4, size=(M, 1)).astype(np.float32)
    nb = K // 32
    # special blocks: all zero, exact ties at scale 1, subnormal scale, single spike
    if nb >= 4:
        x[0, 0:32] = 0.0
        x[0, 32:64] = np.array([127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5] * 4, np.float32)
        x[0, 64:96] = np.float32(2.0 ** -149) * np.arange(-16, 16, dtype=np.float32) * 9
        x[0, 96:128] = 0.0
        x[0, 100] = -3.7
    qx, dx, sx = gpu_quantize(qg, x)
    rq, rd, rs = orc.quantize_act_q8(x)
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(host(dx).view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(host(sx), rs)


def test_quantize_errors(qg):
    import torch
    x = dev(np.zeros((1, 64), np.float32))
    qx, dx, sx = empty((1, 64), torch.int8), empty((1, 2), torch.float32), empty((1, 2), torch.int32)
    with pytest.raises(qg.QGError) as e:
        qg.quantize_act_q8(x, 1, 48, qx, dx, sx)
    assert e.value.status == -2
    with pytest.raises(qg.QGError) as e:
        qg.quantize_act_q8(x, 0, 64, qx, dx, sx)
    assert e.value.status == -2
    assert qg._c_quantize(x.data_ptr(), 1, 64, None, dx.data_ptr(), sx.data_ptr(), None) == -1
    assert qg._c_quantize(x.data_ptr() + 4, 1, 32, qx.data_ptr(), dx.data_ptr(), sx.data_ptr(), None) == -3


# ---------------------------------------------------------------- GEMV parity

def _weights(fmt, g, N, K):
    return synth.q8_0_weight(g, N, K) if fmt == 0 else synth.q4k_weight(g, N, K)


def _run_gemv(qg, fmt, W, N, K, qx, dx, sx, M):
    import torch
    y = sentinel((M, N), torch.float32, 12345.0)
    if fmt == 0:
        qg.qgemv_q8_0(W, N, K, qx, dx, M, y)
    else:
        qg.qgemv_q4k(W, N, K, qx, dx, sx, M, y)
    return host(y)


GEMV_CASES = [
    # fmt, N, K, M : the 512x1024 Q8_0 workload, ragged tiles, non-power-of-two
    # groups per row, the largest K, odd batch sizes
    (0, 512, 1024, 1),
    (0, 37, 256, 1),
    (0, 100, 1280, 3),
    (0, 9, 12288, 2),
    (0, 64, 16384, 1),
    (0, 333, 2048, 9),
    (1, 77, 4096, 1),
    (1, 50, 1792, 4),
    (1, 19, 16384, 2),
    (1, 130, 256, 33 - 1),
]


@pytest.mark.parametrize("fmt,N,K,M", GEMV_CASES)
def test_gemv_parity_small(qg, orc, fmt, N, K, M):
    progress("gemv fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))
    g = np.random.default_rng(1000 + fmt * 100 + N + K + M)
    W = _weights(fmt, g, N, K)
    x = synth.activations(g, M, K)
    qx, dx, sx = gpu_quantize(qg, x)
    y = _run_gemv(qg, fmt, dev(W), N, K, qx, dx, sx, M)
    ref, bound = orc.gemv(fmt, W, N, K, host(qx), host(dx), nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="gemv fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))


def test_q8_0_out_projection_full_size(qg, orc):
    """The 8192 -> 4096 Q8_0 output projection, batch 1, every output vs the oracle."""
    progress("q8_0 4096x8192 full")
    w = synth.WORKLOADS["q8_0_out_4096x8192"]
    g = synth.rng(w["seed"])
    N, K = w["N"], w["K"]
    W = synth.q8_0_weight(g, N, K)
    x = synth.activations(g, 1, K)
    qx, dx, sx = gpu_quantize(qg, x)
    y = _run_gemv(qg, 0, dev(W), N, K, qx, dx, sx, 1)
    ref, bound = orc.gemv(0, W, N, K, host(qx), host(dx), nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="q8_0 4096x8192")


def test_q4k_projection_full_size(qg, orc):
    """The 4096 -> 8192 Q4_K projection, batch 1, every output vs the oracle."""
    progress("q4k 8192x4096 full")
    w = synth.WORKLOADS["q4k_8192x4096"]
    g = synth.rng(w["seed"])
    N, K = w["N"], w["K"]
    W = synth.q4k_weight(g, N, K)
    x = synth.activations(g, 1, K)
    qx, dx, sx = gpu_quantize(qg, x)
    y = _run_gemv(qg, 1, dev(W), N, K, qx, dx, sx, 1)
    ref, bound = orc.gemv(1, W, N, K, host(qx), host(dx), nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="q4k 8192x4096")


def test_batched_sweep_full_size(qg, orc):
    """Q8_0 4096 -> 16384 at M = 1..32: each row of a batched call equals the M = 1 call on
    that token bit for bit; every output of every batch matches the oracle."""
    progress("q8_0 16384x4096 batched sweep")
    w = synth.WORKLOADS["q8_0_16384x4096"]
    g = synth.rng(w["seed"])
    N, K = w["N"], w["K"]
    W = synth.q8_0_weight(g, N, K)
    Wd = dev(W)
    x = synth.activations(g, 32, K)
    qx, dx, sx = gpu_quantize(qg, x)
    singles = [_run_gemv(qg, 0, Wd, N, K, qx[t:t + 1], dx[t:t + 1], sx[t:t + 1], 1) for t in range(32)]
    # the oracle's rows are independent per token: one call covers the prefixes of every batch
    Mmax = max(w["Ms"])
    ref, bound = orc.gemv(0, W, N, K, host(qx[:Mmax]), host(dx[:Mmax]), nthreads=oracle_threads())
    for M in w["Ms"]:
        y = _run_gemv(qg, 0, Wd, N, K, qx[:M], dx[:M], sx[:M], M)
        for t in range(M):
            assert np.array_equal(y[t], singles[t][0]), "batch invariance M=%d t=%d" % (M, t)
        assert_within_bound(y, ref[:M], bound[:M], what="batched M=%d" % M)


def test_paired_equals_two_singles_and_oracle(qg, orc):
    """One quantized 4096-vector feeds 4096->1024 and 4096->512 in one launch."""
    progress("paired 1024+512 x 4096")
    w = synth.WORKLOADS["q8_0_pair_1024+512x4096"]
    g = synth.rng(w["seed"])
    K, N1, N2 = w["K"], w["N1"], w["N2"]
    for fmt in (0, 1):
        W1, W2 = _weights(fmt, g, N1, K), _weights(fmt, g, N2, K)
        x = synth.activations(g, 12, K)
        qx, dx, sx = gpu_quantize(qg, x)
        import torch
        for M in (1, 2, 8, 12):
            y1, y2 = sentinel((M, N1), torch.float32), sentinel((M, N2), torch.float32)
            qg.qgemv_paired(fmt, dev(W1), N1, dev(W2), N2, K, qx[:M], dx[:M], sx[:M], M, y1, y2)
            s1 = _run_gemv(qg, fmt, dev(W1), N1, K, qx[:M], dx[:M], sx[:M], M)
            s2 = _run_gemv(qg, fmt, dev(W2), N2, K, qx[:M], dx[:M], sx[:M], M)
            assert np.array_equal(host(y1), s1) and np.array_equal(host(y2), s2)
            r1, b1 = orc.gemv(fmt, W1, N1, K, host(qx[:M]), host(dx[:M]))
            r2, b2 = orc.gemv(fmt, W2, N2, K, host(qx[:M]), host(dx[:M]))
            assert_within_bound(host(y1), r1, b1, what="paired y1")
            assert_within_bound(host(y2), r2, b2, what="paired y2")


# ---------------------------------------------------------------- Q8_0 batches on the matrix cores

MM_CASES = [
    # N, K, M: one group per row; empty K slices; partial slices of two, four
    # and eight groups (K = 1280, 2304: groups per row not a power of two, with
    # enough rows that a workgroup takes few slices); the 8-block unit (K > 8192)
    # with a partial slice; the largest K; ragged row tiles; 4..32 tokens
    # (batched calls of fewer than 8 tokens run the dot-product engine, so each
    # case also runs qgemm_q8_0, which always takes the matrix cores)
    (37, 256, 4),
    (100, 1280, 5),
    (16384, 1280, 8),
    (32768, 1280, 6),
    (32768, 2304, 5),
    (333, 2048, 9),
    (70, 7168, 17),
    (9, 8448, 7),
    (9, 12288, 32),
    (64, 16384, 16),
    (4096, 4096, 32),
]


@pytest.mark.parametrize("N,K,M", MM_CASES)
def test_q8_0_batch_rows_equal_single_token_calls(qg, orc, N, K, M):
    """A batch of M Q8_0 tokens: every row equals the one-token call on that token, bit for
    bit, and sampled rows match the oracle; the matrix-core form (qgemm_q8_0) gives the
    same bits."""
    import torch
    progress("q8_0 batch N=%d K=%d M=%d" % (N, K, M))
    g = np.random.default_rng(4000 + N + K + M)
    W = synth.q8_0_weight(g, N, K)
    Wd = dev(W)
    qx, dx, sx = gpu_quantize(qg, synth.activations(g, M, K))
    y = _run_gemv(qg, 0, Wd, N, K, qx, dx, sx, M)
    ymm = sentinel((M, N), torch.float32)
    qg.qgemm_q8_0(Wd, N, K, qx, dx, M, ymm)
    assert np.array_equal(host(ymm).view(np.uint32), y.view(np.uint32)), "qgemm_q8_0 vs batched call"
    for t in range(M):
        single = _run_gemv(qg, 0, Wd, N, K, qx[t:t + 1], dx[t:t + 1], sx[t:t + 1], 1)
        assert np.array_equal(y[t].view(np.uint32), single[0].view(np.uint32)), "token %d" % t
    ref, bound = orc.gemv(0, W, N, K, host(qx), host(dx), nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="q8_0 batch N=%d K=%d M=%d" % (N, K, M))


MM_Q4K_CASES = [
    # N, K, M: Q4_K batches on the matrix cores (9 tokens and more): one
    # superblock per row; groups per row not a power of two (partial and empty
    # K slices); the largest K; ragged row and token tiles
    (37, 256, 9),
    (100, 1280, 12),
    (16384, 1280, 9),
    (32768, 2304, 10),
    (70, 7168, 17),
    (9, 12288, 32),
    (64, 16384, 16),
    (8192, 4096, 32),
]


@pytest.mark.parametrize("N,K,M", MM_Q4K_CASES)
def test_q4k_batch_rows_equal_single_token_calls(qg, orc, N, K, M):
    """A batch of M Q4_K tokens: every row equals the one-token call on that token, bit for
    bit, and sampled rows match the oracle."""
    progress("q4k batch N=%d K=%d M=%d" % (N, K, M))
    g = np.random.default_rng(7000 + N + K + M)
    W = synth.q4k_weight(g, N, K)
    Wd = dev(W)
    qx, dx, sx = gpu_quantize(qg, synth.activations(g, M, K))
    y = _run_gemv(qg, 1, Wd, N, K, qx, dx, sx, M)
    for t in range(M):
        single = _run_gemv(qg, 1, Wd, N, K, qx[t:t + 1], dx[t:t + 1], sx[t:t + 1], 1)
        assert np.array_equal(y[t].view(np.uint32), single[0].view(np.uint32)), "token %d" % t
    ref, bound = orc.gemv(1, W, N, K, host(qx), host(dx), nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="q4k batch N=%d K=%d M=%d" % (N, K, M))


@pytest.mark.parametrize("fmt,N,K,M", [(0, 45, 1024, 2), (0, 8, 12288, 1), (1, 33, 2048, 3), (1, 5, 256, 1)])
def test_block_isums_bit_exact(qg, orc, fmt, N, K, M):
    import torch
    progress("isums fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))
    g = np.random.default_rng(2000 + fmt + N + K)
    W = _weights(fmt, g, N, K)
    qx, _, _ = gpu_quantize(qg, synth.activations(g, M, K))
    isum = sentinel((M, N, K // 32), torch.int32)
    qg.qgemv_debug_block_isums(fmt, dev(W), N, K, qx, M, isum)
    assert np.array_equal(host(isum), orc.block_isums(fmt, W, N, K, host(qx)))


def test_integer_weights_are_exact(qg):
    """d = 1 Q8_0 weights and a scale-1 integer activation: every partial sum is an
    integer below 2^24, so the fp32 result equals the int64 matmul exactly."""
    g = np.random.default_rng(31)
    N, K, M = 70, 1024, 2
    q = g.integers(-40, 41, size=(N, K // 32, 32)).astype(np.int8)
    W = synth.q8_0_from_parts(np.ones((N, K // 32), np.float16), q)
    x = fh.integer_activation(g, M, K)
    qx, dx, sx = gpu_quantize(qg, x)
    assert np.all(host(dx) == 1.0)
    y = _run_gemv(qg, 0, dev(W), N, K, qx, dx, sx, M)
    assert np.array_equal(y.astype(np.float64), (x.astype(np.int64) @ q.reshape(N, K).astype(np.int64).T))


def test_zero_weights_give_exact_zero(qg):
    N, K = 16, 512
    W = synth.q8_0_from_parts(np.zeros((N, K // 32), np.float16), np.ones((N, K // 32, 32), np.int8))
    qx, dx, sx = gpu_quantize(qg, synth.activations(np.random.default_rng(3), 1, K))
    y = _run_gemv(qg, 0, dev(W), N, K, qx, dx, sx, 1)
    assert np.all(y == 0.0)


def test_deterministic_across_calls(qg):
    g = np.random.default_rng(77)
    N, K = 1000, 4096
    for fmt in (0, 1):
        Wd = dev(_weights(fmt, g, N, K))
        qx, dx, sx = gpu_quantize(qg, synth.activations(g, 4, K))
        a = _run_gemv(qg, fmt, Wd, N, K, qx, dx, sx, 4)
        b = _run_gemv(qg, fmt, Wd, N, K, qx, dx, sx, 4)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gemv_errors_leave_outputs_untouched(qg):
    import torch
    g = np.random.default_rng(5)
    N, K = 8, 512
    Wd = dev(synth.q8_0_weight(g, N, K))
    qx, dx, sx = gpu_quantize(qg, synth.activations(g, 2, K))
    y = sentinel((2, N), torch.float32, 3.0)
    cases = [
        (lambda: qg._c_q8_0(Wd.data_ptr(), N, 300, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None), -2),
        (lambda: qg._c_q8_0(Wd.data_ptr(), N, K, qx.data_ptr(), dx.data_ptr(), 0, y.data_ptr(), None), -2),
        (lambda: qg._c_q8_0(Wd.data_ptr(), N, K, qx.data_ptr(), dx.data_ptr(), 33, y.data_ptr(), None), -2),
        (lambda: qg._c_q8_0(Wd.data_ptr(), 0, K, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None), -2),
        (lambda: qg._c_q8_0(Wd.data_ptr(), N, 32768, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None), -2),
        (lambda: qg._c_q8_0(None, N, K, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None), -1),
        (lambda: qg._c_q8_0(Wd.data_ptr(), N, K, qx.data_ptr(), dx.data_ptr(), 1, None, None), -1),
        (lambda: qg._c_q8_0(Wd.data_ptr() + 2, N, K, qx.data_ptr(), dx.data_ptr(), 1, y.data_ptr(), None), -3),
        (lambda: qg._c_q4k(Wd.data_ptr(), N, K, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None), -1),
        (lambda: qg._c_paired(7, Wd.data_ptr(), N, Wd.data_ptr(), N, K, qx.data_ptr(), dx.data_ptr(), None, 1,
                              y.data_ptr(), y.data_ptr(), None), -4),
    ]
    for fn, want in cases:
        assert fn() == want
    assert np.all(host(y) == 3.0)


# ---------------------------------------------------------------- fused quantization

@pytest.mark.parametrize("fmt,N,K,M", [(0, 4096, 8192, 1), (0, 300, 4096, 2), (1, 257, 4096, 1), (1, 70, 2048, 5),
                                       (0, 33, 12288, 1), (0, 130, 1024, 9)])
def test_fused_quantize_matches_two_step(qg, fmt, N, K, M):
    """qgemv_*_f32 quantizes in the kernel: y equals quantize_act_q8 + qgemv_* bit for bit, and
    the published Q8 activation equals quantize_act_q8's output."""
    import torch
    progress("fused fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))
    g = np.random.default_rng(3000 + fmt + N + K + M)
    W = dev(_weights(fmt, g, N, K))
    x = synth.activations(g, M, K) * np.float32(3.0)
    qx, dx, sx = gpu_quantize(qg, x)
    ref = _run_gemv(qg, fmt, W, N, K, qx, dx, sx, M)
    y = sentinel((M, N), torch.float32)
    pq, pd, ps = sentinel((M, K), torch.int8, 5), sentinel((M, K // 32), torch.float32), \
        sentinel((M, K // 32), torch.int32)
    f = qg.qgemv_q8_0_f32 if fmt == 0 else qg.qgemv_q4k_f32
    f(W, N, K, dev(x), M, y, pq, pd, ps)
    assert np.array_equal(host(y).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(host(pq), host(qx)) and np.array_equal(host(ps), host(sx))
    assert np.array_equal(host(pd).view(np.uint32), host(dx).view(np.uint32))
    y2 = sentinel((M, N), torch.float32)
    f(W, N, K, dev(x), M, y2)  # without publishing
    assert np.array_equal(host(y2).view(np.uint32), ref.view(np.uint32))


def test_fused_paired(qg):
    import torch
    g = np.random.default_rng(3100)
    K, N1, N2 = 4096, 1024, 512
    for fmt in (0, 1):
        W1, W2 = dev(_weights(fmt, g, N1, K)), dev(_weights(fmt, g, N2, K))
        x = synth.activations(g, 2, K)
        qx, dx, sx = gpu_quantize(qg, x)
        for M in (1, 2):
            y1, y2 = sentinel((M, N1), torch.float32), sentinel((M, N2), torch.float32)
            pq, pd, ps = empty((M, K), torch.int8), empty((M, K // 32), torch.float32), \
                empty((M, K // 32), torch.int32)
            qg.qgemv_paired_f32(fmt, W1, N1, W2, N2, K, dev(x[:M].copy()), M, y1, y2, pq, pd, ps)
            r1 = _run_gemv(qg, fmt, W1, N1, K, qx[:M], dx[:M], sx[:M], M)
            r2 = _run_gemv(qg, fmt, W2, N2, K, qx[:M], dx[:M], sx[:M], M)
            assert np.array_equal(host(y1), r1) and np.array_equal(host(y2), r2)
            assert np.array_equal(host(pq), host(qx[:M])) and np.array_equal(host(ps), host(sx[:M]))


def test_fused_errors(qg):
    import torch
    W = dev(synth.q8_0_weight(np.random.default_rng(1), 8, 512))
    y = sentinel((1, 8), torch.float32, 2.0)
    x = dev(np.zeros((1, 512), np.float32))
    assert qg._c_q8_0_f32(W.data_ptr(), 8, 512, None, 1, y.data_ptr(), None, None, None, None) == -1
    assert qg._c_q8_0_f32(W.data_ptr(), 8, 500, x.data_ptr(), 1, y.data_ptr(), None, None, None, None) == -2
    assert qg._c_q8_0_f32(W.data_ptr(), 8, 512, x.data_ptr() + 4, 1, y.data_ptr(), None, None, None, None) == -3
    assert np.all(host(y) == 2.0)


# ---------------------------------------------------------------- grouped (attention output, low rank)

@pytest.mark.parametrize("fmt,G,N,K,M", [(0, 8, 1024, 4096, 1), (0, 3, 130, 512, 3), (1, 2, 70, 1024, 2),
                                         (0, 1, 96, 256, 5), (1, 5, 33, 256, 1), (0, 8, 1024, 4096, 12),
                                         (1, 3, 100, 2048, 12)])
def test_grouped_parity(qg, orc, fmt, G, N, K, M):
    """Group g against the oracle on matrix g and input slice g; ragged N, G = 1, several tokens."""
    import torch
    progress("grouped fmt=%d G=%d N=%d K=%d M=%d" % (fmt, G, N, K, M))
    g_ = np.random.default_rng(900 + G * 7 + N + K + M + fmt)
    make = synth.q8_0_weight if fmt == 0 else synth.q4k_weight
    Ws = [make(g_, N, K) for _ in range(G)]
    x = synth.activations(g_, M, G * K)
    qx, dx, sx = orc.quantize_act_q8(x)
    y = sentinel((M, G * N), torch.float32, 99.0)
    qg.qgemv_grouped(fmt, dev(np.concatenate(Ws, axis=0)), G, N, K, dev(qx), dev(dx), dev(sx), M, y)
    yh = host(y).reshape(M, G, N)
    nt = oracle_threads()
    for g in range(G):
        sl = slice(g * K, (g + 1) * K)
        ref, bound = orc.gemv(fmt, Ws[g], N, K, qx[:, sl].copy(), dx[:, g * K // 32:(g + 1) * K // 32].copy(),
                              nthreads=nt)
        assert_within_bound(yh[:, g], ref, bound, what="grouped g=%d" % g)


def test_grouped_equals_single_calls(qg):
    """Each group equals the single-matrix call on its slice, bit for bit."""
    g_ = np.random.default_rng(31)
    for fmt, G, N, K, M in ((0, 4, 200, 1024, 2), (0, 3, 100, 2048, 9), (1, 3, 70, 1280, 11)):
        _grouped_equals_singles(qg, g_, G, N, K, M, fmt)


def _grouped_equals_singles(qg, g_, G, N, K, M, fmt=0):
    import torch
    Ws = [_weights(fmt, g_, N, K) for _ in range(G)]
    x = dev(synth.activations(g_, M, G * K))
    qx = torch.empty(M, G * K, dtype=torch.int8, device=x.device)
    dx = torch.empty(M, G * K // 32, dtype=torch.float32, device=x.device)
    sx = torch.empty(M, G * K // 32, dtype=torch.int32, device=x.device)
    qg.quantize_act_q8(x, M, G * K, qx, dx, sx)
    y = sentinel((M, G * N), torch.float32, 99.0)
    qg.qgemv_grouped(fmt, dev(np.concatenate(Ws, axis=0)), G, N, K, qx, dx, sx, M, y)
    yh = host(y).reshape(M, G, N)
    for g in range(G):
        qs = qx[:, g * K:(g + 1) * K].contiguous()
        ds = dx[:, g * K // 32:(g + 1) * K // 32].contiguous()
        ss = sx[:, g * K // 32:(g + 1) * K // 32].contiguous()
        y1 = sentinel((M, N), torch.float32, 99.0)
        if fmt == 0:
            qg.qgemv_q8_0(dev(Ws[g]), N, K, qs, ds, M, y1)
        else:
            qg.qgemv_q4k(dev(Ws[g]), N, K, qs, ds, ss, M, y1)
        assert np.array_equal(host(y1).view(np.uint32), np.ascontiguousarray(yh[:, g]).view(np.uint32)), g


def test_grouped_past_4gib_of_activation(qg, orc):
    """A grouped batch whose activation holds more than 2^32 bytes (32 tokens x 9000
    slices of 16384): sampled groups, including rows past the 2^32-byte mark, match
    the oracle."""
    import torch
    M, G, N, K = 32, 9000, 1, 16384
    assert M * G * K > 1 << 32
    progress("grouped past 4 GiB M=%d G=%d N=%d K=%d" % (M, G, N, K))
    g_ = np.random.default_rng(4242)
    base = synth.q8_0_weight(g_, 64, K)  # row g of the stack is row g % 64 of base
    W = dev(base).repeat((G + 63) // 64, 1)[:G].contiguous()
    gen = torch.Generator(device="cuda").manual_seed(4243)
    qx = torch.randint(-127, 127, (M, G * K), dtype=torch.int8, device="cuda", generator=gen)
    dx = torch.rand((M, G * K // 32), dtype=torch.float32, device="cuda", generator=gen) * 0.01 + 1e-3
    y = sentinel((M, G * N), torch.float32, 99.0)
    qg.qgemv_grouped(0, W, G, N, K, qx, dx, None, M, y)
    yh = host(y).reshape(M, G)
    for g in (0, 1, 4095, 4096, 8191, 8999):
        qs = host(qx[:, g * K:(g + 1) * K].contiguous())
        ds = host(dx[:, g * K // 32:(g + 1) * K // 32].contiguous())
        ref, bound = orc.gemv(0, base[g % 64:g % 64 + 1].copy(), N, K, qs, ds, nthreads=oracle_threads())
        assert_within_bound(yh[:, g:g + 1], ref, bound, what="grouped past 4 GiB g=%d" % g)
    del qx, dx
    torch.cuda.empty_cache()


def test_grouped_most_groups(qg, orc):
    """The most groups a call takes (65535: the grid's y extent), 2 tokens, N = 3, K = 256:
    sampled groups against the oracle, including the first and the last."""
    import torch
    G, N, K, M = 65535, 3, 256, 2
    progress("grouped most groups G=%d" % G)
    g_ = np.random.default_rng(4343)
    base = synth.q8_0_weight(g_, 64 * N, K)  # matrix g is rows 3 (g % 64) .. + 2 of base
    W = dev(base).reshape(64, N, -1).repeat((G + 63) // 64, 1, 1)[:G].reshape(G * N, -1).contiguous()
    x = synth.activations(g_, M, G * K)
    qx, dx, _ = orc.quantize_act_q8(x)
    y = sentinel((M, G * N), torch.float32, 99.0)
    qg.qgemv_grouped(0, W, G, N, K, dev(qx), dev(dx), None, M, y)
    yh = host(y).reshape(M, G, N)
    for gi in sorted(set([0, 1, 63, 64, G - 2, G - 1] + list(g_.choice(G, 40, replace=False)))):
        wg = base[N * (gi % 64):N * (gi % 64) + N].copy()
        sl = slice(gi * K, (gi + 1) * K)
        ref, bound = orc.gemv(0, wg, N, K, qx[:, sl].copy(), dx[:, gi * K // 32:(gi + 1) * K // 32].copy())
        assert_within_bound(yh[:, gi], ref, bound, what="grouped g=%d" % gi)


def test_grouped_errors(qg):
    import torch
    W = dev(synth.q8_0_weight(np.random.default_rng(1), 16, 512))
    qx = dev(np.zeros((1, 1024), np.int8))
    dx = dev(np.ones((1, 32), np.float32))
    y = sentinel((1, 16), torch.float32, 1.0)
    c = qg._c_grouped
    assert c(0, W.data_ptr(), 0, 8, 512, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None) == -2
    assert c(0, W.data_ptr(), 70000, 8, 512, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None) == -2
    assert c(1, W.data_ptr(), 2, 8, 512, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None) == -1
    assert c(3, W.data_ptr(), 2, 8, 512, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None) == -4
    assert c(0, W.data_ptr() + 4, 2, 8, 512, qx.data_ptr(), dx.data_ptr(), None, 1, y.data_ptr(), None) == -3
    torch.cuda.synchronize()
    assert np.all(host(y) == 1.0)


# ---------------------------------------------------------------- Q8_0 prefill on the matrix cores

PREFILL_Q8_0_CASES = [
    # N, K, M: ragged token tiles and row tiles, partial K slices, the 8-block
    # unit, a prefill-sized batch (sampled outputs); then workgroups whose
    # token tiles share the weight stage: 4 tiles with a partial slice (5 of 8
    # groups), 2 tiles (K = 8192), 4 tiles with a partial second slice and a
    # last token block that holds an empty tile
    (100, 1280, 77),
    (333, 2048, 100),
    (64, 16384, 65),
    (1024, 4096, 512),
    (4096, 1280, 500),
    (2048, 8192, 300),
    (8192, 2304, 200),
    (8192, 4096, 512),  # the 512-token prefill of the 4096 -> 8192 projection
    (64, 256, 65536),  # the most tokens (2048 token tiles)
]


@pytest.mark.parametrize("N,K,M", PREFILL_Q8_0_CASES)
def test_qgemm_q8_0_parity_and_rows_equal_decode(qg, orc, N, K, M):
    """The prefill-sized Q8_0 product: every output matches the oracle, and sampled token
    rows equal the one-token decode call on that token bit for bit."""
    import torch
    progress("qgemm_q8_0 N=%d K=%d M=%d" % (N, K, M))
    g = np.random.default_rng(6000 + N + K + M)
    W = synth.q8_0_weight(g, N, K)
    Wd = dev(W)
    qx, dx, _ = orc.quantize_act_q8(synth.activations(g, M, K))
    qxd, dxd = dev(qx), dev(dx)
    y = sentinel((M, N), torch.float32, 7.0)
    qg.qgemm_q8_0(Wd, N, K, qxd, dxd, M, y)
    yh = host(y)
    toks = np.unique(np.concatenate([[0, M - 1, M // 2], g.choice(M, min(M, 12), replace=False)]))
    ref, bound = orc.gemv(0, W, N, K, qx, dx, nthreads=oracle_threads())
    assert_within_bound(yh, ref, bound, what="qgemm_q8_0 N=%d K=%d M=%d" % (N, K, M))
    for t in toks:
        one = _run_gemv(qg, 0, Wd, N, K, qxd[t:t + 1], dxd[t:t + 1], None, 1)
        assert np.array_equal(yh[t].view(np.uint32), one[0].view(np.uint32)), "token %d" % t


def test_qgemm_q8_0_errors(qg):
    import torch
    W = dev(synth.q8_0_weight(np.random.default_rng(2), 8, 512))
    qx = dev(np.zeros((40, 512), np.int8))
    dx = dev(np.ones((40, 16), np.float32))
    y = sentinel((40, 8), torch.float32, 3.0)
    c = qg._c_qgemm_q8_0
    assert c(W.data_ptr(), 8, 512, qx.data_ptr(), dx.data_ptr(), 0, y.data_ptr(), None) == -2
    assert c(W.data_ptr(), 8, 500, qx.data_ptr(), dx.data_ptr(), 40, y.data_ptr(), None) == -2
    assert c(None, 8, 512, qx.data_ptr(), dx.data_ptr(), 40, y.data_ptr(), None) == -1
    assert c(W.data_ptr() + 2, 8, 512, qx.data_ptr(), dx.data_ptr(), 40, y.data_ptr(), None) == -3
    torch.cuda.synchronize()
    assert np.all(host(y) == 3.0)
