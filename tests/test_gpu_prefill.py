"""GPU parity of the Q4_K dequant + MFMA prefill GEMM against the fp64 oracle:
|Y - Y_oracle| <= 1e-5 * sum_k |w_k x_k| per output."""
import numpy as np
import pytest

import synth
from tests import fmt_helpers as fh
from tests.gpu_util import assert_within_bound, dev, host, oracle_threads, progress, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_moe_matvec_amd as qg
    return qg


def run_prefill(qg, W, N, K, xb, M):
    import torch
    y = sentinel((M, N), torch.float32, 99.0)
    qg.qgemm_prefill(qg.FMT_Q4K, dev(W), N, K, dev(xb.view(np.int16)), M, y)
    return host(y)


@pytest.mark.parametrize("N,K,M", [(96, 512, 40), (130, 1280, 129), (256, 1024, 256), (1, 256, 1), (300, 2304, 7)])
def test_prefill_parity_small(qg, orc, N, K, M):
    progress("prefill N=%d K=%d M=%d" % (N, K, M))
    g = np.random.default_rng(500 + N + K + M)
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    y = run_prefill(qg, W, N, K, xb, M)
    ref, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="prefill N=%d K=%d M=%d" % (N, K, M))


def test_prefill_integer_weights_exact(qg):
    """d = 1, dmin = 0 and small-integer activations: every partial sum is an integer
    below 2^24, so Y equals the int64 matmul exactly."""
    import torch
    g = np.random.default_rng(41)
    N, S, M = 70, 2, 33
    K = 256 * S
    sc = g.integers(0, 64, size=(N, S, 8))
    m = g.integers(0, 64, size=(N, S, 8))
    q = g.integers(0, 16, size=(N, S, 8, 32))
    W = fh.pack_q4k_matrix(np.ones((N, S)), np.zeros((N, S)), sc, m, q)
    xi = g.integers(-4, 5, size=(M, K))
    xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = run_prefill(qg, W, N, K, xb, M)
    Wi = (sc[..., None] * q).reshape(N, K).astype(np.int64)
    assert np.array_equal(y.astype(np.float64), (xi @ Wi.T).astype(np.float64))


def test_prefill_full_size_sampled_rows(qg, orc):
    """The 512-token prefill of the 4096 -> 8192 Q4_K projection; 96 sampled weight rows
    checked against the oracle for all 512 tokens."""
    progress("prefill 512x8192x4096")
    w = synth.WORKLOADS["q4k_prefill_512x8192x4096"]
    g = synth.rng(w["seed"])
    N, K, M = w["N"], w["K"], w["M"]
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    y = run_prefill(qg, W, N, K, xb, M)
    rows = np.sort(np.random.default_rng(9).choice(N, 96, replace=False))
    ref, bound = orc.prefill(orc.FMT_Q4K, W[rows], len(rows), K, xb, nthreads=oracle_threads())
    assert_within_bound(y[:, rows], ref, bound, what="prefill full")
    # deterministic and row-independent of the batch: token 77 alone gives the same row
    y1 = run_prefill(qg, W, N, K, xb[77:78].copy(), 1)
    assert np.array_equal(y1[0].view(np.uint32), y[77].view(np.uint32))


def test_prefill_errors(qg):
    import torch
    W = dev(synth.q4k_weight(np.random.default_rng(1), 8, 512))
    x = dev(np.zeros((4, 512), np.int16))
    y = sentinel((4, 8), torch.float32, 1.0)
    c = qg._c_prefill
    assert c(0, W.data_ptr(), 8, 512, x.data_ptr(), 4, y.data_ptr(), None) == -4
    assert c(1, None, 8, 512, x.data_ptr(), 4, y.data_ptr(), None) == -1
    assert c(1, W.data_ptr(), 8, 300, x.data_ptr(), 4, y.data_ptr(), None) == -2
    assert c(1, W.data_ptr(), 8, 512, x.data_ptr(), 0, y.data_ptr(), None) == -2
    assert c(1, W.data_ptr() + 4, 8, 512, x.data_ptr(), 4, y.data_ptr(), None) == -3
    assert np.all(host(y) == 1.0)
