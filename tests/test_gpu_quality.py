"""GPU parity of the fp32-activation Q8_0 product (no activation quantization) against
the fp64 oracle: |y - y_oracle| <= 1e-5 * sum_k |w_k x_k| per output."""
import numpy as np
import pytest

import synth
from tests.gpu_util import assert_within_bound, dev, host, oracle_threads, progress, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_moe_matvec_amd as qg
    return qg


def run(qg, W, N, K, x, M):
    import torch
    y = sentinel((M, N), torch.float32, 99.0)
    qg.qgemv_q8_0_quality(dev(W), N, K, dev(x), M, y)
    return host(y)


@pytest.mark.parametrize("N,K,M", [(512, 1024, 1), (4096, 8192, 1), (130, 2304, 3), (1, 256, 1), (77, 16384, 2),
                                   (300, 4096, 32), (64, 12288, 5)])
def test_quality_parity(qg, orc, N, K, M):
    """Ragged N, 1 and 32 tokens (several staged chunks at large K), both unit sizes (K <= 8192
    and above)."""
    progress("quality N=%d K=%d M=%d" % (N, K, M))
    g = np.random.default_rng(700 + N + K + M)
    W = synth.q8_0_weight(g, N, K)
    x = synth.activations(g, M, K)
    y = run(qg, W, N, K, x, M)
    ref, bound = orc.gemv_fx(orc.FMT_Q8_0, W, N, K, x, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="quality N=%d K=%d M=%d" % (N, K, M))


def test_quality_wide_range_activation(qg, orc):
    """x as given, no 8-bit rounding: tokens 1e-30 and 1e30 apart, and a block whose small
    entries a Q8 activation would round to 0, are still within the bound."""
    g = np.random.default_rng(71)
    N, K, M = 96, 1024, 3
    W = synth.q8_0_weight(g, N, K)
    x = synth.activations(g, M, K)
    x[1] *= np.float32(1e-30)
    x[2] *= np.float32(1e30)
    x[0, :32] = 1e-6
    x[0, 0] = 1000.0
    y = run(qg, W, N, K, x, M)
    ref, bound = orc.gemv_fx(orc.FMT_Q8_0, W, N, K, x)
    assert_within_bound(y, ref, bound, what="quality wide range")


def test_quality_row_of_batch_equals_single_token(qg):
    g = np.random.default_rng(72)
    N, K, M = 200, 4096, 6
    W = synth.q8_0_weight(g, N, K)
    x = synth.activations(g, M, K)
    y = run(qg, W, N, K, x, M)
    y3 = run(qg, W, N, K, x[3:4].copy(), 1)
    assert np.array_equal(y3[0].view(np.uint32), y[3].view(np.uint32))


def test_quality_errors(qg):
    import torch
    W = dev(synth.q8_0_weight(np.random.default_rng(1), 8, 512))
    x = dev(np.zeros((2, 512), np.float32))
    y = sentinel((2, 8), torch.float32, 1.0)
    c = qg._c_quality
    assert c(None, 8, 512, x.data_ptr(), 2, y.data_ptr(), None) == -1
    assert c(W.data_ptr(), 8, 300, x.data_ptr(), 2, y.data_ptr(), None) == -2
    assert c(W.data_ptr(), 8, 512, x.data_ptr(), 33, y.data_ptr(), None) == -2
    assert c(W.data_ptr(), 0, 512, x.data_ptr(), 2, y.data_ptr(), None) == -2
    assert c(W.data_ptr() + 4, 8, 512, x.data_ptr(), 2, y.data_ptr(), None) == -3
    torch.cuda.synchronize()
    assert np.all(host(y) == 1.0)
