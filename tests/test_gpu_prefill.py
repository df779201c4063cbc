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


VARIANTS = ["plain", "ws"]


def run_prefill(qg, W, N, K, xb, M, variant="plain"):
    """qgemm_prefill (conversion inside the GEMM) or qgemm_prefill_ws (pre-pass
    into a workspace, which starts filled with garbage)."""
    import torch
    y = sentinel((M, N), torch.float32, 99.0)
    if variant == "plain":
        qg.qgemm_prefill(qg.FMT_Q4K, dev(W), N, K, dev(xb.view(np.int16)), M, y)
    else:
        nb = qg.qgemm_prefill_workspace_bytes(M, K)
        ws = sentinel((nb,), torch.uint8, 0xA5)
        qg.qgemm_prefill_ws(qg.FMT_Q4K, dev(W), N, K, dev(xb.view(np.int16)), M, y, ws, nb)
    return host(y)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("N,K,M", [(96, 512, 40), (130, 1280, 129), (256, 1024, 256), (1, 256, 1), (300, 2304, 7),
                                   (200, 2560, 300), (64, 16384, 33)])
def test_prefill_parity_small(qg, orc, N, K, M, variant):
    """Ragged N and M tails, K of 1..10 superblocks (partial min-term windows) and the largest K."""
    progress("prefill %s N=%d K=%d M=%d" % (variant, N, K, M))
    g = np.random.default_rng(500 + N + K + M)
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    y = run_prefill(qg, W, N, K, xb, M, variant)
    ref, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="prefill %s N=%d K=%d M=%d" % (variant, N, K, M))


def scaled_bf16(xb, scale):
    import torch
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float() * scale
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("scale", [2.0 ** 40, 2.0 ** -40, 1.0])
def test_prefill_ws_activation_range(qg, orc, scale):
    """The pre-pass scales each token by a power of two, so activations far outside
    fp16's range (and rows mixing magnitudes 2^20 apart) stay within the bound."""
    progress("prefill ws activation scale 2^%d" % int(np.log2(scale)))
    g = np.random.default_rng(77)
    N, K, M = 144, 1024, 20
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    xb = scaled_bf16(xb, scale)
    xb[3] = scaled_bf16(xb[3:4], 2.0 ** -20)[0]  # one quiet token
    xb[5, :100] = scaled_bf16(xb[5:6, :100], 2.0 ** 10)[0]  # one token with loud early inputs
    xb[7] = 0  # an all-zero token
    y = run_prefill(qg, W, N, K, xb, M, "ws")
    ref, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="prefill ws scale %g" % scale)
    assert np.all(y[7] == 0.0)


def test_prefill_ws_rows_spanning_wide_magnitudes(qg, orc):
    """Rows whose elements span 2^60: those more than ~2^32 below the row's largest become
    fp16 subnormals (or 0) after the per-token power of two; the product stays within the
    bound, which they barely touch."""
    progress("prefill ws rows spanning 2^60")
    g = np.random.default_rng(91)
    N, K, M = 96, 1024, 20
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    # per element a power of two between 2^-30 and 2^30 (bf16 keeps it exactly)
    exps = g.integers(-30, 31, size=(M, K)).astype(np.float64)
    import torch
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy() * np.exp2(exps)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = run_prefill(qg, W, N, K, xb, M, "ws")
    ref, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="prefill ws wide rows")


def set_scales(W, N, K, d, dmin):
    """Overwrite the fp16 d and dmin of every superblock of a Q4_K matrix."""
    sb = W.reshape(N, K // 256, 144)
    sb[:, :, 0:2] = np.asarray(d, np.float16).view(np.uint8).reshape(N, K // 256, 2)
    sb[:, :, 2:4] = np.asarray(dmin, np.float16).view(np.uint8).reshape(N, K // 256, 2)
    return W


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("kind", ["large", "tiny", "mixed"])
def test_prefill_scale_range(qg, orc, variant, kind):
    """d and dmin across fp16's range: large (0.05 .. 60000), tiny (1e-7 .. 1e-6,
    partly subnormal) and mixed (log-uniform over 6e-8 .. 65504 per superblock, so a
    row's superblocks differ by up to 2^30): the min term's per-window power-of-two
    scaling keeps every output within the bound."""
    progress("prefill %s d/dmin %s" % (variant, kind))
    g = np.random.default_rng(78)
    N, K, M = 80, 2048, 24
    W = synth.q4k_weight(g, N, K)
    shape = (N, K // 256)
    if kind == "large":
        d, dmin = g.uniform(0.05, 60000, shape), g.uniform(0.05, 60000, shape)
    elif kind == "tiny":
        d, dmin = g.uniform(1e-7, 1e-6, shape), g.uniform(1e-7, 1e-6, shape)
    else:
        d = np.exp(g.uniform(np.log(6e-8), np.log(65504), shape))
        dmin = np.exp(g.uniform(np.log(6e-8), np.log(65504), shape))
    W = set_scales(W, N, K, d, dmin)
    xb = synth.bf16_activations(g, M, K)
    y = run_prefill(qg, W, N, K, xb, M, variant)
    ref, bound = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    assert_within_bound(y, ref, bound, what="prefill %s scales %s" % (variant, kind))


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_integer_weights_exact(qg, variant):
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
    y = run_prefill(qg, W, N, K, xb, M, variant)
    Wi = (sc[..., None] * q).reshape(N, K).astype(np.int64)
    assert np.array_equal(y.astype(np.float64), (xi @ Wi.T).astype(np.float64))


_FULL_REF = {}


def _prefill_oracle_full(orc, W, N, K, xb):
    """The oracle of the full-size prefill, computed once for both variants."""
    key = (N, K, xb.shape[0])
    if key not in _FULL_REF:
        _FULL_REF[key] = orc.prefill(orc.FMT_Q4K, W, N, K, xb, nthreads=oracle_threads())
    return _FULL_REF[key]


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_full_size(qg, orc, variant):
    """The 512-token prefill of the 4096 -> 8192 Q4_K projection: every output checked
    against the oracle."""
    progress("prefill %s 512x8192x4096" % variant)
    w = synth.WORKLOADS["q4k_prefill_512x8192x4096"]
    g = synth.rng(w["seed"])
    N, K, M = w["N"], w["K"], w["M"]
    W = synth.q4k_weight(g, N, K)
    xb = synth.bf16_activations(g, M, K)
    y = run_prefill(qg, W, N, K, xb, M, variant)
    ref, bound = _prefill_oracle_full(orc, W, N, K, xb)
    assert_within_bound(y, ref, bound, what="prefill full")
    # deterministic and row-independent of the batch: token 77 alone gives the same row
    y1 = run_prefill(qg, W, N, K, xb[77:78].copy(), 1, variant)
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


def test_prefill_ws_errors(qg):
    import torch
    W = dev(synth.q4k_weight(np.random.default_rng(1), 8, 512))
    x = dev(np.zeros((4, 512), np.int16))
    y = sentinel((4, 8), torch.float32, 1.0)
    nb = qg.qgemm_prefill_workspace_bytes(4, 512)
    ws = torch.zeros(nb + 64, dtype=torch.uint8, device=x.device)
    c = qg._c_prefill_ws
    assert c(1, W.data_ptr(), 8, 512, x.data_ptr(), 4, y.data_ptr(), None, nb, None) == -1
    assert c(1, W.data_ptr(), 8, 512, x.data_ptr(), 4, y.data_ptr(), ws.data_ptr(), nb - 1, None) == -5
    assert c(1, W.data_ptr(), 8, 512, x.data_ptr(), 4, y.data_ptr(), ws.data_ptr() + 8, nb, None) == -3
    assert c(0, W.data_ptr(), 8, 512, x.data_ptr(), 4, y.data_ptr(), ws.data_ptr(), nb, None) == -4
    assert c(1, W.data_ptr(), 8, 300, x.data_ptr(), 4, y.data_ptr(), ws.data_ptr(), nb, None) == -2
    torch.cuda.synchronize()
    assert np.all(host(y) == 1.0)
