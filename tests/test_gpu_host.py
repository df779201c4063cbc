"""Host-side behaviour on the GPU: the streaming-read diagnostic reads every byte it
is given, and the library can be driven from several host threads at once."""
import os
import subprocess
import sys

import numpy as np
import pytest

from gpu_util import dev, empty, host, progress

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("nbytes,kib,waves", [(16, 1, 1), (4096 * 3 + 48, 2, 4), (1 << 20, 4, 4),
                                              (35651584, 8, 8), ((1 << 22) + 16 * 7, 16, 16)])
def test_stream_read_xor(nbytes, kib, waves):
    import routed_moe_matvec_amd as qg
    progress("stream_read %d bytes, %d KiB per wave, %d waves" % (nbytes, kib, waves))
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = dev(words.view(np.int32))
    groups = qg.qg_stream_read_bursts(nbytes, kib)
    out = empty((groups,), __import__("torch").int32)
    qg.qg_stream_read(buf, nbytes, kib, waves, out, groups)
    got = np.bitwise_xor.reduce(host(out).view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))


_THREADS_SCRIPT = r"""
import sys, threading
sys.path.insert(0, %(root)r)
import numpy as np, torch
import routed_moe_matvec_amd as qg
import synth
torch.cuda.init()
g = synth.rng(11)
K, N, M = 4096, 1024, 12
W8 = synth.q8_0_weight(g, N, K); W4 = synth.q4k_weight(g, N, K)
x = synth.activations(g, M, K)
E, D, F, T, topk = 16, 512, 256, 2, 4
gates = [torch.from_numpy(synth.q4k_weight(g, F, D)).cuda() for _ in range(E)]
ups = [torch.from_numpy(synth.q4k_weight(g, F, D)).cuda() for _ in range(E)]
downs = [torch.from_numpy(synth.q4k_weight(g, D, F)).cuda() for _ in range(E)]
ids = torch.from_numpy(synth.moe_ids_uniform(g, T, E, topk)).cuda()
rw = torch.from_numpy(synth.routing_weights(g, T, topk)).cuda()
xm = torch.from_numpy(synth.activations(g, T, D)).cuda()
tabs = [qg.pointer_table(l, "cuda") for l in (gates, ups, downs)]
Wd8, Wd4, xd = (torch.from_numpy(a).cuda() for a in (W8, W4, x))

def work(stream):
    # one call of each launch path that sets a kernel attribute on first use
    with torch.cuda.stream(stream):
        qx = torch.empty(M, K, dtype=torch.int8, device="cuda")
        dx = torch.empty(M, K // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(M, K // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(xd, M, K, qx, dx, sx, stream=stream)
        outs = []
        for m in (1, 4, M):
            y8 = torch.empty(m, N, dtype=torch.float32, device="cuda")
            y4 = torch.empty(m, N, dtype=torch.float32, device="cuda")
            qg.qgemv_q8_0(Wd8, N, K, qx, dx, m, y8, stream=stream)
            qg.qgemv_q4k(Wd4, N, K, qx, dx, sx, m, y4, stream=stream)
            outs += [y8, y4]
        mq = torch.empty(T, D, dtype=torch.int8, device="cuda")
        md = torch.empty(T, D // 32, dtype=torch.float32, device="cuda")
        ms = torch.empty(T, D // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(xm, T, D, mq, md, ms, stream=stream)
        nb = qg.moe_routed_workspace_bytes(T, topk, E, D, F)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        ym = torch.empty(T, D, dtype=torch.float32, device="cuda")
        qg.moe_routed_qgemv(mq, md, ms, T, D, F, E, topk, ids, rw, tabs[0], tabs[1], tabs[2], ym, ws, nb, st,
                            stream=stream)
        outs.append(ym)
    stream.synchronize()
    return [o.cpu().numpy() for o in outs]

results = [None, None]
start = threading.Barrier(2)
def run(i):
    s = torch.cuda.Stream()
    start.wait()
    results[i] = work(s)
ts = [threading.Thread(target=run, args=(i,)) for i in range(2)]
for t in ts: t.start()
for t in ts: t.join()
ref = work(torch.cuda.Stream())
for r in results:
    assert r is not None
    for a, b in zip(r, ref):
        assert np.array_equal(a, b)
print("THREADS_OK")
"""


def test_two_host_threads_first_calls():
    """Two host threads make their first calls of every launch path at the same time, each on
    its own stream, in a fresh process (so the per-device set-up really races); both get the
    results of a later single-threaded call, bit for bit."""
    progress("two host threads, fresh process")
    p = subprocess.run([sys.executable, "-c", _THREADS_SCRIPT % {"root": ROOT}], capture_output=True, text=True,
                       timeout=110)
    assert p.returncode == 0 and "THREADS_OK" in p.stdout, p.stdout[-2000:] + p.stderr[-2000:]
