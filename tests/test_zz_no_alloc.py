"""moe_routed_qgemv_noalloc, called through the C ABI: it gives the results of
moe_routed_qgemv_fmt with a caller workspace bit for bit (the same kernels on
the library's fixed device array), on two calls in a row, the second with a
smaller input, for Q4_K and FP4 experts; sizes past the array are rejected
before anything is launched."""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_util import dev, empty, host, progress, sentinel

pytestmark = pytest.mark.gpu


def _experts(fmt, E, D, F, seed):
    g = synth.rng(seed)
    mats = [[dev(synth.weight(fmt, g, n, k)) for _ in range(E)] for (n, k) in ((F, D), (F, D), (D, F))]
    return mats


def _call_both(qg, fmt, tabs, E, D, F, T, topk, seed):
    import torch
    g = synth.rng(seed)
    ids = dev(synth.moe_ids_uniform(g, T, E, topk))
    rw = dev(synth.routing_weights(g, T, topk))
    x = dev(synth.activations(g, T, D))
    qx, dx, sx = empty((T, D), torch.int8), empty((T, D // 32), torch.float32), empty((T, D // 32), torch.int32)
    qg.quantize_act_q8(x, T, D, qx, dx, sx)
    # the existing entry point with a caller workspace
    nb = qg.moe_routed_workspace_bytes(T, topk, E, D, F)
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
    y_ref, st_ref = sentinel((T, D), torch.float32, 5.0), sentinel((1,), torch.int32, -9)
    qg.moe_routed_qgemv_fmt(fmt, qx, dx, sx, T, D, F, E, topk, ids, rw, tabs[0], tabs[1], tabs[2], y_ref, ws, nb,
                            st_ref)
    # the no-allocation entry point, straight through ctypes
    y, st = sentinel((T, D), torch.float32, -5.0), sentinel((1,), torch.int32, -9)
    f = ctypes.CDLL(qg.library_path()).moe_routed_qgemv_noalloc  # a handle of its own (own argtypes)
    vp = ctypes.c_void_p
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, vp, vp, vp] + [ctypes.c_int] * 5 + [vp] * 7 + [vp]
    stream = torch.cuda.current_stream().cuda_stream
    rc = f(fmt, qx.data_ptr(), dx.data_ptr(), sx.data_ptr(), T, D, F, E, topk, ids.data_ptr(), rw.data_ptr(),
           tabs[0].data_ptr(), tabs[1].data_ptr(), tabs[2].data_ptr(), y.data_ptr(), st.data_ptr(), stream)
    assert rc == 0, qg.qg_status_string(rc)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0 and int(host(st_ref)[0]) == 0
    assert np.array_equal(host(y).view(np.uint32), host(y_ref).view(np.uint32))


@pytest.mark.parametrize("fmt", [1, 3])
def test_noalloc_equals_workspace_call_twice(fmt):
    import torch
    import routed_moe_matvec_amd as qg
    E, D, F, topk = 64, 4096, 2048, 6
    progress("moe_routed_qgemv_noalloc fmt=%d E=%d" % (fmt, E))
    mats = _experts(fmt, E, D, F, 70 + fmt)
    tabs = [qg.pointer_table(lst, "cuda") for lst in mats]
    _call_both(qg, fmt, tabs, E, D, F, 16, topk, 1)  # 96 pairs: the larger call first
    _call_both(qg, fmt, tabs, E, D, F, 3, topk, 2)   # then a smaller one on the same array
    torch.cuda.synchronize()


def test_noalloc_rejects_sizes_past_the_array():
    import torch
    import routed_moe_matvec_amd as qg
    T, topk, E, D, F = 33, 6, 256, 4096, 2048
    assert qg.moe_routed_workspace_bytes(T, topk, E, D, F) > qg.MOE_SCRATCH_BYTES
    assert qg.moe_routed_workspace_bytes(32, topk, E, D, F) <= qg.MOE_SCRATCH_BYTES
    y = sentinel((T, D), torch.float32, 3.0)
    st = sentinel((1,), torch.int32, -9)
    fake = empty((1024,), torch.int32)
    with pytest.raises(qg.QGError) as e:
        qg.moe_routed_qgemv_noalloc(1, fake, fake, fake, T, D, F, E, topk, fake, fake, fake, fake, fake, y, st)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert np.all(host(y) == 3.0) and int(host(st)[0]) == -9
