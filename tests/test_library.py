"""The C-ABI library without a GPU: it loads, exports every function the public
header declares, and its host-side logic (argument checks, workspace sizing,
status strings) behaves as documented.  No call here reaches a kernel launch:
every checked call fails validation first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"#[^\n]*", " ", src)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import routed_moe_matvec_amd as qg
    return ctypes.CDLL(qg.library_path())


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["quantize_act_q8", "qgemv_q8_0", "qgemv_q4k", "qgemv_paired", "moe_routed_qgemv",
                 "moe_routed_workspace_bytes", "moe_routed_workspace_layout", "qgemm_prefill", "qg_status_string",
                 "qgemv_debug_block_isums"]:
        assert want in names, want


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_the_header():
    import routed_moe_matvec_amd as qg
    for n in declared_functions():
        assert callable(getattr(qg, n, None)), n


def test_status_strings(lib):
    import routed_moe_matvec_amd as qg
    for code in range(-6, 1):
        assert qg.qg_status_string(code) not in ("", "unknown status")
    assert qg.qg_status_string(-77) == "unknown status"


def test_host_validation_without_gpu(lib):
    """Rejected calls return their code before touching the device."""
    vp = ctypes.c_void_p
    fake = vp(1 << 40)  # never dereferenced: every call below fails validation first
    f = lib.qgemv_q8_0
    f.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp]
    assert f(None, 8, 512, fake, fake, 1, fake, None) == -1
    assert f(fake, 8, 300, fake, fake, 1, fake, None) == -2
    assert f(fake, 8, 512, fake, fake, 33, fake, None) == -2
    assert f(fake, 0, 512, fake, fake, 1, fake, None) == -2
    assert f(vp((1 << 40) + 8), 8, 512, fake, fake, 1, fake, None) == -3
    q = lib.quantize_act_q8
    q.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
    assert q(fake, 1, 40, fake, fake, fake, None) == -2
    assert q(fake, 1, 64, None, fake, fake, None) == -1
    p = lib.qgemm_prefill
    p.argtypes = [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp, vp]
    assert p(0, fake, 8, 512, fake, 4, fake, None) == -4
    pw = lib.qgemm_prefill_ws
    pw.argtypes = [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    assert pw(1, fake, 8, 512, fake, 4, fake, None, 1 << 20, None) == -1
    assert pw(1, fake, 8, 512, fake, 4, fake, fake, 100, None) == -5
    assert pw(1, fake, 8, 512, fake, 4, fake, vp((1 << 40) + 8), 1 << 20, None) == -3
    assert pw(1, fake, 8, 768 + 1, fake, 4, fake, fake, 1 << 20, None) == -2


def test_moe_workspace_sizing():
    import routed_moe_matvec_amd as qg
    T, topk, E, D, F = 8, 6, 256, 4096, 2048
    nbytes = qg.moe_routed_workspace_bytes(T, topk, E, D, F)
    lay = qg.moe_routed_workspace_layout(T, topk, E, D, F)
    P, Ucap = T * topk, min(T * topk, E)
    sizes = {"NUNIQ": 4, "UNIQ": 4 * Ucap, "SLOT": 4 * P, "PAIR_OFF": 4 * (Ucap + 1), "PAIRS": 4 * P,
             "G": 4 * P * F, "V": 4 * P * F, "H": 4 * P * F, "HQ": P * F, "HD": 4 * P * F // 32,
             "HS": 4 * P * F // 32, "O": 4 * P * D, "HOT": 4 * (1 + 2 * (P // 32 + P // qg.MOE_MM_PAIRS + 1))}
    names = qg.WS_REGIONS
    for a, b in zip(names, names[1:]):
        assert lay[b] >= lay[a] + sizes[a] and lay[b] % 256 == 0
    assert nbytes >= lay["HOT"] + sizes["HOT"]
    assert qg.moe_routed_workspace_bytes(8, 6, 256, 4000, 2048) == 0
    assert qg.moe_routed_workspace_bytes(2000, 6, 256, 4096, 2048) == 0  # more than 8192 pairs
    with pytest.raises(qg.QGError):
        qg.moe_routed_workspace_layout(0, 6, 256, 4096, 2048)


def test_prefill_workspace_sizing():
    import routed_moe_matvec_amd as qg
    for M, K in [(1, 256), (7, 2304), (512, 4096), (300, 16384)]:
        nb = qg.qgemm_prefill_workspace_bytes(M, K)
        # fp16 x [M, K], int32 exponents [M], fp16 hi and lo block sums [M, K / 32] each
        need = 2 * M * K + 4 * M + 2 * (2 * M * (K // 32))
        assert nb >= need, (M, K)
        assert nb % 256 == 0 and nb <= need + 4 * 256
    for M, K in [(0, 256), (4, 300), (4, 128), (4, 16384 + 256)]:
        assert qg.qgemm_prefill_workspace_bytes(M, K) == 0, (M, K)


def test_matrix_bytes_match_the_documented_layout():
    """qg_matrix_bytes agrees with the storage the generators write (codes, padding to
    256 bytes, scales) for the block-scaled formats and with whole rows for the others."""
    import routed_moe_matvec_amd as qg
    import synth
    for N, K in [(1, 256), (127, 512), (129, 4096), (300, 7168), (4096, 16384)]:
        assert qg.qg_matrix_bytes(0, N, K) == N * (K // 32) * 34
        assert qg.qg_matrix_bytes(1, N, K) == N * (K // 256) * 144
        for fmt in (2, 3):
            assert qg.qg_matrix_bytes(fmt, N, K) == synth.scaled_matrix_bytes(fmt, N, K), (fmt, N, K)
    for fmt, N, K in [(4, 8, 512), (2, 0, 512), (3, 8, 300), (2, 8, 128), (3, 8, 16384 + 256)]:
        assert qg.qg_matrix_bytes(fmt, N, K) == 0, (fmt, N, K)


def test_mx_host_validation_without_gpu(lib):
    vp = ctypes.c_void_p
    fake = vp(1 << 40)
    f = lib.qgemv_mx
    f.argtypes = [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp]
    assert f(0, fake, 8, 512, fake, fake, 1, fake, None) == -4   # Q8_0 is not a block-scaled format
    assert f(2, None, 8, 512, fake, fake, 1, fake, None) == -1
    assert f(3, fake, 8, 384, fake, fake, 1, fake, None) == -2
    assert f(3, fake, 8, 512, fake, fake, 33, fake, None) == -2
    assert f(2, vp((1 << 40) + 4), 8, 512, fake, fake, 1, fake, None) == -3
    m = lib.moe_routed_qgemv_fmt
    m.argtypes = [ctypes.c_int] + [vp] * 3 + [ctypes.c_int] * 5 + [vp] * 7 + [ctypes.c_size_t, vp, vp]
    assert m(0, fake, fake, fake, 1, 4096, 2048, 256, 6, fake, fake, fake, fake, fake, fake, fake, 1 << 30,
             fake, None) == -4
    assert m(3, fake, fake, fake, 1, 4096, 2000, 256, 6, fake, fake, fake, fake, fake, fake, fake, 1 << 30,
             fake, None) == -2
    assert m(2, fake, fake, fake, 1, 4096, 2048, 256, 6, fake, fake, fake, fake, fake, fake, fake, 16,
             fake, None) == -5
    q = lib.qgemm_q8_0
    q.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp]
    assert q(fake, 8, 512, fake, fake, 0, fake, None) == -2
    assert q(fake, 8, 512, fake, fake, 65537, fake, None) == -2
    assert q(fake, 8, 384 + 1, fake, fake, 64, fake, None) == -2
    assert q(fake, 8, 512, None, fake, 64, fake, None) == -1


def test_workspace_regions_match_header():
    """The binding's region list and the matrix-core pair threshold are the header's."""
    import re
    import routed_moe_matvec_amd as qg
    hdr = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    regions = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define QG_WS_(\w+) (\d+)", hdr)}
    count = regions.pop("COUNT")
    assert count == len(qg.WS_REGIONS)
    assert [name for name, _ in sorted(regions.items(), key=lambda kv: kv[1])] == qg.WS_REGIONS
    assert int(re.search(r"#define QG_MOE_MM_PAIRS (\d+)", hdr).group(1)) == qg.MOE_MM_PAIRS


def test_stream_read_validation_without_gpu(lib):
    """The streaming-read diagnostic's burst count and argument checks."""
    import routed_moe_matvec_amd as qg
    assert qg.qg_stream_read_bursts(1 << 30, 4) == (1 << 30) // 4096
    assert qg.qg_stream_read_bursts(35651584, 8) == -(-35651584 // 8192)
    assert qg.qg_stream_read_bursts(16, 16) == 1
    for args in [(0, 4), (1000, 4), (4096, 3), (4096, 32)]:
        assert qg.qg_stream_read_bursts(*args) == 0, args
    vp = ctypes.c_void_p
    fake = vp(1 << 40)
    f = lib.qg_stream_read
    f.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]
    assert f(None, 4096, 4, 4, fake, 16, None) == -1
    assert f(fake, 4096 * 4, 1, 4, fake, 3, None) == -2  # needs 4 bursts
    assert f(fake, 4100, 4, 4, fake, 16, None) == -2
    assert f(fake, 4096, 4, 0, fake, 16, None) == -2
    assert f(fake, 4096, 4, 17, fake, 16, None) == -2
    assert f(vp((1 << 40) + 8), 4096, 4, 4, fake, 16, None) == -3
    assert f(fake, 4096, 4, 4, vp((1 << 40) + 2), 16, None) == -3
