"""GPU parity of the routed-MoE decode (compact expert table, gate/up, SiLU*up requant,
down, weighted combine), called through the C ABI, checked stage by stage against the
CPU oracle on the same seeded inputs.

Staged checks (the GPU's fp32 h is the single hand-off point):
  table        == oracle table (np.unique semantics), bit-exact
  g, v         within 1e-5 * sum|w x| of the oracle; bit-equal to qgemv_q4k on the same expert
  h            within 1e-6 * |silu(g)*v| (fp64, on the GPU's g and v)
  hq, hd, hs   == oracle Q8 quantization of the GPU's h, bit-exact
  o            within 1e-5 * sum|w x| of the oracle down projection of the GPU's hq
  y            within 1e-5 * sum_k |rw| * bound(o) of sum_k rw * o_oracle
End to end from scratch (h quantized by the oracle itself): within 1e-3 * bound.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import assert_within_bound, dev, empty, host, oracle_threads, progress, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_moe_matvec_amd as qg
    return qg


class MoeProblem:
    """Experts, ids, routing weights and activations on the host and the device."""

    def __init__(self, qg, E, D, F, T, topk, seed, ids=None, only_selected=False, zipf=False, fmt=1):
        import torch
        g = synth.rng(seed)
        self.E, self.D, self.F, self.T, self.topk, self.fmt = E, D, F, T, topk, fmt
        if ids is None:
            ids = synth.moe_ids_zipf(g, T, E, topk) if zipf else synth.moe_ids_uniform(g, T, E, topk)
        self.ids = np.asarray(ids, np.int32)
        self.rw = synth.routing_weights(g, T, topk)
        self.x = synth.activations(g, T, D)
        needed = set(int(e) for e in self.ids.ravel() if 0 <= e < E)
        self.gate, self.up, self.down = [None] * E, [None] * E, [None] * E
        for e in range(E):
            if only_selected and e not in needed:
                continue
            ge = np.random.default_rng([seed, e])  # per-expert stream: independent of which are built
            self.gate[e] = synth.weight(fmt, ge, F, D)
            self.up[e] = synth.weight(fmt, ge, F, D)
            self.down[e] = synth.weight(fmt, ge, D, F)
        self.dgate = [None if w is None else dev(w) for w in self.gate]
        self.dup = [None if w is None else dev(w) for w in self.up]
        self.ddown = [None if w is None else dev(w) for w in self.down]
        self.qg = qg
        xd = dev(self.x)
        self.qx = empty((T, D), torch.int8)
        self.dx = empty((T, D // 32), torch.float32)
        self.sx = empty((T, D // 32), torch.int32)
        qg.quantize_act_q8(xd, T, D, self.qx, self.dx, self.sx)

    def run(self, ids=None, rw=None, gate=None, up=None, down=None, ws_fill=0):
        import torch
        qg = self.qg
        ids = self.ids if ids is None else np.asarray(ids, np.int32)
        rw = self.rw if rw is None else np.asarray(rw, np.float32)
        T, topk = ids.shape
        nbytes = qg.moe_routed_workspace_bytes(T, topk, self.E, self.D, self.F)
        ws = torch.full((nbytes,), ws_fill, dtype=torch.uint8, device="cuda")
        status = sentinel((1,), torch.int32, -99)
        y = sentinel((T, self.D), torch.float32, 777.0)
        tabs = [qg.pointer_table(lst, "cuda") for lst in (gate or self.dgate, up or self.dup, down or self.ddown)]
        if self.fmt == 1:
            qg.moe_routed_qgemv(self.qx[:T], self.dx[:T], self.sx[:T], T, self.D, self.F, self.E, topk, dev(ids),
                                dev(rw), tabs[0], tabs[1], tabs[2], y, ws, nbytes, status)
        else:
            qg.moe_routed_qgemv_fmt(self.fmt, self.qx[:T], self.dx[:T], self.sx[:T], T, self.D, self.F, self.E,
                                    topk, dev(ids), dev(rw), tabs[0], tabs[1], tabs[2], y, ws, nbytes, status)
        torch.cuda.synchronize()
        return host(y), ws, int(host(status)[0])

    def regions(self, ws, T=None):
        """Views of the workspace regions as numpy arrays."""
        qg = self.qg
        T = self.T if T is None else T
        P = T * self.topk
        lay = qg.moe_routed_workspace_layout(T, self.topk, self.E, self.D, self.F)
        raw = host(ws)
        F, D = self.F, self.D

        def view(name, dtype, count):
            o = lay[name]
            return raw[o:o + count * np.dtype(dtype).itemsize].view(dtype)

        U = int(view("NUNIQ", np.int32, 1)[0])
        return dict(
            n_uniq=U, uniq=view("UNIQ", np.int32, U), slot=view("SLOT", np.int32, P),
            pair_off=view("PAIR_OFF", np.int32, U + 1), pairs=view("PAIRS", np.int32, P),
            g=view("G", np.float32, P * F).reshape(P, F), v=view("V", np.float32, P * F).reshape(P, F),
            h=view("H", np.float32, P * F).reshape(P, F), hq=view("HQ", np.int8, P * F).reshape(P, F),
            hd=view("HD", np.float32, P * F // 32).reshape(P, F // 32),
            hs=view("HS", np.int32, P * F // 32).reshape(P, F // 32),
            o=view("O", np.float32, P * D).reshape(P, D))


def check_staged(qg, orc, pb: MoeProblem, y, ws, pairs_to_check=None, tokens_to_check=None):
    """Stage-by-stage parity of one MoE call (see the module docstring)."""
    F, D, topk = pb.F, pb.D, pb.topk
    R = pb.regions(ws)
    tab = orc.moe_table(pb.ids, pb.E)
    assert R["n_uniq"] == tab["n_uniq"]
    assert np.array_equal(R["uniq"], tab["uniq"])
    assert np.array_equal(R["slot"], tab["slot"].ravel())
    assert np.array_equal(R["pair_off"], tab["pair_off"])
    assert np.array_equal(R["pairs"], tab["pairs"])
    qx, dx = host(pb.qx), host(pb.dx)
    P = pb.T * topk
    check = range(P) if pairs_to_check is None else pairs_to_check
    nt = oracle_threads()
    o_ref = {}
    # the oracle runs once per expert over all of its checked pairs (rows are independent per token)
    by_expert = {}
    for p in check:
        if R["slot"][p] >= 0:  # a pair with an invalid id has no stages
            by_expert.setdefault(int(pb.ids.ravel()[p]), []).append(p)
    for e, ps in sorted(by_expert.items()):
        ps = np.asarray(ps)
        ts = ps // topk
        gr, gb = orc.gemv(pb.fmt, pb.gate[e], F, D, qx[ts], dx[ts], nthreads=nt)
        vr, vb = orc.gemv(pb.fmt, pb.up[e], F, D, qx[ts], dx[ts], nthreads=nt)
        assert_within_bound(R["g"][ps], gr, gb, what="g of expert %d" % e)
        assert_within_bound(R["v"][ps], vr, vb, what="v of expert %d" % e)
        g64, v64 = R["g"][ps].astype(np.float64), R["v"][ps].astype(np.float64)
        h_ref = g64 / (1.0 + np.exp(-g64)) * v64
        assert np.all(np.abs(R["h"][ps] - h_ref) <= 1e-6 * np.abs(h_ref) + 1e-30), "h of expert %d" % e
        hq, hd, hs = orc.quantize_act_q8(R["h"][ps])
        assert np.array_equal(R["hq"][ps], hq) and np.array_equal(R["hs"][ps], hs)
        assert np.array_equal(R["hd"][ps].view(np.uint32), hd.view(np.uint32))
        orf, ob = orc.gemv(pb.fmt, pb.down[e], D, F, R["hq"][ps], R["hd"][ps], nthreads=nt)
        assert_within_bound(R["o"][ps], orf, ob, what="o of expert %d" % e)
        for i, p in enumerate(ps):
            o_ref[int(p)] = (orf[i], ob[i])
    toks = range(pb.T) if tokens_to_check is None else tokens_to_check
    for t in toks:
        acc = np.zeros(D)
        bnd = np.zeros(D)
        for k in range(topk):
            p = t * topk + k
            if R["slot"][p] < 0:
                continue
            orf, ob = o_ref[p]
            acc += float(pb.rw[t, k]) * orf
            bnd += abs(float(pb.rw[t, k])) * ob
        assert_within_bound(y[t:t + 1], acc[None], bnd[None], what="y token %d" % t)
    return R


def test_moe_small_staged_and_end_to_end(qg, orc):
    for (E, D, F, T, topk, seed) in [(16, 512, 256, 1, 6, 1), (16, 512, 256, 3, 6, 2), (10, 768, 512, 8, 4, 3),
                                     (8, 256, 256, 9, 8, 4)]:
        progress("moe small E=%d D=%d F=%d T=%d topk=%d" % (E, D, F, T, topk))
        pb = MoeProblem(qg, E, D, F, T, topk, seed)
        y, ws, st = pb.run()
        assert st == 0
        check_staged(qg, orc, pb, y, ws)
        ye, be, ste = orc.moe_routed(host(pb.qx), host(pb.dx), pb.ids, pb.rw, pb.gate, pb.up, pb.down, D, F,
                                     nthreads=oracle_threads())
        assert ste == 0
        assert_within_bound(y, ye, be, rel=1e-3, what="end-to-end")


def test_moe_gate_equals_dense_q4k_call(qg):
    """The expert GEMVs and qgemv_q4k share one engine: g is bit-equal to the dense call."""
    import torch
    pb = MoeProblem(qg, 12, 1024, 512, 4, 3, 7)
    y, ws, st = pb.run()
    R = pb.regions(ws)
    for p in range(pb.T * pb.topk):
        t, e = p // pb.topk, int(pb.ids.ravel()[p])
        out = torch.empty(1, pb.F, dtype=torch.float32, device="cuda")
        qg.qgemv_q4k(pb.dgate[e], pb.F, pb.D, pb.qx[t:t + 1], pb.dx[t:t + 1], pb.sx[t:t + 1], 1, out)
        assert np.array_equal(host(out)[0].view(np.uint32), R["g"][p].view(np.uint32))


def test_moe_full_size_256_experts_t1_t8(qg, orc):
    """The routed-MoE workload: 256 Q4_K experts (gate/up 4096->2048, down 2048->4096),
    top-6 uniform, T = 1 and T = 8; unselected experts are NULL in the pointer table."""
    w = synth.WORKLOADS["moe_e256_t8"]
    for T in (1, 8):
        progress("moe full E=256 T=%d" % T)
        pb = MoeProblem(qg, w["E"], w["D"], w["F"], T, w["topk"], w["seed"] + T, only_selected=True)
        y, ws, st = pb.run()
        assert st == 0
        check_staged(qg, orc, pb, y, ws)


def test_moe_zipf_384_experts_t64(qg, orc):
    """384 experts, 64 tokens, Zipf(1.1) popularity: the table exactly, and every stage of
    every one of the 384 pairs and every token's output against the oracle."""
    w = synth.WORKLOADS["moe_e384_t64_zipf"]
    progress("moe zipf E=384 T=64")
    pb = MoeProblem(qg, w["E"], w["D"], w["F"], w["T"], w["topk"], w["seed"], zipf=True, only_selected=True)
    y, ws, st = pb.run()
    assert st == 0
    counts = np.bincount(pb.ids.ravel(), minlength=pb.E)
    assert counts.max() >= 20  # expert reuse across tokens really happens
    check_staged(qg, orc, pb, y, ws)


@pytest.mark.parametrize("E,D,F,T,topk,seed,zipf", [(4, 1280, 512, 48, 3, 41, False),
                                                     (6, 512, 256, 40, 3, 42, False),
                                                     (40, 768, 256, 12, 6, 43, True)])
def test_moe_popular_experts_on_matrix_cores(qg, orc, E, D, F, T, topk, seed, zipf):
    """From QG_MOE_MM_PAIRS tokens on, experts with that many pairs or more run on the
    matrix cores: the work-item list is exact, every stage matches the oracle, and g, v
    and o of those experts equal the one-token dense calls bit for bit (more than 32
    pairs per expert, groups per row not a power of two; the last case mixes them with
    experts on the dot-product kernels)."""
    import torch
    progress("moe matrix-core experts E=%d D=%d F=%d T=%d topk=%d" % (E, D, F, T, topk))
    pb = MoeProblem(qg, E, D, F, T, topk, seed, zipf=zipf)
    y, ws, st = pb.run()
    assert st == 0
    R = check_staged(qg, orc, pb, y, ws)
    lay = qg.moe_routed_workspace_layout(T, topk, E, D, F)
    raw = host(ws)
    hot = raw[lay["HOT"]:].view(np.int32)
    counts = np.diff(R["pair_off"])
    want = [(u, m0) for u in range(R["n_uniq"]) if counts[u] >= qg.MOE_MM_PAIRS for m0 in range(0, counts[u], 32)]
    assert hot[0] == len(want) and len(want) > 0
    assert [tuple(hot[1 + 2 * i:3 + 2 * i]) for i in range(len(want))] == want
    for u in sorted(set(u for u, _ in want)):
        e = int(R["uniq"][u])
        for p in R["pairs"][R["pair_off"][u]:R["pair_off"][u + 1]]:
            t = int(p) // topk
            for wd, key in ((pb.dgate[e], "g"), (pb.dup[e], "v")):
                out = torch.empty(1, F, dtype=torch.float32, device="cuda")
                qg.qgemv_q4k(wd, F, D, pb.qx[t:t + 1], pb.dx[t:t + 1], pb.sx[t:t + 1], 1, out)
                assert np.array_equal(host(out)[0].view(np.uint32), R[key][p].view(np.uint32)), (key, p)
            out = torch.empty(1, D, dtype=torch.float32, device="cuda")
            qg.qgemv_q4k(pb.ddown[e], D, F, dev(R["hq"][p:p + 1]), dev(R["hd"][p:p + 1]), dev(R["hs"][p:p + 1]),
                         1, out)
            assert np.array_equal(host(out)[0].view(np.uint32), R["o"][p].view(np.uint32)), ("o", p)


def test_moe_largest_table(qg, orc):
    """The largest table: the most experts and the most pairs (4096 experts, 1024 tokens x
    top-8 = 8192 pairs, Zipf(1.1) popularity, small matrices D = F = 256): the table and
    the matrix-core work list exactly, and every stage of every pair and every token's
    output against the oracle."""
    E, D, F, T, topk = qg.MAX_EXPERTS, 256, 256, 1024, 8
    assert T * topk == qg.MAX_MOE_PAIRS
    progress("moe largest table E=%d T=%d topk=%d" % (E, T, topk))
    pb = MoeProblem(qg, E, D, F, T, topk, 77, zipf=True, only_selected=True)
    y, ws, st = pb.run()
    assert st == 0
    R = check_staged(qg, orc, pb, y, ws)
    counts = np.diff(R["pair_off"])
    assert counts.max() > 32 * 8 and R["n_uniq"] > 1000  # many-tile experts and a wide table
    lay = qg.moe_routed_workspace_layout(T, topk, E, D, F)
    hot = host(ws)[lay["HOT"]:].view(np.int32)
    want = [(u, m0) for u in range(R["n_uniq"]) if counts[u] >= qg.MOE_MM_PAIRS for m0 in range(0, counts[u], 32)]
    assert hot[0] == len(want)
    assert [tuple(hot[1 + 2 * i:3 + 2 * i]) for i in range(len(want))] == want


def test_moe_invariants(qg):
    pb = MoeProblem(qg, 20, 512, 256, 6, 6, 11)
    y, _, _ = pb.run()
    # deterministic
    y2, _, _ = pb.run()
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    # expert relabelling (ids and pointer tables permuted together) changes nothing
    lab = np.random.default_rng(0).permutation(pb.E)
    inv = np.argsort(lab)
    yl, _, _ = pb.run(ids=lab[pb.ids], gate=[pb.dgate[i] for i in inv], up=[pb.dup[i] for i in inv],
                      down=[pb.ddown[i] for i in inv])
    assert np.array_equal(y.view(np.uint32), yl.view(np.uint32))
    # duplicated experts inside a token's top-k are allowed; weights on duplicates add up
    ids = pb.ids.copy()
    ids[0, 1] = ids[0, 0]
    rw = pb.rw.copy()
    yd, ws, st = pb.run(ids=ids, rw=rw)
    assert st == 0 and np.all(np.isfinite(yd))


def test_moe_token_permutation(qg):
    """Rows of a permuted batch are the permuted rows (activations permuted on the host)."""
    import torch
    pb = MoeProblem(qg, 20, 512, 256, 5, 6, 12)
    y, _, _ = pb.run()
    perm = np.array([4, 2, 0, 3, 1])
    idx = perm.tolist()
    pb.qx, pb.dx, pb.sx = pb.qx[idx].contiguous(), pb.dx[idx].contiguous(), pb.sx[idx].contiguous()
    yp, _, _ = pb.run(ids=pb.ids[perm], rw=pb.rw[perm])
    assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


def test_moe_device_errors(qg):
    pb = MoeProblem(qg, 16, 512, 256, 4, 6, 13)
    base, _, _ = pb.run()
    # invalid ids: status set, the pair contributes nothing, the rest unaffected
    for bad in (-1, 16, 1 << 30):
        ids = pb.ids.copy()
        ids[2, 3] = bad
        y, ws, st = pb.run(ids=ids)
        assert st == qg.DEV_BAD_EXPERT
        rw0 = pb.rw.copy()
        rw0[2, 3] = 0.0
        yz, _, _ = pb.run(rw=rw0)
        assert np.array_equal(y[2], yz[2])
        for t in (0, 1, 3):
            assert np.array_equal(y[t], base[t])
        R = pb.regions(ws)
        assert R["slot"][2 * pb.topk + 3] == -1
    # a selected expert without weights: status set, its pairs contribute nothing
    e = int(pb.ids[1, 0])
    gate = list(pb.dgate)
    gate[e] = None
    y, ws, st = pb.run(gate=gate)
    assert st == qg.DEV_NULL_EXPERT
    R = pb.regions(ws)
    assert e not in R["uniq"].tolist()
    rw0 = np.where(pb.ids == e, 0.0, pb.rw).astype(np.float32)
    yz, _, _ = pb.run(rw=rw0)
    assert np.array_equal(y.view(np.uint32), yz.view(np.uint32))


ONE_TOKEN_CASES = ["bad_id", "null_gate", "misaligned_down", "bad_id_and_null", "all_invalid", "duplicate"]


@pytest.mark.parametrize("case", ONE_TOKEN_CASES)
def test_moe_one_token_table_and_status(qg, orc, case):
    """One token (at most 64 pairs, where the first expert launch builds the table itself):
    over a workspace filled with 0xFF, the table equals the oracle's table of the ids with every
    unusable expert's ids taken as invalid, the status word is the documented one (a bad id
    before an unusable expert), and the dropped pairs contribute exactly nothing."""
    one_token_table_case(qg, orc, case, fmt=1)


def one_token_table_case(qg, orc, case, fmt):
    E, D, F, topk = 16, 512, 256, 6
    pb = MoeProblem(qg, E, D, F, 1, topk, 21, fmt=fmt)
    ids = pb.ids.copy()
    gate, down = list(pb.dgate), list(pb.ddown)
    dropped = set()
    if case in ("bad_id", "bad_id_and_null"):
        ids[0, 3] = E
    if case in ("null_gate", "bad_id_and_null"):
        dropped.add(int(ids[0, 0]))
        gate[int(ids[0, 0])] = None
    if case == "misaligned_down":
        e = int(ids[0, 1])
        down[e] = pb.ddown[e].reshape(-1)[8:]  # 8 bytes in: never dereferenced
        assert down[e].data_ptr() % 16 == 8
        dropped.add(e)
    if case == "all_invalid":
        ids[:] = -1
    if case == "duplicate":
        ids[0, 4] = ids[0, 2]
    progress("moe one-token table fmt=%d case=%s ids=%s" % (fmt, case, ids.tolist()))
    y, ws, st = pb.run(ids=ids, gate=gate, down=down, ws_fill=0xFF)
    bad_id = bool(np.any((ids < 0) | (ids >= E)))
    assert st == (qg.DEV_BAD_EXPERT if bad_id else (qg.DEV_NULL_EXPERT if dropped else qg.DEV_OK))
    eff = np.where(np.isin(ids, sorted(dropped)), -1, ids).astype(np.int32)
    tab = orc.moe_table(eff, E)
    R = pb.regions(ws)
    assert R["n_uniq"] == tab["n_uniq"]
    assert np.array_equal(R["uniq"], tab["uniq"])
    assert np.array_equal(R["slot"], tab["slot"].ravel())
    assert np.array_equal(R["pair_off"], tab["pair_off"])
    npairs = int(tab["pair_off"][-1])
    assert np.array_equal(R["pairs"][:npairs], tab["pairs"])
    if case == "duplicate":
        pb.ids = ids
        check_staged(qg, orc, pb, y, ws)
        return
    # dropped pairs add nothing: the same as their weights set to zero with usable experts
    keep = (eff >= 0) & (eff < E)
    rw0 = np.where(keep, pb.rw, 0.0).astype(np.float32)
    yz, _, stz = pb.run(rw=rw0)
    assert stz == qg.DEV_OK
    assert np.array_equal(y.view(np.uint32), yz.view(np.uint32))
    if case == "all_invalid":
        assert R["n_uniq"] == 0 and np.all(y == 0.0)


@pytest.mark.parametrize("T,topk", [(1, 64), (1, 65), (8, 8), (5, 13)])
def test_moe_one_token_many_pairs(qg, orc, T, topk):
    """64 pairs (the table built in the first expert launch) and 65 (the table kernel), with one
    token and with several: stage-by-stage parity over a workspace filled with 0xFF."""
    progress("moe many pairs T=%d topk=%d" % (T, topk))
    pb = MoeProblem(qg, 80, 256, 256, T, topk, 22)
    y, ws, st = pb.run(ws_fill=0xFF)
    assert st == 0
    check_staged(qg, orc, pb, y, ws)


def test_moe_host_errors_touch_nothing(qg):
    import torch
    pb = MoeProblem(qg, 8, 256, 256, 2, 2, 14)
    nbytes = qg.moe_routed_workspace_bytes(2, 2, 8, 256, 256)
    assert nbytes > 0 and qg.moe_routed_workspace_bytes(2, 2, 8, 300, 256) == 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y = sentinel((2, 256), torch.float32, 5.0)
    st = sentinel((1,), torch.int32, -99)
    ids, rw = dev(pb.ids), dev(pb.rw)
    tabs = [qg.pointer_table(l, "cuda") for l in (pb.dgate, pb.dup, pb.ddown)]
    c = qg._c_moe

    def call(**kw):
        args = dict(qx=pb.qx.data_ptr(), dx=pb.dx.data_ptr(), sx=pb.sx.data_ptr(), T=2, D=256, F=256, E=8, topk=2,
                    ids=ids.data_ptr(), rw=rw.data_ptr(), gate=tabs[0].data_ptr(), up=tabs[1].data_ptr(),
                    down=tabs[2].data_ptr(), y=y.data_ptr(), ws=ws.data_ptr(), nb=nbytes, status=st.data_ptr())
        args.update(kw)
        return c(args["qx"], args["dx"], args["sx"], args["T"], args["D"], args["F"], args["E"], args["topk"],
                 args["ids"], args["rw"], args["gate"], args["up"], args["down"], args["y"], args["ws"], args["nb"],
                 args["status"], None)

    assert call(nb=nbytes - 1) == -5
    assert call(ws=None) == -1 and call(status=None) == -1 and call(gate=None) == -1
    assert call(D=300) == -2 and call(T=0) == -2 and call(E=0) == -2 and call(topk=0) == -2
    assert call(T=8193, topk=1) == -2
    assert call(qx=pb.qx.data_ptr() + 4) == -3
    assert np.all(host(y) == 5.0) and host(st)[0] == -99
