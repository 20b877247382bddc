"""GPU parity of quantise-then-dispatch (fgq_quant_dispatch_1x128).

Everything is compared bit for bit with the oracle (oracle.dispatch): the
offsets, both index maps, and the codes and scales of every routed row.
Cases: one pair; ragged routings with dropped and out-of-range ids; more
than one 256-pair routing block and a partial last block; E = 4096 (the
limit); top-1; nothing routed; T = 0; the full dispatch workload
(4096 tokens, top-8 of 32 experts, K = 7168).  Output rows past the routed
count keep their canary bytes, and the dispatched rows feed the grouped
GEMM, which must match the oracle's product of the oracle's rows.
"""
import numpy as np
import pytest

import oracle
from synth import make_workload, normal_bf16, rng_for, route_ids
from tests.gpu_util import CANARY, Guarded, dev_bf16, host_bf16_f64, log

pytestmark = pytest.mark.gpu


def _run(fgq, x, ids, E, guard=False):
    import torch
    T, K = x.shape
    topk = ids.shape[1]
    R = T * topk
    q = s = None
    if guard:
        qg = Guarded(R, K, torch.uint8)
        q = qg.view
    out = fgq.quant_dispatch_1x128(dev_bf16(x), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(), E,
                                   q=q)
    torch.cuda.synchronize()
    q, s, off, src, dest = out
    res = dict(q=q.cpu().numpy(), s=s.cpu().numpy(), off=off.cpu().numpy(), src=src.cpu().numpy(),
               dest=dest.cpu().numpy())
    if guard:
        qg.check_canaries()
        res["guard"] = qg
    return res


def _compare(res, x, ids, E, what):
    qo, so, offo, srco, desto = oracle.quant_dispatch_ref(x, ids, E)
    R = int(offo[-1])
    log(f"{what}: {R} routed rows")
    assert np.array_equal(res["off"], offo), what
    assert np.array_equal(res["dest"], desto), what
    assert np.array_equal(res["src"][:R], srco), what
    assert np.array_equal(res["q"][:R], qo), what
    assert np.array_equal(res["s"][:R].view(np.uint32), so.view(np.uint32)), what
    return R


@pytest.mark.parametrize("T,topk,E,K,drop,seed", [
    (1, 1, 1, 128, 0.0, 0),
    (5, 2, 3, 256, 0.2, 1),
    (100, 8, 32, 384, 0.05, 2),
    (777, 4, 5, 640, 0.0, 3),       # 3108 pairs: twelve full 256-pair routing blocks and a partial one
    (1000, 8, 300, 128, 0.1, 4),
    (300, 6, 4096, 128, 0.0, 5),    # the largest expert count
    (3000, 1, 7, 256, 0.0, 6),
])
def test_dispatch_routed_rows(fgq_gpu, T, topk, E, K, drop, seed):
    x = normal_bf16((T, K), 1.0, rng_for(seed, 60))
    ids = route_ids(T, topk, E, 1.1, rng_for(seed, 61), drop=drop)
    res = _run(fgq_gpu, x, ids, E, guard=True)
    R = _compare(res, x, ids, E, f"dispatch T={T} topk={topk} E={E} K={K} drop={drop}")
    # rows past the routed count are never written
    assert np.all(res["q"][R:] == CANARY)


@pytest.mark.parametrize("e8m0", [False, True])
@pytest.mark.parametrize("layout", ["row", "kmajor"])
def test_dispatch_scale_layouts(fgq_gpu, layout, e8m0):
    """Both ways the scales are written: contiguous per row (each routed row
    gets its scales from the quantiser) and K-block-major (one scale per
    token tile in the workspace, then a gather in row order).  Scales match
    the oracle bit for bit; rows past the routed count and the guard bands
    are never written."""
    import torch
    T, topk, E, K = 777, 4, 5, 640
    R = T * topk
    x = normal_bf16((T, K), 1.0, rng_for(11, 60))
    ids = route_ids(T, topk, E, 1.1, rng_for(11, 61), drop=0.1)
    dt = torch.uint8 if e8m0 else torch.float32
    if layout == "row":
        sg = Guarded(R, K // 128, dt)
        s = sg.view
    else:
        sg = Guarded(K // 128, R, dt)
        s = sg.view.t()
    fn = fgq_gpu.quant_dispatch_1x128_e8m0 if e8m0 else fgq_gpu.quant_dispatch_1x128
    q, s_out, off, src, dest = fn(dev_bf16(x), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(), E, s=s)
    torch.cuda.synchronize()
    sg.check_canaries()
    ref = oracle.quant_dispatch_e8m0_ref if e8m0 else oracle.quant_dispatch_ref
    qo, so, offo, _, _ = ref(x, ids, E)
    Rr = int(offo[-1])
    log(f"dispatch scales {layout} {'e8m0' if e8m0 else 'f32'}: {Rr} routed rows of {R}")
    sh = np.ascontiguousarray(s.cpu().numpy())
    assert np.array_equal(q.cpu().numpy()[:Rr], qo)
    assert np.array_equal(sh[:Rr].view(np.uint8), np.ascontiguousarray(so).view(np.uint8))
    assert np.all(sh[Rr:].view(np.uint8) == CANARY)


def test_dispatch_out_of_range_ids(fgq_gpu):
    rng = np.random.default_rng(7)
    T, topk, E, K = 500, 3, 9, 256
    x = normal_bf16((T, K), 1.0, rng_for(7, 60))
    ids = rng.integers(-3, E + 3, size=(T, topk)).astype(np.int32)   # repeats and invalid ids allowed
    ids[0, :] = np.iinfo(np.int32).min
    ids[1, :] = np.iinfo(np.int32).max
    res = _run(fgq_gpu, x, ids, E)
    _compare(res, x, ids, E, "dispatch with out-of-range ids")


def test_dispatch_nothing_routed_and_empty(fgq_gpu):
    import torch
    x = normal_bf16((64, 128), 1.0, rng_for(8, 60))
    ids = np.full((64, 2), -1, np.int32)
    res = _run(fgq_gpu, x, ids, 5, guard=True)
    assert res["off"].tolist() == [0] * 6 and np.all(res["dest"] == -1)
    assert np.all(res["q"] == CANARY)
    # T = 0: offsets are still written
    off = torch.full((6,), 77, dtype=torch.int32, device="cuda")
    fgq_gpu.quant_dispatch_1x128(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"),
                                 torch.empty((0, 2), dtype=torch.int32, device="cuda"), 5, offsets=off)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0] * 6


def test_dispatch_full_workload(fgq_gpu):
    """4096 tokens x top-8 of 32 experts, K = 7168: the launch the benchmark times."""
    d = make_workload("dispatch")
    x, ids, E = d["X"], d["ids"], d["E"]
    res = _run(fgq_gpu, x, ids, E)
    offo, srco, desto = oracle.dispatch_ref(ids, E)
    assert np.array_equal(res["off"], offo) and np.array_equal(res["dest"], desto)
    assert np.array_equal(res["src"], srco)
    qt, st = oracle.quant_act_1x128(x)      # every routed row is its token's quantisation
    tok = srco.astype(np.int64) // d["topk"]
    assert np.array_equal(res["q"], qt[tok])
    assert np.array_equal(res["s"].view(np.uint32), st[tok].view(np.uint32))
    log(f"dispatch workload: {int(offo[-1])} rows, expert sizes {np.diff(offo).min()}..{np.diff(offo).max()}")


@pytest.mark.parametrize("mode", [0, 1])
def test_dispatch_feeds_grouped_gemm(fgq_gpu, mode):
    """Dispatched rows straight into the grouped GEMM (total_rows = T * topk)."""
    import torch
    T, topk, E, K, N = 300, 4, 6, 512, 256
    x = normal_bf16((T, K), 1.0, rng_for(9, 60))
    ids = route_ids(T, topk, E, 1.1, rng_for(9, 61), drop=0.1)
    w = normal_bf16((E, N, K), 0.02, rng_for(9, 62))
    q, s, off, src, dest = fgq_gpu.quant_dispatch_1x128(dev_bf16(x), torch.from_numpy(ids).cuda(), E)
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(w))
    c = fgq_gpu.grouped_gemm_fp8_blockscaled(q, s, qw, sw, off, mode=mode)
    torch.cuda.synchronize()
    qo, so, offo, _, _ = oracle.quant_dispatch_ref(x, ids, E)
    qwo, swo = oracle.quant_w_128x128(w)
    ref = oracle.grouped_gemm_ref(qo, so, qwo, swo, offo)
    R = int(offo[-1])
    g = oracle.gemm_gate(host_bf16_f64(c[:R]), ref)
    log(f"dispatch -> grouped GEMM mode {mode}: normwise {g['normwise']:.3e}, max elem {g['max_elem_rel']:.3e}")
    assert g["finite"] and g["normwise"] <= 2e-3
    if mode == 0:
        assert g["ok"]


def test_dispatch_deterministic(fgq_gpu):
    """Repeated dispatches give identical offsets, maps, codes and scales,
    on the fused-scan path (few blocks) and the separate-scan path."""
    import torch
    for T, topk, E, K in ((1000, 8, 32, 256), (1000, 8, 300, 128)):
        x = dev_bf16(normal_bf16((T, K), 1.0, rng_for(12, T + E)))
        ids = torch.from_numpy(route_ids(T, topk, E, 1.1, rng_for(12, E), drop=0.05)).cuda()
        def routed(out):
            # rows past the routed count are never written: compare the rest
            q, sc, off, src, dest = out
            R = int(off[-1])
            return [q[:R], sc[:R].view(torch.int32), off, src[:R], dest]
        first = [t.clone() for t in routed(fgq_gpu.quant_dispatch_1x128(x, ids, E))]
        for rep in range(4):
            out = routed(fgq_gpu.quant_dispatch_1x128(x, ids, E))
            torch.cuda.synchronize()
            for a, b in zip(first, out):
                assert torch.equal(a, b), (T, E, rep)
    log("dispatch determinism: 5 runs identical on both scan paths")
