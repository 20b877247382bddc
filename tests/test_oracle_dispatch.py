"""Pins of the quantise-then-dispatch oracle (oracle.dispatch).

  * brute force: per-expert lists built by one pass over the pairs in index
    order (no sort), on tiny routings with dropped and out-of-range ids;
  * invariants at workload size: offsets partition the rows, row_src is a
    permutation of the routed pairs, dest inverts it, experts ascend along
    the rows and pair indices ascend inside each expert;
  * special cases: nothing routed; top-1 routing of token t to expert t is
    the identity; one expert takes every pair;
  * the codes and scales of every routed row are those of its token's row
    under quant_act_1x128 (itself pinned in test_oracle_quant.py).
"""
import numpy as np
import pytest

from oracle import dispatch_ref, quant_act_1x128, quant_dispatch_ref
from synth import make_workload, normal_bf16, rng_for, route_ids


def _brute(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    lists = [[] for _ in range(E)]
    for i, e in enumerate(flat):
        if 0 <= e < E:
            lists[e].append(i)
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(lists[e]))
    row_src = [i for e in range(E) for i in lists[e]]
    dest = [-1] * len(flat)
    for r, i in enumerate(row_src):
        dest[i] = r
    return offsets, row_src, dest


@pytest.mark.parametrize("T,topk,E,seed", [(1, 1, 1, 0), (5, 2, 3, 1), (17, 4, 6, 2), (64, 8, 32, 3), (33, 3, 5, 4)])
def test_dispatch_brute_force(T, topk, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, topk)).astype(np.int32)   # includes ids that are not routed
    off, src, dest = dispatch_ref(ids, E)
    b_off, b_src, b_dest = _brute(ids, E)
    assert off.tolist() == b_off and src.tolist() == b_src and dest.tolist() == b_dest


def _check_invariants(ids, E, off, src, dest):
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    R = int(valid.sum())
    assert off[0] == 0 and off[-1] == R and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(src), np.nonzero(valid)[0])
    assert np.array_equal(dest[src], np.arange(R)) and np.all(dest[~valid] == -1)
    e_of_row = flat[src]
    assert np.all(np.diff(e_of_row) >= 0)
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_dispatch_invariants_workload():
    d = make_workload("dispatch", parts={"ids"})
    off, src, dest = dispatch_ref(d["ids"], d["E"])
    _check_invariants(d["ids"], d["E"], off, src, dest)
    assert off[-1] == d["T"] * d["topk"]   # every slot is routed in the workload


def test_dispatch_invariants_with_drops():
    ids = route_ids(3000, 6, 40, 1.1, rng_for(9, 52), drop=0.1)
    off, src, dest = dispatch_ref(ids, 40)
    _check_invariants(ids, 40, off, src, dest)
    assert 0 < off[-1] < ids.size


def test_dispatch_special_cases():
    ids = np.full((7, 3), -1, np.int32)
    off, src, dest = dispatch_ref(ids, 4)
    assert off.tolist() == [0] * 5 and src.size == 0 and np.all(dest == -1)
    ids = np.arange(10, dtype=np.int32)[:, None]
    off, src, dest = dispatch_ref(ids, 10)
    assert off.tolist() == list(range(11)) and src.tolist() == list(range(10)) and dest.tolist() == list(range(10))
    ids = np.zeros((9, 2), np.int32)
    off, src, dest = dispatch_ref(ids, 3)
    assert off.tolist() == [0, 18, 18, 18] and src.tolist() == list(range(18))


def test_quant_dispatch_rows_are_token_quantisations():
    T, topk, E, K = 50, 4, 7, 384
    x = normal_bf16((T, K), 1.0, rng_for(10, 53))
    ids = route_ids(T, topk, E, 1.1, rng_for(10, 54), drop=0.05)
    q, s, off, src, dest = quant_dispatch_ref(x, ids, E)
    qt, st = quant_act_1x128(x)
    tok = src.astype(np.int64) // topk
    assert q.shape == (off[-1], K) and s.shape == (off[-1], K // 128)
    assert np.array_equal(q, qt[tok]) and np.array_equal(s.view(np.uint32), st[tok].view(np.uint32))
