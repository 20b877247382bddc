"""GPU parity of the block-scaled FP8 GEMM and its grouped variant.

Gate (from the workload definition): normwise relative error <= 2e-3 against
the oracle's float64 result from the same dequantised operands, and
elementwise <= 1e-2 relative wherever |ref| > 1e-2 * rms(ref).  The default
mode (exact products on the FP16 matrix cores) must meet it everywhere.

The FP8-matrix-core mode sums each group of 8 consecutive products in a
window about 13 bits below the group's largest product (measured on gfx950,
see tests/test_gpu_mfma_precision.py), so its elementwise check adds that
window's worst case to the tolerance:
    |C - C*| <= 1e-2 |C*| + sum_kb |sa sw| * sum_groups 8 * 2**-12 * max_g |a b|
(the normwise gate is unchanged).

  * exact pin: integer-valued codes with power-of-two scales make every
    partial sum exact in binary32, so the GPU result must equal the oracle's
    result rounded to BF16, bit for bit, at K = 7168;
  * one-hot rows pin the scale indexing across tiles;
  * the tolerance gate on every workload: whole problems at reduced rows
    (operands quantised by the oracle, so the GEMM is tested on its own),
    and the full sizes in the benchmark's launch configuration, quantised on
    the GPU and checked on sampled rows against the oracle's own
    quantisation and product;
  * ragged M, K = 128, strided operands, guard bands around C;
  * grouped: empty experts, one expert holding every row, single-row
    experts, counts that are not multiples of the tile, E = 1 equals dense.
"""
import math

import numpy as np
import pytest

import oracle
from synth import make_workload, normal_bf16, rng_for
from tests.gpu_util import Guarded, dev_bf16, dev_f32, dev_u8, host_bf16_f64, log

pytestmark = pytest.mark.gpu


MODES = [0, 1]   # fgq.GEMM_EXACT, fgq.GEMM_FP8_CORE


def fp8_core_slack(qa, sa, qw, sw, rows, cols):
    """Worst-case truncation of the FP8 matrix core's 8-product groups for the
    selected outputs (float64): sum over chunks and groups of 8 * 2**-12 times
    the group's largest |product|, times |sa sw|."""
    A = oracle.e4m3_decode(qa[rows]).astype(np.float64)
    W = oracle.e4m3_decode(qw[cols]).astype(np.float64)
    M, K = A.shape
    N = W.shape[0]
    out = np.zeros((M, N))
    for kb in range(K // 128):
        a = np.abs(A[:, 128 * kb:128 * kb + 128]).reshape(M, 16, 8)
        w = np.abs(W[:, 128 * kb:128 * kb + 128]).reshape(N, 16, 8)
        gmax = np.max(a[:, None, :, :] * w[None, :, :, :], axis=3).sum(axis=2)   # [M, N]
        scale = np.abs(sa[rows, kb][:, None] * sw[np.asarray(cols) // 128, kb][None, :])
        out += 8 * 2.0 ** -12 * gmax * scale
    return out


def fp8_core_slack_all(qa, sa, qw, sw):
    """fp8_core_slack loosened so that it covers every output of C = A W^T at
    once: a group's largest |product| is at most the group's largest |a|
    times its largest |w|, so the sum over groups is a product of the two
    group-maximum matrices.  E4M3 magnitudes increase with the code's low
    seven bits, so the maxima are taken on the codes and decoded once."""
    M, K = qa.shape
    N = qw.shape[0]
    amax = oracle.e4m3_decode((qa & 0x7F).reshape(M, K // 8, 8).max(axis=2)).astype(np.float64)
    wmax = oracle.e4m3_decode((qw & 0x7F).reshape(N, K // 8, 8).max(axis=2)).astype(np.float64)
    out = np.zeros((M, N))
    for kb in range(K // 128):
        g = slice(16 * kb, 16 * kb + 16)
        scale = np.abs(sa[:, kb][:, None] * sw[np.arange(N) // 128, kb][None, :])
        out += 8 * 2.0 ** -12 * (amax[:, g] @ wmax[:, g].T) * scale
    return out


def _check(c, ref, what, mode, qa=None, sa=None, qw=None, sw=None, rows=None):
    if mode == 0:
        return _gate(c, ref, what)
    g = oracle.gemm_gate(c, ref)
    log(f"{what} [fp8 core]: normwise {g['normwise']:.3e}, max elem {g['max_elem_rel']:.3e}")
    assert g["finite"] and g["normwise"] <= 2e-3, (what, g)
    rng = np.random.default_rng(0)
    M, N = ref.shape
    rs = np.arange(M) if M <= 64 else np.sort(rng.choice(M, 64, replace=False))
    cs = np.arange(N) if N <= 512 else np.sort(rng.choice(N, 512, replace=False))
    src_rows = np.asarray(rows)[rs] if rows is not None else rs
    slack = fp8_core_slack(qa, sa, qw, sw, src_rows, cs)
    sub_c, sub_r = c[np.ix_(rs, cs)], ref[np.ix_(rs, cs)]
    assert np.all(np.abs(sub_c - sub_r) <= 1e-2 * np.abs(sub_r) + slack), what
    # every output, against the looser bound from the group maxima
    all_rows = np.asarray(rows) if rows is not None else np.arange(M)
    loose = fp8_core_slack_all(qa[all_rows], sa[all_rows], qw, sw)
    assert np.all(np.abs(c - ref) <= 1e-2 * np.abs(ref) + loose), (what, "all outputs")
    return g


def _gemm(fgq, qa, sa, qw, sw, ldc=None, lda=None, mode=0, sa_kmajor=False):
    import torch
    M, K = qa.shape
    N = qw.shape[0]
    if lda is not None:
        pad = np.zeros((M, lda), np.uint8)
        pad[:, :K] = qa
        qa_d = dev_u8(pad)[:, :K]
    else:
        qa_d = dev_u8(qa)
    cg = Guarded(M, N, torch.bfloat16, ld=ldc)
    sa_d = dev_f32(np.ascontiguousarray(sa.T)).t() if sa_kmajor else dev_f32(sa)
    fgq.gemm_fp8_blockscaled(qa_d, sa_d, dev_u8(qw), dev_f32(sw), out=cg.view, mode=mode)
    torch.cuda.synchronize()
    cg.check_canaries()
    return host_bf16_f64(cg.view)


def _gate(c, ref, what):
    g = oracle.gemm_gate(c, ref)
    floor = oracle.gemm_gate(oracle.bf16_round_f64(ref), ref)["normwise"]
    log(f"{what}: normwise {g['normwise']:.3e} (bf16 floor {floor:.3e}), max elem {g['max_elem_rel']:.3e}")
    assert g["ok"], (what, g)
    return g


def _int_codes(shape, rng):
    ints = rng.integers(-8, 9, size=shape)
    table = {0: 0}
    for v in range(1, 9):
        e = int(math.floor(math.log2(v)))
        table[v] = ((e + 7) << 3) | int((v / 2 ** e - 1) * 8)
        table[-v] = table[v] | 0x80
    lut = np.array([table[v] for v in range(-8, 9)], dtype=np.uint8)
    return lut[ints + 8]


@pytest.mark.parametrize("mode", MODES)
def test_gemm_integer_codes_bit_exact(fgq_gpu, mode):
    rng = np.random.default_rng(0)
    M, N, K = 200, 384, 7168
    qa, qw = _int_codes((M, K), rng), _int_codes((N, K), rng)
    sa = (2.0 ** rng.integers(-1, 2, (M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-1, 2, (N // 128, K // 128))).astype(np.float32)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    c = _gemm(fgq_gpu, qa, sa, qw, sw, mode=mode)
    assert np.array_equal(c, oracle.bf16_round_f64(ref))


@pytest.mark.parametrize("mode", MODES)
def test_gemm_one_hot_scale_indexing(fgq_gpu, mode):
    rng = np.random.default_rng(1)
    M, N, K = 150, 512, 1024
    qa = np.zeros((M, K), np.uint8)
    ks = rng.integers(0, K, M)
    qa[np.arange(M), ks] = 0x38
    qw = np.full((N, K), 0x38, np.uint8)
    sa = rng.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    c = _gemm(fgq_gpu, qa, sa, qw, sw, mode=mode)
    # one product per output: exact up to the rounding of sa*sw and the BF16 output
    assert np.all(np.abs(c - ref) <= np.abs(ref) * (2.0 ** -8 + 2.0 ** -22))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lda,ldc", [(1, 128, 128, None, None), (129, 256, 384, None, None),
                                           (300, 384, 1024, 1040, 392), (64, 128, 7168, None, None),
                                           (255, 640, 2048, None, 648), (513, 768, 512, None, None),
                                           (256, 256, 256, None, None)])
def test_gemm_shapes_oracle_operands(fgq_gpu, M, N, K, lda, ldc, mode):
    a = normal_bf16((M, K), 1.0, rng_for(5, M))
    w = normal_bf16((N, K), 0.02, rng_for(5, N + 1))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    c = _gemm(fgq_gpu, qa, sa, qw, sw, ldc=ldc, lda=lda, mode=mode)
    _check(c, ref, f"gemm {M}x{N}x{K}", mode, qa, sa, qw, sw)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", [(129, 256, 384), (300, 512, 1024), (64, 128, 7168)])
def test_gemm_scale_layouts_agree(fgq_gpu, M, N, K, mode):
    """Activation scales stored K-block-major (strides (1, M)) give the same
    bits as row-major storage, and pass the gate."""
    a = normal_bf16((M, K), 1.0, rng_for(8, M))
    w = normal_bf16((N, K), 0.02, rng_for(8, N + 1))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    c_row = _gemm(fgq_gpu, qa, sa, qw, sw, mode=mode)
    c_kmaj = _gemm(fgq_gpu, qa, sa, qw, sw, mode=mode, sa_kmajor=True)
    assert np.array_equal(c_row, c_kmaj)
    _check(c_kmaj, oracle.gemm_ref(qa, sa, qw, sw), f"gemm {M}x{N}x{K} K-major scales", mode, qa, sa, qw, sw)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name,rows", [("tiny", None), ("decode", None), ("prefill", 384)])
def test_gemm_workloads_oracle_operands(fgq_gpu, name, rows, mode):
    d = make_workload(name, rows=rows)
    qa, sa = oracle.quant_act_1x128(d["A"])
    qw, sw = oracle.quant_w_128x128(d["W"])
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    c = _gemm(fgq_gpu, qa, sa, qw, sw, mode=mode)
    _check(c, ref, f"gemm {name}", mode, qa, sa, qw, sw)
    # reported, not gated: distance to the unquantised BF16 product
    a64 = oracle.f32_from_bf16(d["A"]).astype(np.float64)
    w64 = oracle.f32_from_bf16(d["W"]).astype(np.float64)
    exact = a64 @ w64.T
    log(f"  vs unquantised BF16 operands: normwise {np.linalg.norm(c - exact) / np.linalg.norm(exact):.3e}")


@pytest.mark.parametrize("mode", MODES)
def test_gemm_prefill_full_size_sampled(fgq_gpu, mode):
    """8192x7168x18432 end to end on the GPU (quantise A and W, GEMM) as the
    benchmark runs it; 192 sampled rows against the oracle's own
    quantisation and float64 product."""
    import torch
    d = make_workload("prefill")
    A, W = d["A"], d["W"]
    qa, sa = fgq_gpu.quant_act_1x128(dev_bf16(A))
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(W))
    c = fgq_gpu.gemm_fp8_blockscaled(qa, sa, qw, sw, mode=mode)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(A.shape[0], 192, replace=False))
    rows[0], rows[-1] = 0, A.shape[0] - 1
    qao, sao = oracle.quant_act_1x128(A[rows])
    qwo, swo = oracle.quant_w_128x128(W)
    ref = oracle.gemm_ref(qao, sao, qwo, swo)
    _check(host_bf16_f64(c[rows.tolist()]), ref, "prefill full (sampled rows)", mode, qao, sao, qwo, swo)


# ------------------------------------------------------------------ grouped

def _grouped(fgq, qa, sa, qw, sw, offsets, mode=0):
    import torch
    R = qa.shape[0]
    N = qw.shape[1]
    cg = Guarded(R, N, torch.bfloat16)
    fgq.grouped_gemm_fp8_blockscaled(dev_u8(qa), dev_f32(sa), dev_u8(qw), dev_f32(sw),
                                     torch.from_numpy(np.asarray(offsets, np.int32)).cuda(), out=cg.view,
                                     mode=mode)
    torch.cuda.synchronize()
    cg.check_canaries()
    return host_bf16_f64(cg.view)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("counts", [[0, 200, 0, 57], [300, 0, 0, 0], [1, 1, 1, 130], [0, 0, 0, 5],
                                    [129, 127, 128, 256], [0, 700, 1, 0, 256, 255]])
def test_grouped_ragged_counts(fgq_gpu, counts, mode):
    E, N, K = len(counts), 256, 512
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    a = normal_bf16((R, K), 1.0, rng_for(6, R))
    w = normal_bf16((E, N, K), 0.02, rng_for(6, 7))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    ref = oracle.grouped_gemm_ref(qa, sa, qw, sw, off)
    c = _grouped(fgq_gpu, qa, sa, qw, sw, off, mode=mode)
    if mode == 0:
        _gate(c, ref, f"grouped {counts}")
    else:
        _check_grouped_fp8(c, ref, qa, sa, qw, sw, off, f"grouped {counts}")


def _check_grouped_fp8(c, ref, qa, sa, qw, sw, off, what):
    g = oracle.gemm_gate(c, ref)
    log(f"{what} [fp8 core]: normwise {g['normwise']:.3e}, max elem {g['max_elem_rel']:.3e}")
    assert g["finite"] and g["normwise"] <= 2e-3, (what, g)
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            rows = np.arange(r0, min(r1, r0 + 32))
            cols = np.arange(min(qw.shape[1], 256))
            slack = fp8_core_slack(qa, sa, qw[e], sw[e], rows, cols)
            sub_c, sub_r = c[np.ix_(rows, cols)], ref[np.ix_(rows, cols)]
            assert np.all(np.abs(sub_c - sub_r) <= 1e-2 * np.abs(sub_r) + slack), (what, e)
            # every row of the expert, against the looser bound
            loose = fp8_core_slack_all(qa[r0:r1], sa[r0:r1], qw[e], sw[e])
            assert np.all(np.abs(c[r0:r1] - ref[r0:r1]) <= 1e-2 * np.abs(ref[r0:r1]) + loose), (what, e, "all")


@pytest.mark.parametrize("mode", MODES)
def test_grouped_single_expert_equals_dense(fgq_gpu, mode):
    M, N, K = 333, 384, 1024
    a = normal_bf16((M, K), 1.0, rng_for(7, 1))
    w = normal_bf16((1, N, K), 0.02, rng_for(7, 2))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    g = _grouped(fgq_gpu, qa, sa, qw, sw, [0, M], mode=mode)
    d = _gemm(fgq_gpu, qa, sa, qw[0], sw[0], mode=mode)
    assert np.array_equal(g, d)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["grouped_up", "fused_down"])
def test_grouped_workloads_reduced_rows(fgq_gpu, name, mode):
    d = make_workload(name, rows=1500)
    qa, sa = oracle.quant_act_1x128(d["A"])
    qw, sw = oracle.quant_w_128x128(d["W"])
    ref = oracle.grouped_gemm_ref(qa, sa, qw, sw, d["offsets"])
    c = _grouped(fgq_gpu, qa, sa, qw, sw, d["offsets"], mode=mode)
    what = f"{name} rows={d['R']} counts={d['counts'].tolist()}"
    if mode == 0:
        _gate(c, ref, what)
    else:
        _check_grouped_fp8(c, ref, qa, sa, qw, sw, d["offsets"], what)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["grouped_up", "fused_down"])
def test_grouped_full_size_sampled(fgq_gpu, name, mode):
    """Full grouped problem quantised and multiplied on the GPU; for a few
    experts (the largest, a small one, the last non-empty) sampled rows are
    checked against the oracle's own quantisation and product."""
    import torch
    d = make_workload(name)
    A, W, off = d["A"], d["W"], d["offsets"]
    qa, sa = fgq_gpu.quant_act_1x128(dev_bf16(A))
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(W))
    c = fgq_gpu.grouped_gemm_fp8_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).cuda(), mode=mode)
    torch.cuda.synchronize()
    counts = d["counts"]
    nz = np.nonzero(counts)[0]
    pick = {int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), int(nz[-1])}
    rng = np.random.default_rng(3)
    for e in sorted(pick):
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 64)]))
        qao, sao = oracle.quant_act_1x128(A[rows])
        qwo, swo = oracle.quant_w_128x128(W[e])
        ref = oracle.gemm_ref(qao, sao, qwo, swo)
        _check(host_bf16_f64(c[rows.tolist()]), ref, f"{name} full, expert {e} ({r1 - r0} rows)", mode,
               qao, sao, qwo, swo)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_moe_decode_full_size(fgq_gpu, mode):
    """Decode-shaped MoE (256 tokens, top-8 of 32 experts, at most 256 rows per
    expert) dispatched and multiplied on the GPU, as the benchmark runs it;
    every row of three experts (the largest, a small one, the last) is checked
    against the oracle's own dispatch, quantisation and product."""
    import torch
    d = make_workload("moe_decode")
    X, W, ids, E = d["X"], d["W"], d["ids"], d["E"]
    qa, sa, off, _, _ = fgq_gpu.quant_dispatch_1x128(dev_bf16(X), torch.from_numpy(ids).cuda(), E)
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(W))
    c = fgq_gpu.grouped_gemm_fp8_blockscaled(qa, sa, qw, sw, off, mode=mode)
    torch.cuda.synchronize()
    offo, srco, _ = oracle.dispatch_ref(ids, E)
    assert np.array_equal(off.cpu().numpy(), offo)
    counts = np.diff(offo)
    nz = np.nonzero(counts)[0]
    for e in sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), int(nz[-1])}):
        r0, r1 = int(offo[e]), int(offo[e + 1])
        toks = srco[r0:r1].astype(np.int64) // d["topk"]
        qao, sao = oracle.quant_act_1x128(X[toks])
        qwo, swo = oracle.quant_w_128x128(W[e])
        ref = oracle.gemm_ref(qao, sao, qwo, swo)
        _check(host_bf16_f64(c[r0:r1]), ref, f"moe_decode expert {e} ({r1 - r0} rows)", mode, qao, sao, qwo, swo)


@pytest.mark.parametrize("mode", MODES)
def test_gemm_and_grouped_deterministic(fgq_gpu, mode):
    """Repeated calls on the same inputs give byte-identical C on the
    large-tile path, the split-K path (a decode shape) and the grouped path,
    with other launches in between: nothing depends on timing (no atomics,
    fixed reduction orders)."""
    import torch
    E = 4
    a = dev_bf16(normal_bf16((640, 2048), 1.0, rng_for(40, 1)))
    ad = dev_bf16(normal_bf16((64, 7168), 1.0, rng_for(40, 2)))
    w = dev_bf16(normal_bf16((1024, 2048), 0.02, rng_for(40, 3)))
    wd = dev_bf16(normal_bf16((4096, 7168), 0.02, rng_for(40, 4)))
    wg = dev_bf16(normal_bf16((E, 256, 2048), 0.02, rng_for(40, 5)))
    qa, sa = fgq_gpu.quant_act_1x128(a)
    qad, sad = fgq_gpu.quant_act_1x128(ad)
    qw, sw = fgq_gpu.quant_w_128x128(w)
    qwd, swd = fgq_gpu.quant_w_128x128(wd)
    qwg, swg = fgq_gpu.quant_w_128x128(wg)
    off = torch.tensor([0, 300, 300, 557, 640], dtype=torch.int32, device="cuda")
    runs = {
        "dense": lambda: fgq_gpu.gemm_fp8_blockscaled(qa, sa, qw, sw, mode=mode),
        "split-K": lambda: fgq_gpu.gemm_fp8_blockscaled(qad, sad, qwd, swd, mode=mode),
        "grouped": lambda: fgq_gpu.grouped_gemm_fp8_blockscaled(qa, sa, qwg, swg, off, mode=mode),
    }
    first = {k: f().clone() for k, f in runs.items()}
    for rep in range(4):
        for k, f in runs.items():
            c = f()
            torch.cuda.synchronize()
            assert torch.equal(c.view(torch.int16), first[k].view(torch.int16)), (k, rep)
    log(f"GEMM determinism mode {mode}: 5 runs each of dense, split-K and grouped identical")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", [(2112, 6144, 2560), (2816, 6144, 2560)])
def test_gemm_last_round_split(fgq_gpu, M, N, K, mode):
    """Large products whose last round of tiles is split along K into
    partial sums in the workspace (2112 rows: the exact mode's 264 tiles are
    one round and 8; 2816 rows: both modes, up to 5 parts): the tolerance
    gate with the workspace, and without one (the plain launch).  K is above
    2048, where the exact mode takes its large tiles."""
    import torch
    a = normal_bf16((M, K), 1.0, rng_for(41, M))
    w = normal_bf16((N, K), 0.02, rng_for(41, N))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    ref = oracle.gemm_ref(qa, sa, qw, sw)
    assert fgq_gpu.gemm_workspace_bytes(M, N, K) > 0
    qa_d, sa_d, qw_d, sw_d = dev_u8(qa), dev_f32(sa), dev_u8(qw), dev_f32(sw)
    c_split = fgq_gpu.gemm_fp8_blockscaled(qa_d, sa_d, qw_d, sw_d, mode=mode)
    c_plain = fgq_gpu.gemm_fp8_blockscaled(qa_d, sa_d, qw_d, sw_d, mode=mode,
                                           workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    _check(host_bf16_f64(c_split), ref, f"last-round split {M}x{N}x{K}", mode, qa, sa, qw, sw)
    _check(host_bf16_f64(c_plain), ref, f"plain {M}x{N}x{K}", mode, qa, sa, qw, sw)


def test_gemm_on_side_stream_keeps_its_scratch(fgq_gpu):
    # A call on a stream other than the current one allocates its output and
    # split-K workspace from that stream's pool: memory allocated and written
    # on the current stream right after the call cannot be the workspace the
    # kernels are still writing.  Checked against the same call on the current
    # stream, bit for bit.
    import torch
    rng = np.random.default_rng(3)
    M, N, K = 64, 4096, 7168
    qa = _int_codes((M, K), rng)
    qw = _int_codes((N, K), rng)
    sa = (2.0 ** rng.integers(-1, 2, (M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-1, 2, (N // 128, K // 128))).astype(np.float32)
    assert fgq_gpu.gemm_workspace_bytes(M, N, K) > 0      # the split-K path, which needs scratch
    qa_d, qw_d, sa_d, sw_d = dev_u8(qa), dev_u8(qw), dev_f32(sa), dev_f32(sw)
    want = fgq_gpu.gemm_fp8_blockscaled(qa_d, sa_d, qw_d, sw_d)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs, fills = [], []
    for _ in range(4):
        outs.append(fgq_gpu.gemm_fp8_blockscaled(qa_d, sa_d, qw_d, sw_d, stream=side))
        # allocate and write on the current stream while the side stream runs
        fills.append(torch.full((fgq_gpu.gemm_workspace_bytes(M, N, K) // 4,), 7.0, device="cuda"))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = want.view(torch.int16).cpu().numpy()
    for o in outs:
        assert np.array_equal(o.view(torch.int16).cpu().numpy(), ref)
    for f in fills:
        assert bool((f == 7.0).all())
