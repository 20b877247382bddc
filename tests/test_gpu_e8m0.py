"""GPU parity of the power-of-two (E8M0) scale variant.

Quantisers: codes and scale bytes byte-identical to ``oracle.e8m0``
(activation tiles, weight blocks, fused RMSNorm): zero, subnormal-only,
huge and power-of-two-maximum tiles, ragged rows, row-major, K-block-major
and odd-address byte layouts, guard bands around every output, and the full
workload sizes on sampled rows.

GEMMs (scales applied by the matrix core):
  * promote: the gate of the binary32-scale GEMM's FP8-core mode (normwise
    2e-3 and the 8-product window slack elementwise), exact on integer
    codes, and bit-identical to that FP8-core mode when it is given the same
    power-of-two scales as binary32 (same tiles, same chunk order, and the
    unit's scaling is exact);
  * in-core: the unit aligns its accumulator operand and the chunk's
    8-product group sums to the largest of them and truncates about 24 bits
    below (pinned below through the debug entry); the elementwise bound adds
    that loss per chunk to the promote slack, and the normwise gate is the
    same 2e-3;
  * grouped: ragged counts, one expert equals dense, the decode-shaped MoE
    workload dispatched on the GPU.
"""
import numpy as np
import pytest

import oracle
from synth import bf16_bits_from_f32, make_workload, normal_bf16, rng_for
from tests.gpu_util import Guarded, dev_bf16, dev_f32, dev_u8, host_bf16_f64, log
from tests.test_gpu_gemm import fp8_core_slack, fp8_core_slack_all

pytestmark = pytest.mark.gpu

PROMOTE, IN_CORE = 0, 1
ACCS = [PROMOTE, IN_CORE]


# ------------------------------------------------------------------ quantisers

def _scale_buffer(rows, cols, layout):
    """Guarded uint8 scale output of logical shape [rows, cols] in one of three
    layouts; returns (guard, view)."""
    import torch
    if layout == "row":
        g = Guarded(rows, cols, torch.uint8)
        return g, g.view
    if layout == "kmajor":
        g = Guarded(cols, rows, torch.uint8)
        return g, g.view.t()
    # "odd": row-major, starting one byte past an aligned address
    g = Guarded(1, rows * cols + 1, torch.uint8)
    return g, g.view[0, 1:].view(rows, cols)


def _q8_act(fgq, x_bits, layout="row"):
    import torch
    M, K = x_bits.shape
    qg = Guarded(M, K, torch.uint8)
    sg, s = _scale_buffer(M, K // 128, layout)
    fgq.quant_act_1x128_e8m0(dev_bf16(x_bits), q=qg.view, s=s)
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    return qg.view.cpu().numpy(), s.cpu().numpy()


def _same(q, b, qo, bo, what):
    assert q.shape == qo.shape and b.shape == bo.shape, what
    bad = np.nonzero(q != qo)
    assert bad[0].size == 0, f"{what}: {bad[0].size} code mismatches, first at {tuple(x[0] for x in bad)}"
    badb = np.nonzero(b != bo)
    assert badb[0].size == 0, f"{what}: {badb[0].size} scale mismatches, first at {tuple(x[0] for x in badb)}"


@pytest.mark.parametrize("layout", ["row", "kmajor", "odd"])
@pytest.mark.parametrize("M,K", [(1, 128), (37, 640), (300, 7168), (1000, 2048)])
def test_quant_act_e8m0(fgq_gpu, M, K, layout):
    log(f"quant_act_1x128_e8m0 {M}x{K} {layout}")
    x = normal_bf16((M, K), 1.0, rng_for(11, M + K))
    q, b = _q8_act(fgq_gpu, x, layout)
    qo, bo = oracle.quant_act_1x128_e8m0(x)
    _same(q, b, qo, bo, f"act e8m0 {M}x{K} {layout}")


def _special_tiles():
    rng = rng_for(12, 1)
    x = normal_bf16((8, 1536), 1.0, rng)
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(8, 12, 128).copy()
    xf[0, 0] = 0.0                                                       # all zero
    xf[0, 1] = -0.0                                                      # all negative zero
    xf[0, 2] = np.ldexp(np.float32(1.0), -133) * rng.integers(-3, 4, 128)  # BF16 subnormals only
    xf[0, 3] *= np.float32(1e30)                                         # huge
    xf[0, 4] *= np.float32(1e-30)                                        # tiny normals
    xf[0, 5, 7] = np.float32(3.3895313892515355e38)                      # largest BF16
    for kb in range(6, 12):                                              # max-abs exactly 448 * 2^k
        k = kb * 3 - 20
        xf[0, kb] = np.clip(xf[0, kb], -3, 3) * np.float32(2.0 ** (k + 7))
        xf[0, kb, kb] = np.float32(448.0 * 2.0 ** k)
    for kb in range(12):                                                 # max-abs just above 448 * 2^k
        k = kb - 6
        xf[1, kb] = np.clip(xf[1, kb], -3, 3) * np.float32(2.0 ** (k + 7))
        xf[1, kb, 3] = -np.float32(448.0 * 2.0 ** k) * np.float32(1 + 2 ** -7)
    xf[2] *= np.float32(-1.0)
    return bf16_bits_from_f32(xf.reshape(8, 1536))


@pytest.mark.parametrize("layout", ["row", "kmajor"])
def test_quant_act_e8m0_special_tiles(fgq_gpu, layout):
    x = _special_tiles()
    q, b = _q8_act(fgq_gpu, x, layout)
    qo, bo = oracle.quant_act_1x128_e8m0(x)
    _same(q, b, qo, bo, f"act e8m0 special tiles {layout}")
    assert b[0, 0] == 0 and b[0, 1] == 0 and b[0, 2] == 0
    assert np.all(q[0, 128:256] == 0x80)                                 # -0 keeps its sign


@pytest.mark.parametrize("shape", [(128, 128), (3, 256, 384), (1024, 7168)])
def test_quant_w_e8m0(fgq_gpu, shape):
    import torch
    log(f"quant_w_128x128_e8m0 {shape}")
    w = normal_bf16(shape, 0.02, rng_for(13, shape[-1]))
    if len(shape) == 3:
        w[1, 5, 130] = bf16_bits_from_f32(np.array([7.0], np.float32))[0]   # one block with an outlier
    q, s = fgq_gpu.quant_w_128x128_e8m0(dev_bf16(w))
    torch.cuda.synchronize()
    qo, so = oracle.quant_w_128x128_e8m0(w)
    _same(q.cpu().numpy(), s.cpu().numpy(), qo, so, f"w e8m0 {shape}")


@pytest.mark.parametrize("M,K", [(1, 128), (5, 640), (33, 2048), (7, 7168), (4103, 7168), (3, 16384)])
def test_fused_rmsnorm_e8m0(fgq_gpu, M, K):
    import torch
    log(f"fused_rmsnorm_quant_e8m0 {M}x{K}")
    x = normal_bf16((M, K), 1.5, rng_for(14, K))
    g = normal_bf16((K,), 1.0, rng_for(14, K + 1))
    qg = Guarded(M, K, torch.uint8)
    sg, s = _scale_buffer(M, K // 128, "kmajor")
    fgq_gpu.fused_rmsnorm_quant_e8m0(dev_bf16(x), dev_bf16(g), 1e-6, q=qg.view, s=s)
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    qo, bo = oracle.fused_rmsnorm_quant_e8m0(x, g, 1e-6)
    _same(qg.view.cpu().numpy(), s.cpu().numpy(), qo, bo, f"fused e8m0 {M}x{K}")


def test_quant_e8m0_full_size_sampled(fgq_gpu):
    """The prefill activations (8192 x 7168) and weights (18432 x 7168) on the
    GPU; sampled rows and weight row blocks against the oracle."""
    import torch
    d = make_workload("prefill")
    A, W = d["A"], d["W"]
    q, b = fgq_gpu.quant_act_1x128_e8m0(dev_bf16(A))
    qw, bw = fgq_gpu.quant_w_128x128_e8m0(dev_bf16(W))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(4).choice(A.shape[0], 256, replace=False))
    qo, bo = oracle.quant_act_1x128_e8m0(A[rows])
    _same(q.cpu().numpy()[rows], b.cpu().numpy()[rows], qo, bo, "prefill A e8m0 (sampled rows)")
    qwh, bwh = qw.cpu().numpy(), bw.cpu().numpy()
    for nb in (0, 77, W.shape[0] // 128 - 1):
        qwo, bwo = oracle.quant_w_128x128_e8m0(W[nb * 128:(nb + 1) * 128])
        _same(qwh[nb * 128:(nb + 1) * 128], bwh[nb:nb + 1], qwo, bwo, f"prefill W e8m0 block row {nb}")


@pytest.mark.parametrize("T,topk,E,K,drop", [(1, 1, 1, 128, 0.0), (777, 4, 5, 640, 0.1), (300, 6, 4096, 128, 0.0),
                                              (4096, 8, 32, 7168, 0.0)])
def test_quant_dispatch_e8m0(fgq_gpu, T, topk, E, K, drop):
    """Quantise-then-dispatch with E8M0 scales: routing, codes and scale bytes
    bit for bit (the last case is the dispatch workload's size)."""
    import torch
    from synth import route_ids
    log(f"quant_dispatch_1x128_e8m0 T={T} topk={topk} E={E} K={K}")
    x = normal_bf16((T, K), 1.0, rng_for(15, T))
    ids = route_ids(T, topk, E, 1.1, rng_for(15, T + 1), drop=drop)
    qg = Guarded(T * topk, K, torch.uint8)
    q, b, off, src, dest = fgq_gpu.quant_dispatch_1x128_e8m0(dev_bf16(x), torch.from_numpy(ids).cuda(), E, q=qg.view)
    torch.cuda.synchronize()
    qg.check_canaries()
    qo, bo, offo, srco, desto = oracle.quant_dispatch_e8m0_ref(x, ids, E)
    R = int(offo[-1])
    assert np.array_equal(off.cpu().numpy(), offo) and np.array_equal(dest.cpu().numpy(), desto)
    assert np.array_equal(src.cpu().numpy()[:R], srco)
    _same(q.cpu().numpy()[:R], b.cpu().numpy()[:R], qo, bo, f"dispatch e8m0 T={T}")


# ------------------------------------------------------------------ the scaled matrix-core operation

def _unit(fgq, A, B, sa, sb, C):
    import torch
    qa = oracle.e4m3_encode(np.asarray(A, np.float32))
    qb = oracle.e4m3_encode(np.asarray(B, np.float32))
    d = fgq.debug_mfma_e8m0_16x16x128(dev_u8(qa), dev_u8(qb), dev_u8(np.asarray(sa, np.uint8)),
                                      dev_u8(np.asarray(sb, np.uint8)), dev_f32(C))
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def test_unit_scaling_is_exact(fgq_gpu):
    """With a zero accumulator, the scaled operation is the unscaled one times
    2^(sa - 127) 2^(sb - 127), exactly, per row of A and column of B."""
    import torch
    rng = np.random.default_rng(20)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for trial in range(8):
        qa, qb = rng.choice(codes, (16, 128)), rng.choice(codes, (16, 128))
        sa = rng.integers(100, 150, 16).astype(np.uint8)
        sb = rng.integers(100, 150, 16).astype(np.uint8)
        A, B = oracle.e4m3_decode(qa), oracle.e4m3_decode(qb)
        d = _unit(fgq_gpu, A, B, sa, sb, np.zeros((16, 16)))
        d0 = fgq_gpu.debug_mfma_16x16x128(dev_u8(qa), dev_u8(qb))
        torch.cuda.synchronize()
        d0 = d0.cpu().numpy().astype(np.float64)
        want = d0 * np.ldexp(1.0, sa.astype(np.int64) - 127)[:, None] * np.ldexp(1.0, sb.astype(np.int64) - 127)[None, :]
        assert np.array_equal(d, want), trial


def _tiny_products(fgq, ks, r):
    """C = 2^r plus products of 1 * 2^-9 at K positions ks: returns the part
    of the products that survives, in units of 2^-9."""
    qa = np.zeros((16, 128), np.uint8)
    qb = np.zeros((16, 128), np.uint8)
    qa[0, ks], qb[0, ks] = 0x38, 0x01
    C = np.zeros((16, 16))
    C[0, 0] = 2.0 ** r
    return (_unit(fgq, oracle.e4m3_decode(qa), oracle.e4m3_decode(qb), np.full(16, 127), np.full(16, 127), C)[0, 0]
            - 2.0 ** r) / 2.0 ** -9


def test_unit_accumulator_window(fgq_gpu):
    """How the scaled operation adds its accumulator operand C: like a
    binary32 addition for one product (kept up to 23 bits below C, a tie to
    even at 24), but each 8-product group sum is dropped once it lies about
    25 bits below C, where a binary32 sum would still keep it."""
    assert _tiny_products(fgq_gpu, [0], 14) == 1          # 2^-9 vs 2^14: exact in binary32
    assert _tiny_products(fgq_gpu, [0], 15) == 0          # half an ulp of 2^15: tie to even
    every_group = list(range(0, 128, 8))                 # 16 group sums of 2^-9
    assert _tiny_products(fgq_gpu, every_group, 15) == 16
    assert _tiny_products(fgq_gpu, every_group, 16) == 0  # binary32 would keep all 16 (ulp 2^-7)
    assert _tiny_products(fgq_gpu, list(range(128)), 18) == 128   # group sums 2^-6
    assert _tiny_products(fgq_gpu, list(range(128)), 19) == 0


# ------------------------------------------------------------------ GEMMs

def _gemm8(fgq, qa, ba, qw, bw, acc, ba_kmajor=False, ldc=None):
    import torch
    M, K = qa.shape
    N = qw.shape[0]
    cg = Guarded(M, N, torch.bfloat16, ld=ldc)
    ba_d = dev_u8(np.ascontiguousarray(ba.T)).t() if ba_kmajor else dev_u8(ba)
    fgq.gemm_fp8_e8m0(dev_u8(qa), ba_d, dev_u8(qw), dev_u8(bw), out=cg.view, accumulate=acc)
    torch.cuda.synchronize()
    cg.check_canaries()
    return host_bf16_f64(cg.view)


def _gemm_f32(fgq, qa, sa, qw, sw, mode):
    import torch
    c = fgq.gemm_fp8_blockscaled(dev_u8(qa), dev_f32(sa), dev_u8(qw), dev_f32(sw), mode=mode)
    torch.cuda.synchronize()
    return host_bf16_f64(c)


def in_core_slack(qa, ba, qw, bw, rows, cols):
    """Extra error of accumulating in the matrix core.  Chunk kb's operation
    truncates C and its 16 group sums about 24 bits below the largest of
    them: at most 17 * 2^-24 of that maximum per chunk, taken here as 2^-19
    (four times the measured worst case).  The maximum is bounded by the sum
    of |products| of the chunks before kb (the running sum) plus those of
    chunk kb."""
    A = oracle.e4m3_decode(qa[rows]).astype(np.float64)
    W = oracle.e4m3_decode(qw[cols]).astype(np.float64)
    sa = oracle.e8m0_decode(ba[rows])
    sw = oracle.e8m0_decode(bw[np.asarray(cols) // 128])
    K = A.shape[1]
    out = np.zeros((A.shape[0], W.shape[0]))
    run = np.zeros_like(out)
    for kb in range(K // 128):
        sl = slice(128 * kb, 128 * kb + 128)
        mag = (np.abs(A[:, sl]) @ np.abs(W[:, sl]).T) * sa[:, kb][:, None] * sw[:, kb][None, :]
        out += 2.0 ** -19 * (run + mag)
        run += mag
    return out


def _check8(c, ref, what, acc, qa, ba, qw, bw, rows=None):
    g = oracle.gemm_gate(c, ref)
    name = "promote" if acc == PROMOTE else "in-core"
    log(f"{what} [e8m0 {name}]: normwise {g['normwise']:.3e}, max elem {g['max_elem_rel']:.3e}")
    assert g["finite"], (what, g)
    assert g["normwise"] <= 2e-3, (what, g)
    rng = np.random.default_rng(0)
    M, N = ref.shape
    rs = np.arange(M) if M <= 64 else np.sort(rng.choice(M, 64, replace=False))
    cs = np.arange(N) if N <= 512 else np.sort(rng.choice(N, 512, replace=False))
    src = np.asarray(rows)[rs] if rows is not None else rs
    slack = fp8_core_slack(qa, oracle.e8m0_decode(ba), qw, oracle.e8m0_decode(bw), src, cs)
    if acc == IN_CORE:
        slack = slack + in_core_slack(qa, ba, qw, bw, src, cs)
    sub_c, sub_r = c[np.ix_(rs, cs)], ref[np.ix_(rs, cs)]
    over = np.abs(sub_c - sub_r) - (1e-2 * np.abs(sub_r) + slack)
    assert np.all(over <= 0), (what, float(over.max()))
    # every output, against the looser bound from the group maxima.  The
    # in-core part (in_core_slack) is at most K/128 * 2^-19 times the sum of
    # |products|, and that sum is at most 2^12 times the group-maxima slack.
    all_rows = np.asarray(rows) if rows is not None else np.arange(M)
    loose = fp8_core_slack_all(qa[all_rows], oracle.e8m0_decode(ba[all_rows]), qw, oracle.e8m0_decode(bw))
    if acc == IN_CORE:
        loose = loose * (1 + (qa.shape[1] // 128) * 2.0 ** -7)
    over = np.abs(c - ref) - (1e-2 * np.abs(ref) + loose)
    assert np.all(over <= 0), (what, "all outputs", float(over.max()))
    return g


def _int_codes(shape, rng):
    ints = rng.integers(-8, 9, size=shape)
    lut = {0: 0}
    for v in range(1, 9):
        e = int(np.floor(np.log2(v)))
        lut[v] = ((e + 7) << 3) | int((v / 2 ** e - 1) * 8)
        lut[-v] = lut[v] | 0x80
    table = np.array([lut[v] for v in range(-8, 9)], dtype=np.uint8)
    return table[ints + 8]


def test_gemm8_promote_integer_codes_exact(fgq_gpu):
    """Small-integer codes and power-of-two scales: every chunk sum and every
    promoted partial sum is exact in binary32, so the result is the oracle's
    rounded to BF16, bit for bit (K = 7168)."""
    rng = np.random.default_rng(21)
    M, N, K = 200, 384, 7168
    qa, qw = _int_codes((M, K), rng), _int_codes((N, K), rng)
    ba = rng.integers(126, 129, (M, K // 128)).astype(np.uint8)
    bw = rng.integers(126, 129, (N // 128, K // 128)).astype(np.uint8)
    c = _gemm8(fgq_gpu, qa, ba, qw, bw, PROMOTE)
    assert np.array_equal(c, oracle.bf16_round_f64(oracle.gemm_e8m0_ref(qa, ba, qw, bw)))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (129, 256, 384), (64, 18432, 7168), (513, 768, 512),
                                   (384, 18432, 7168)])
def test_gemm8_promote_equals_fp8_core(fgq_gpu, M, N, K):
    """Power-of-two scales given as bytes (scaled by the unit) and as binary32
    (promotion FMA): the same bits, on the dense, split-K and large-tile paths."""
    a = normal_bf16((M, K), 1.0, rng_for(22, M))
    w = normal_bf16((N, K), 0.02, rng_for(22, N + 1))
    qa, ba = oracle.quant_act_1x128_e8m0(a)
    qw, bw = oracle.quant_w_128x128_e8m0(w)
    c8 = _gemm8(fgq_gpu, qa, ba, qw, bw, PROMOTE)
    cf = _gemm_f32(fgq_gpu, qa, oracle.e8m0_decode(ba).astype(np.float32), qw,
                   oracle.e8m0_decode(bw).astype(np.float32), 1)
    assert np.array_equal(c8, cf)


@pytest.mark.parametrize("acc", ACCS)
@pytest.mark.parametrize("M,N,K,ldc,kmajor", [(1, 128, 128, None, False), (129, 256, 384, None, True),
                                              (300, 384, 1024, 392, False), (64, 128, 7168, None, True),
                                              (255, 640, 2048, 648, False), (513, 768, 512, None, True)])
def test_gemm8_shapes(fgq_gpu, M, N, K, ldc, kmajor, acc):
    a = normal_bf16((M, K), 1.0, rng_for(23, M))
    w = normal_bf16((N, K), 0.02, rng_for(23, N + 1))
    qa, ba = oracle.quant_act_1x128_e8m0(a)
    qw, bw = oracle.quant_w_128x128_e8m0(w)
    ref = oracle.gemm_e8m0_ref(qa, ba, qw, bw)
    c = _gemm8(fgq_gpu, qa, ba, qw, bw, acc, ba_kmajor=kmajor, ldc=ldc)
    _check8(c, ref, f"gemm e8m0 {M}x{N}x{K}", acc, qa, ba, qw, bw)


@pytest.mark.parametrize("acc", ACCS)
@pytest.mark.parametrize("name,rows", [("tiny", None), ("decode", None), ("prefill", 384)])
def test_gemm8_workloads(fgq_gpu, name, rows, acc):
    """Gate against the oracle; also logs the accuracy study: each path's
    distance to the product of the unquantised BF16 operands."""
    d = make_workload(name, rows=rows)
    qa, ba = oracle.quant_act_1x128_e8m0(d["A"])
    qw, bw = oracle.quant_w_128x128_e8m0(d["W"])
    ref = oracle.gemm_e8m0_ref(qa, ba, qw, bw)
    c = _gemm8(fgq_gpu, qa, ba, qw, bw, acc)
    _check8(c, ref, f"gemm {name}", acc, qa, ba, qw, bw)
    a64 = oracle.f32_from_bf16(d["A"]).astype(np.float64)
    w64 = oracle.f32_from_bf16(d["W"]).astype(np.float64)
    exact = a64 @ w64.T
    nrm = np.linalg.norm(exact)
    qaf, saf = oracle.quant_act_1x128(d["A"])
    qwf, swf = oracle.quant_w_128x128(d["W"])
    cf = _gemm_f32(fgq_gpu, qaf, saf, qwf, swf, 0)
    log(f"  vs unquantised BF16: e8m0 {'promote' if acc == PROMOTE else 'in-core'} "
        f"{np.linalg.norm(c - exact) / nrm:.3e}; binary32 scales, exact mode {np.linalg.norm(cf - exact) / nrm:.3e}; "
        f"quantisation alone: e8m0 {np.linalg.norm(ref - exact) / nrm:.3e}, "
        f"binary32 {np.linalg.norm(oracle.gemm_ref(qaf, saf, qwf, swf) - exact) / nrm:.3e}")


@pytest.mark.parametrize("acc", ACCS)
def test_gemm8_last_round_split(fgq_gpu, acc):
    """2816 rows in 256x256 tiles are one round of 256 tiles and 8 more: the
    last 8 are split 4 ways along K into partial sums in the workspace.  The
    split and the plain launch (no workspace) against the oracle; promote
    also bit for bit against the FP8-core mode fed the same power-of-two
    scales as binary32, which takes the same split."""
    import torch
    M, N, K = 2816, 6144, 2048
    a = normal_bf16((M, K), 1.0, rng_for(42, M))
    w = normal_bf16((N, K), 0.02, rng_for(42, N))
    qa, ba = oracle.quant_act_1x128_e8m0(a)
    qw, bw = oracle.quant_w_128x128_e8m0(w)
    ref = oracle.gemm_e8m0_ref(qa, ba, qw, bw)
    assert fgq_gpu.gemm_workspace_bytes(M, N, K) > 0
    qa_d, ba_d, qw_d, bw_d = dev_u8(qa), dev_u8(ba), dev_u8(qw), dev_u8(bw)
    c_split = fgq_gpu.gemm_fp8_e8m0(qa_d, ba_d, qw_d, bw_d, accumulate=acc)
    c_plain = fgq_gpu.gemm_fp8_e8m0(qa_d, ba_d, qw_d, bw_d, accumulate=acc,
                                    workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    split, plain = host_bf16_f64(c_split), host_bf16_f64(c_plain)
    _check8(split, ref, f"e8m0 last-round split {M}x{N}x{K}", acc, qa, ba, qw, bw)
    _check8(plain, ref, f"e8m0 plain {M}x{N}x{K}", acc, qa, ba, qw, bw)
    if acc == PROMOTE:
        cf = _gemm_f32(fgq_gpu, qa, oracle.e8m0_decode(ba).astype(np.float32), qw,
                       oracle.e8m0_decode(bw).astype(np.float32), 1)
        assert np.array_equal(split, cf)


@pytest.mark.parametrize("acc", ACCS)
def test_gemm8_prefill_full_size_sampled(fgq_gpu, acc):
    """8192 x 18432 x 7168 quantised and multiplied on the GPU as the
    benchmark runs it; 128 sampled rows against the oracle."""
    import torch
    d = make_workload("prefill")
    A, W = d["A"], d["W"]
    qa, ba = fgq_gpu.quant_act_1x128_e8m0(dev_bf16(A))
    qw, bw = fgq_gpu.quant_w_128x128_e8m0(dev_bf16(W))
    c = fgq_gpu.gemm_fp8_e8m0(qa, ba, qw, bw, accumulate=acc)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(A.shape[0], 128, replace=False))
    rows[0], rows[-1] = 0, A.shape[0] - 1
    qao, bao = oracle.quant_act_1x128_e8m0(A[rows])
    qwo, bwo = oracle.quant_w_128x128_e8m0(W)
    ref = oracle.gemm_e8m0_ref(qao, bao, qwo, bwo)
    _check8(host_bf16_f64(c[rows.tolist()]), ref, "prefill full (sampled rows)", acc, qao, bao, qwo, bwo)


def _grouped8(fgq, qa, ba, qw, bw, offsets, acc):
    import torch
    R, N = qa.shape[0], qw.shape[1]
    cg = Guarded(R, N, torch.bfloat16)
    fgq.grouped_gemm_fp8_e8m0(dev_u8(qa), dev_u8(ba), dev_u8(qw), dev_u8(bw),
                              torch.from_numpy(np.asarray(offsets, np.int32)).cuda(), out=cg.view, accumulate=acc)
    torch.cuda.synchronize()
    cg.check_canaries()
    return host_bf16_f64(cg.view)


@pytest.mark.parametrize("acc", ACCS)
@pytest.mark.parametrize("counts", [[0, 200, 0, 57], [1, 1, 1, 130], [129, 127, 128, 256], [0, 700, 1, 0, 256, 255]])
def test_grouped8_ragged(fgq_gpu, counts, acc):
    E, N, K = len(counts), 256, 512
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    a = normal_bf16((R, K), 1.0, rng_for(24, R))
    w = normal_bf16((E, N, K), 0.02, rng_for(24, 7))
    qa, ba = oracle.quant_act_1x128_e8m0(a)
    qw, bw = oracle.quant_w_128x128_e8m0(w)
    ref = oracle.grouped_gemm_e8m0_ref(qa, ba, qw, bw, off)
    c = _grouped8(fgq_gpu, qa, ba, qw, bw, off, acc)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            _check8(c[r0:r1], ref[r0:r1], f"grouped {counts} expert {e}", acc, qa[r0:r1], ba[r0:r1], qw[e], bw[e])


@pytest.mark.parametrize("acc", ACCS)
def test_grouped8_single_expert_equals_dense(fgq_gpu, acc):
    M, N, K = 333, 384, 1024
    a = normal_bf16((M, K), 1.0, rng_for(25, 1))
    w = normal_bf16((1, N, K), 0.02, rng_for(25, 2))
    qa, ba = oracle.quant_act_1x128_e8m0(a)
    qw, bw = oracle.quant_w_128x128_e8m0(w)
    assert np.array_equal(_grouped8(fgq_gpu, qa, ba, qw, bw, [0, M], acc), _gemm8(fgq_gpu, qa, ba, qw[0], bw[0], acc))


@pytest.mark.parametrize("acc", ACCS)
def test_grouped8_moe_decode_full_size(fgq_gpu, acc):
    """Decode-shaped MoE (256 tokens, top-8 of 32 experts): routing on the
    GPU, activations and expert weights quantised with E8M0 scales on the
    GPU, the grouped GEMM in the decode configuration; every row of three
    experts against the oracle."""
    import torch
    d = make_workload("moe_decode")
    X, W, ids, E = d["X"], d["W"], d["ids"], d["E"]
    qa, ba, off, src, _ = fgq_gpu.quant_dispatch_1x128_e8m0(dev_bf16(X), torch.from_numpy(ids).cuda(), E)
    qw, bw = fgq_gpu.quant_w_128x128_e8m0(dev_bf16(W))
    c = fgq_gpu.grouped_gemm_fp8_e8m0(qa, ba, qw, bw, off, accumulate=acc)
    torch.cuda.synchronize()
    offo, srco, _ = oracle.dispatch_ref(ids, E)
    assert np.array_equal(off.cpu().numpy(), offo)
    counts = np.diff(offo)
    nz = np.nonzero(counts)[0]
    for e in sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), int(nz[-1])}):
        r0, r1 = int(offo[e]), int(offo[e + 1])
        toks = srco[r0:r1].astype(np.int64) // d["topk"]
        qao, bao = oracle.quant_act_1x128_e8m0(X[toks])
        qwo, bwo = oracle.quant_w_128x128_e8m0(W[e])
        ref = oracle.gemm_e8m0_ref(qao, bao, qwo, bwo)
        _check8(host_bf16_f64(c[r0:r1]), ref, f"moe_decode expert {e} ({r1 - r0} rows)", acc, qao, bao, qwo, bwo)
