"""GPU parity of the quantisation kernels against the CPU oracle.

Codes and scales must be byte-identical.  Covered: the device E4M3 encoder
over every float32 in [2**-11, 448] and both signs; all five workloads'
quantisation inputs (whole tensors at reduced row counts, sampled rows and
blocks at the full sizes the benchmark uses); edge cases (all-zero and
negative-zero tiles, BF16 subnormals, exact E4M3 tiles, ragged row counts,
strided inputs and transposed scale layouts, empty inputs); run-to-run
determinism; and guard bands around every output."""
import numpy as np
import pytest

import oracle
from synth import bf16_bits_from_f32, make_workload, normal_bf16, rng_for
from tests.gpu_util import Guarded, dev_bf16, log

pytestmark = pytest.mark.gpu


def _q_and_s(fgq, x_bits, M, K, ldx=None, ldq=None, scale_t=False):
    """Run the device 1x128 quantiser with guarded outputs; return host copies."""
    import torch
    ldx = K if ldx is None else ldx
    xp = np.zeros((M, ldx), np.uint16)
    xp[:, :K] = x_bits
    x = dev_bf16(xp)[:, :K]
    qg = Guarded(M, K, torch.uint8, ld=ldq)
    if scale_t:
        sg = Guarded(K // 128, M, torch.float32)
        s_view = sg.view.t()
    else:
        sg = Guarded(M, K // 128, torch.float32)
        s_view = sg.view
    fgq.quant_act_1x128(x, q=qg.view, s=s_view)
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    return qg.view.cpu().numpy(), s_view.cpu().numpy()


def _assert_same(q, s, qo, so, what):
    assert q.shape == qo.shape and s.shape == so.shape, what
    bad = np.nonzero(q != qo)
    assert bad[0].size == 0, f"{what}: {bad[0].size} code mismatches, first at {bad[0][0]},{bad[1][0]}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{what}: scale bits differ"


# ------------------------------------------------------------------ encoder

def test_device_e4m3_encoder_exhaustive(fgq_gpu):
    """Every float32 in [2**-11, 448] (and its negative) through the device
    clamp + convert, against the oracle encoder; plus values above 448
    (clamped to 0x7E) and below 2**-11 (zero)."""
    import torch
    lo = int(np.float32(2.0 ** -11).view(np.uint32))
    hi = int(np.float32(448.0).view(np.uint32))
    step = 1 << 24
    for sign in (0, 1 << 31):
        for start in range(lo, hi + 1, step):
            n = min(hi + 1, start + step) - start
            dev = fgq_gpu.debug_encode_e4m3(start | sign, n).cpu().numpy()
            y = (np.arange(start, start + n, dtype=np.uint32) | np.uint32(sign)).view(np.float32)
            ref = oracle.e4m3_encode(y)
            assert np.array_equal(dev, ref), hex(start | sign)
        log("encoder sweep done for sign", sign)
    for sign in (0, 1 << 31):
        # above 448 up to FLT_MAX: clamped
        for start in (hi + 1, int(np.float32(3.0e38).view(np.uint32)), int(np.float32(1000.0).view(np.uint32))):
            dev = fgq_gpu.debug_encode_e4m3(start | sign, 1 << 20).cpu().numpy()
            assert np.all(dev == (0xFE if sign else 0x7E))
        # tiny values, including zero and float32 subnormals
        dev = fgq_gpu.debug_encode_e4m3(0 | sign, 1 << 22).cpu().numpy()
        assert np.all(dev == (0x80 if sign else 0x00))
        dev = fgq_gpu.debug_encode_e4m3((lo - (1 << 22)) | sign, 1 << 22).cpu().numpy()
        assert np.all(dev == (0x80 if sign else 0x00))
    torch.cuda.synchronize()


# ------------------------------------------------------------------ activations

@pytest.mark.parametrize("name,rows", [("tiny", None), ("decode", None), ("prefill", 700),
                                       ("grouped_up", 600), ("fused_down", 517)])
def test_quant_act_workloads_whole(fgq_gpu, name, rows):
    d = make_workload(name, rows=rows, parts={"A"})
    A = d["A"]
    M, K = A.shape
    q, s = _q_and_s(fgq_gpu, A, M, K)
    qo, so = oracle.quant_act_1x128(A)
    _assert_same(q, s, qo, so, f"{name} act {M}x{K}")
    log(f"act {name} {M}x{K} bit-exact")


def test_quant_act_full_size_sampled_rows(fgq_gpu):
    """Full prefill and grouped-up activations in the benchmark's launch
    configuration; 2048 sampled rows checked against the oracle."""
    import torch
    for name in ("prefill", "grouped_up"):
        d = make_workload(name, parts={"A"})
        A = d["A"]
        M, K = A.shape
        q, s = fgq_gpu.quant_act_1x128(dev_bf16(A))
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(1).choice(M, 2048, replace=False))
        rows[0], rows[-1] = 0, M - 1
        qo, so = oracle.quant_act_1x128(A[rows])
        _assert_same(q[rows.tolist()].cpu().numpy(), s[rows.tolist()].cpu().numpy(), qo, so, name)
        log(f"act {name} full {M}x{K}: sampled rows bit-exact")
        del q, s


def test_quant_act_edge_cases(fgq_gpu):
    rng = np.random.default_rng(3)
    K = 640
    x = rng.standard_normal((37, K)).astype(np.float32)
    x[0, :128] = 0.0                       # zero tile
    x[1, :128] = -0.0                      # negative-zero tile
    x[2, 128:256] = rng.standard_normal(128) * 1e-39   # BF16 subnormals
    x[3, :] = 448.0 * 2.0 ** -7            # exact
    codes = rng.integers(0, 0x7E, 128)
    x[4, 256:384] = oracle.e4m3_decode(codes.astype(np.uint8)) * 2.0 ** 5
    x[4, 300] = 448 * 2.0 ** 5
    x[5, :] *= 1e4
    x[6, 512:] = -x[6, 512:] * 1e-20
    xb = bf16_bits_from_f32(x)
    qo, so = oracle.quant_act_1x128(xb)
    for kw in ({}, {"ldx": 768}, {"ldq": 656}, {"scale_t": True}, {"ldx": 1024, "ldq": 1024, "scale_t": True}):
        q, s = _q_and_s(fgq_gpu, xb, 37, K, **kw)
        _assert_same(q, s, qo, so, f"edge {kw}")
    for M in (1, 2, 15, 16, 17, 33, 37):
        q, s = _q_and_s(fgq_gpu, xb[:M], M, K)
        _assert_same(q, s, qo[:M], so[:M], f"M={M}")


def test_quant_act_empty(fgq_gpu):
    import torch
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = fgq_gpu.quant_act_1x128(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_quant_act_deterministic(fgq_gpu):
    import torch
    A = make_workload("decode", parts={"A"})["A"]
    x = dev_bf16(A)
    q0, s0 = fgq_gpu.quant_act_1x128(x)
    for _ in range(5):
        q1, s1 = fgq_gpu.quant_act_1x128(x)
        assert torch.equal(q0, q1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))


# ------------------------------------------------------------------ weights

def _wq(fgq, w_bits, ldq=None):
    import torch
    B, N, K = w_bits.shape
    qg = Guarded(B * N, K, torch.uint8, ld=ldq)
    sg = Guarded(B * (N // 128), K // 128, torch.float32)
    q3 = qg.view.reshape(B, N, K) if ldq is None else qg.view.as_strided((B, N, K), (N * ldq, ldq, 1))
    fgq.quant_w_128x128(dev_bf16(w_bits), q=q3, s=sg.view.reshape(B, N // 128, K // 128))
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    return q3.cpu().numpy(), sg.view.reshape(B, N // 128, K // 128).cpu().numpy()


def test_quant_w_tiny_and_batched_edge(fgq_gpu):
    W = make_workload("tiny", parts={"W"})["W"]
    q, s = _wq(fgq_gpu, W[None])
    qo, so = oracle.quant_w_128x128(W)
    _assert_same(q[0], s[0], qo, so, "tiny W")
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((3, 256, 384)) * 0.02).astype(np.float32)
    w[1, :128, :128] = 0.0
    w[2, 128:, 256:] *= 1e6
    wb = bf16_bits_from_f32(w)
    qo, so = oracle.quant_w_128x128(wb)
    for ldq in (None, 400):
        q, s = _wq(fgq_gpu, wb, ldq=ldq)
        _assert_same(q.reshape(-1, 384), s.reshape(-1, 3), qo.reshape(-1, 384), so.reshape(-1, 3), f"batched ldq={ldq}")


def test_quant_w_full_size_sampled_blocks(fgq_gpu):
    """Dense 18432x7168 and grouped 32x4096x7168 weights, full launch; sampled
    128-row block stripes checked against the oracle."""
    import torch
    rng = np.random.default_rng(5)
    W = make_workload("prefill", parts={"W"})["W"]
    q, s = fgq_gpu.quant_w_128x128(dev_bf16(W))
    torch.cuda.synchronize()
    for nb in sorted(rng.choice(W.shape[0] // 128, 6, replace=False).tolist() + [0, W.shape[0] // 128 - 1]):
        qo, so = oracle.quant_w_128x128(W[nb * 128:(nb + 1) * 128])
        _assert_same(q[nb * 128:(nb + 1) * 128].cpu().numpy(), s[nb:nb + 1].cpu().numpy(), qo, so, f"dense nb={nb}")
    log("dense W full: sampled stripes bit-exact")
    del W, q, s
    d = make_workload("grouped_up", parts={"W"})
    W = d["W"]
    q, s = fgq_gpu.quant_w_128x128(dev_bf16(W))
    torch.cuda.synchronize()
    for e in (0, 13, 31):
        for nb in (0, 17, 31):
            qo, so = oracle.quant_w_128x128(W[e, nb * 128:(nb + 1) * 128])
            _assert_same(q[e, nb * 128:(nb + 1) * 128].cpu().numpy(), s[e, nb:nb + 1].cpu().numpy(), qo, so,
                         f"grouped e={e} nb={nb}")
    log("grouped W full: sampled stripes bit-exact")


def test_quant_w_down_proj_whole_expert(fgq_gpu):
    W = make_workload("fused_down", parts={"W"})["W"]
    import torch
    q, s = fgq_gpu.quant_w_128x128(dev_bf16(W))
    torch.cuda.synchronize()
    for e in (0, 31):
        qo, so = oracle.quant_w_128x128(W[e])
        _assert_same(q[e].cpu().numpy(), s[e].cpu().numpy(), qo, so, f"down e={e}")


# ------------------------------------------------------------------ fused RMSNorm

def _fused(fgq, xb, gb, eps, ldq=None, scale_t=False):
    import torch
    M, K = xb.shape
    qg = Guarded(M, K, torch.uint8, ld=ldq)
    if scale_t:
        sg = Guarded(K // 128, M, torch.float32)
        sv = sg.view.t()
    else:
        sg = Guarded(M, K // 128, torch.float32)
        sv = sg.view
    fgq.fused_rmsnorm_quant(dev_bf16(xb), dev_bf16(gb), eps, q=qg.view, s=sv)
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    return qg.view.cpu().numpy(), sv.cpu().numpy()


def test_fused_workload_rows(fgq_gpu):
    d = make_workload("fused_down", rows=1027, parts={"X", "gamma"})
    q, s = _fused(fgq_gpu, d["X"], d["gamma"], d["eps"])
    qo, so = oracle.fused_rmsnorm_quant(d["X"], d["gamma"], d["eps"])
    _assert_same(q, s, qo, so, "fused 1027x7168")


@pytest.mark.parametrize("scale_t", [False, True])
def test_fused_many_rows_ragged(fgq_gpu, scale_t):
    # 4103 rows at K 7168, every row against the oracle: 1026 workgroups of
    # four rows, the last holding three (its fourth wave loads nothing and
    # stores nothing), with row-major and K-block-major scales
    d = make_workload("fused_down", rows=4103, parts={"X", "gamma"})
    q, s = _fused(fgq_gpu, d["X"], d["gamma"], d["eps"], scale_t=scale_t)
    qo, so = oracle.fused_rmsnorm_quant(d["X"], d["gamma"], d["eps"])
    _assert_same(q, s, qo, so, f"fused 4103x7168 scale_t={scale_t}")


def test_fused_full_size_sampled_rows(fgq_gpu):
    import torch
    d = make_workload("fused_down", parts={"X", "gamma"})
    X = d["X"]
    q, s = fgq_gpu.fused_rmsnorm_quant(dev_bf16(X), dev_bf16(d["gamma"]), d["eps"])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(X.shape[0], 2048, replace=False))
    rows[0], rows[-1] = 0, X.shape[0] - 1
    qo, so = oracle.fused_rmsnorm_quant(X[rows], d["gamma"], d["eps"])
    _assert_same(q[rows.tolist()].cpu().numpy(), s[rows.tolist()].cpu().numpy(), qo, so, "fused full")


@pytest.mark.parametrize("K", [128, 640, 2048, 4096, 8192, 8320, 16384])
def test_fused_shapes(fgq_gpu, K):
    rng = np.random.default_rng(K)
    M = 9
    x = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    x[1] = 1.0                   # constant row
    x[2] *= 1e-5                 # eps matters
    x[3, :5] *= 300
    xb = bf16_bits_from_f32(x)
    gb = bf16_bits_from_f32(rng.uniform(0.5, 1.5, K).astype(np.float32))
    qo, so = oracle.fused_rmsnorm_quant(xb, gb, 1e-6)
    q, s = _fused(fgq_gpu, xb, gb, 1e-6, ldq=K + 16, scale_t=(K == 640))
    _assert_same(q, s, qo, so, f"fused K={K}")


@pytest.mark.parametrize("K", [1024, 7168])
def test_fused_r64_crafted_rows(fgq_gpu, K):
    # the crafted rows that pin the oracle's summation order (their first 1024
    # values; zeros after): where the order changes rstd, it changes the codes
    # and scales, which must still match the oracle bit for bit
    from tests.test_oracle_quant import _R64_CASES
    rows = []
    for make, _, _ in _R64_CASES:
        x = np.zeros(K, np.float32)
        x[:1024] = make()
        rows.append(x)
    x = np.stack(rows)
    xb = bf16_bits_from_f32(x)
    gb = bf16_bits_from_f32(np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32))
    qo, so = oracle.fused_rmsnorm_quant(xb, gb, 1e-6)
    q, s = _fused(fgq_gpu, xb, gb, 1e-6)
    _assert_same(q, s, qo, so, f"fused crafted rows K={K}")
