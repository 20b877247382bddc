"""The C ABI without a GPU: the library loads, exports every function that
include/fgq.h declares, and rejects bad arguments on the host before any HIP
call (so these run on a machine with no GPU).  Empty problems return FGQ_OK
and launch nothing."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgq.h")

OK, NULL, SHAPE, ALIGN, STRIDE, UNSUP = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    import fine_grained_fp8_quant_amd as fgq
    if not os.path.exists(fgq.library_path()):
        from fine_grained_fp8_quant_amd.build import build
        build()
    return fgq.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("fgq_quant_act_1x128", "fgq_quant_w_128x128", "fgq_fused_rmsnorm_quant",
              "fgq_gemm_fp8_blockscaled", "fgq_grouped_gemm_fp8_blockscaled", "fgq_quant_dispatch_1x128",
              "fgq_quant_act_1x128_e8m0", "fgq_quant_w_128x128_e8m0", "fgq_fused_rmsnorm_quant_e8m0",
              "fgq_gemm_fp8_e8m0", "fgq_grouped_gemm_fp8_e8m0", "fgq_quant_dispatch_1x128_e8m0",
              "fgq_gemm_bf16a_fp8_blockscaled"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.fgq_abi_version() == 6
    for code in range(8):
        assert lib.fgq_status_string(code)
    assert lib.fgq_status_string(99) == b"unknown status"
    assert lib.fgq_last_hip_error() == 0


P = 1 << 20          # a fake, 16-byte aligned "device" address: never dereferenced on error paths
Q = P + 4096
S = P + 8192


def act(lib, x=P, ldx=256, M=4, K=256, q=Q, ldq=256, s=S, s_sm=2, s_skb=1):
    return lib.fgq_quant_act_1x128(x, ldx, M, K, q, ldq, s, s_sm, s_skb, None)


def test_quant_act_validation(lib):
    assert act(lib, M=-1) == SHAPE
    assert act(lib, K=100) == UNSUP
    assert act(lib, M=0) == OK                      # empty: nothing launched
    assert act(lib, x=0) == NULL
    assert act(lib, q=0) == NULL
    assert act(lib, s=0) == NULL
    assert act(lib, x=P + 2) == ALIGN
    assert act(lib, q=Q + 8) == ALIGN
    assert act(lib, s=S + 2) == ALIGN
    assert act(lib, ldx=128) == STRIDE
    assert act(lib, ldx=260) == STRIDE
    assert act(lib, ldq=264) == STRIDE
    assert act(lib, s_sm=-1) == STRIDE


def wq(lib, w=P, ldw=256, w_bs=256 * 128, B=2, N=128, K=256, q=Q, ldq=256, q_bs=256 * 128, s=S,
       s_snb=2, s_skb=1, s_bs=2):
    return lib.fgq_quant_w_128x128(w, ldw, w_bs, B, N, K, q, ldq, q_bs, s, s_snb, s_skb, s_bs, None)


def test_quant_w_validation(lib):
    assert wq(lib, B=-1) == SHAPE
    assert wq(lib, N=100) == UNSUP
    assert wq(lib, K=64) == UNSUP
    assert wq(lib, B=0) == OK
    assert wq(lib, w=0) == NULL
    assert wq(lib, w=P + 8) == ALIGN
    assert wq(lib, w_bs=100) == STRIDE               # overlapping experts
    assert wq(lib, q_bs=256 * 128 - 16) == STRIDE
    assert wq(lib, ldq=256 + 8) == STRIDE


def test_fused_validation(lib):
    f = lib.fgq_fused_rmsnorm_quant
    assert f(P, 256, 0, ctypes.c_float(1e-6), 4, 256, Q, 256, S, 2, 1, None) == NULL
    assert f(P, 256, Q + 4, ctypes.c_float(1e-6), 4, 256, Q, 256, S, 2, 1, None) == ALIGN
    assert f(P, 32768, Q, ctypes.c_float(1e-6), 4, 32768, Q, 32768, S, 256, 1, None) == UNSUP
    assert f(P, 256, Q, ctypes.c_float(1e-6), 0, 256, Q, 256, S, 2, 1, None) == OK


def gemm(lib, qa=P, lda=256, sa=S, sa_sm=2, sa_skb=1, qw=Q, ldw=256, sw=S, sw_snb=2, sw_skb=1, c=Q,
         ldc=256, M=4, N=256, K=256, mode=0, ws=0, ws_bytes=0):
    return lib.fgq_gemm_fp8_blockscaled(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc,
                                        M, N, K, mode, ws, ws_bytes, None)


def test_gemm_validation(lib):
    assert gemm(lib, M=-1) == SHAPE
    assert gemm(lib, mode=2) == UNSUP
    assert gemm(lib, mode=-1) == UNSUP
    assert gemm(lib, N=100) == UNSUP
    assert gemm(lib, K=0) == UNSUP
    assert gemm(lib, K=200) == UNSUP
    assert gemm(lib, M=0) == OK
    assert gemm(lib, N=0) == OK
    assert gemm(lib, qa=0) == NULL
    assert gemm(lib, sw=0) == NULL
    assert gemm(lib, c=Q + 2) == ALIGN
    assert gemm(lib, sa=S + 1) == ALIGN
    assert gemm(lib, lda=128) == STRIDE
    assert gemm(lib, ldw=264) == STRIDE
    assert gemm(lib, ldc=128) == STRIDE
    assert gemm(lib, sa_skb=-1) == STRIDE
    # operand rows are addressed by 32-bit offsets inside a tile: strides
    # above 2^24 bytes would wrap them
    assert gemm(lib, lda=(1 << 24) + 16) == UNSUP
    assert gemm(lib, ldw=(1 << 24) + 16) == UNSUP
    assert gemm(lib, lda=1 << 40) == UNSUP
    assert lib.fgq_gemm_fp8_e8m0(P, 256, S, 2, 1, Q, (1 << 24) + 16, S, 2, 1, Q, 256, 4, 256, 256, 0, 0, 0,
                                 None) == UNSUP
    assert lib.fgq_gemm_workspace_bytes(0, 256, 256) == 0
    # small M (memory-bound) shapes split K and need an FP32 workspace
    need = lib.fgq_gemm_workspace_bytes(64, 18432, 7168)
    assert need > 0 and need % (64 * 18432 * 4) == 0
    # large M: partial sums for the last round's tiles, split along K.  8192 rows in
    # 192x256 tiles (exact mode) are 3096 tiles: 12 rounds of 256 and 24 tiles,
    # split 10 ways (the FP8 tiles, 2304 of them, fill 9 rounds exactly)
    assert lib.fgq_gemm_workspace_bytes(8192, 18432, 7168) == 24 * 10 * 192 * 256 * 4
    # a last round more than half full is not split
    assert lib.fgq_gemm_workspace_bytes(8064, 18432, 7168) == 0
    # 2112 rows are 264 exact-mode tiles (one round and 8, split 5 ways at K 2560) and
    # 216 FP8 tiles; with K at most 2048 the exact mode takes 128x128 tiles, unsplit
    assert lib.fgq_gemm_workspace_bytes(2112, 6144, 2560) == 8 * 5 * 192 * 256 * 4
    assert lib.fgq_gemm_workspace_bytes(2112, 6144, 2048) == 0
    # the larger of the two modes' splits: 2816 rows are 360 exact-mode tiles (104 in
    # the last round, 2 parts) and 264 FP8 tiles (8 in the last round, 5 parts at K 2560)
    assert lib.fgq_gemm_workspace_bytes(2816, 6144, 2560) == 104 * 2 * 192 * 256 * 4
    # parts are capped at 16 (and at a quarter of the K chunks)
    assert lib.fgq_gemm_workspace_bytes(2112, 6144, 8192) == 8 * 16 * 192 * 256 * 4
    assert lib.fgq_gemm_workspace_bytes(2112, 6144, 3072) == 8 * 6 * 192 * 256 * 4
    # fewer tiles than compute units: one round, nothing to split
    assert lib.fgq_gemm_workspace_bytes(1024, 6144, 7168) == 0
    assert gemm(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168) == NULL     # no workspace
    assert gemm(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168, ws=P, ws_bytes=need - 1) == SHAPE
    assert gemm(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168, ws=P + 16, ws_bytes=need) == ALIGN


def grouped(lib, E=4, R=100, offsets=S, w_es=256 * 256, N=256, K=256, qa=P, ldc=256, mode=0, lda=256, ldw=256):
    return lib.fgq_grouped_gemm_fp8_blockscaled(qa, lda, S, 2, 1, Q, ldw, w_es, S, 2, 1, 4, offsets, E, R,
                                                Q, ldc, N, K, mode, None)


def test_grouped_validation(lib):
    assert grouped(lib, E=-1) == SHAPE
    assert grouped(lib, mode=7) == UNSUP
    assert grouped(lib, R=-1) == SHAPE
    assert grouped(lib, E=70000) == UNSUP
    assert grouped(lib, K=100) == UNSUP
    assert grouped(lib, E=0) == OK
    assert grouped(lib, R=0) == OK
    assert grouped(lib, offsets=0) == NULL
    assert grouped(lib, qa=0) == NULL
    assert grouped(lib, offsets=S + 2) == ALIGN
    assert grouped(lib, w_es=100 * 16) == STRIDE
    assert grouped(lib, ldc=128) == STRIDE
    assert grouped(lib, lda=(1 << 24) + 16) == UNSUP
    assert grouped(lib, ldw=(1 << 24) + 16, w_es=256 * ((1 << 24) + 16)) == UNSUP


def test_debug_validation(lib):
    assert lib.fgq_debug_encode_e4m3(0, -1, P, None) == SHAPE
    assert lib.fgq_debug_encode_e4m3(0, 0, 0, None) == OK
    assert lib.fgq_debug_encode_e4m3(0, 16, 0, None) == NULL
    assert lib.fgq_debug_copy(P, Q, 15, None) == ALIGN
    assert lib.fgq_debug_copy(P + 1, Q, 16, None) == ALIGN


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    import fine_grained_fp8_quant_amd as fgq
    monkeypatch.setenv("FGQ_LIB", str(tmp_path / "missing.so"))
    saved = fgq.lib
    try:
        fgq.lib = None
        with pytest.raises(fgq.FgqError):
            fgq.load_library()
    finally:
        fgq.lib = saved
    importlib.invalidate_caches()


def dispatch(lib, x=P, ldx=256, T=4, K=256, ids=S, topk=2, E=3, q=Q, ldq=256, s=S + 1024, s_sm=1, s_skb=8,
             off=S + 2048, src=S + 3072, dest=S + 4096, ws=P + 65536, ws_bytes=1 << 20):
    return lib.fgq_quant_dispatch_1x128(x, ldx, T, K, ids, topk, E, q, ldq, s, s_sm, s_skb, off, src, dest,
                                        ws, ws_bytes, None)


def test_dispatch_validation(lib):
    assert dispatch(lib, T=-1) == SHAPE
    assert dispatch(lib, topk=0) == SHAPE
    assert dispatch(lib, E=0) == SHAPE
    assert dispatch(lib, E=4097) == UNSUP
    assert dispatch(lib, K=200) == UNSUP
    assert dispatch(lib, K=128 * 65536) == UNSUP     # K / 128 beyond the scale gather's grid
    assert dispatch(lib, T=1 << 20, topk=1 << 12) == UNSUP      # 2^32 pairs
    assert dispatch(lib, off=0) == NULL
    assert dispatch(lib, off=S + 2050) == ALIGN
    assert dispatch(lib, ids=0) == NULL
    assert dispatch(lib, src=0) == NULL
    assert dispatch(lib, dest=S + 4098) == ALIGN
    assert dispatch(lib, x=P + 8) == ALIGN
    assert dispatch(lib, q=0) == NULL
    assert dispatch(lib, ldq=128) == STRIDE
    assert dispatch(lib, s_skb=-1) == STRIDE
    need = lib.fgq_quant_dispatch_workspace_bytes(4, 2, 3, 256)
    assert need > 0
    assert dispatch(lib, ws=0) == NULL
    assert dispatch(lib, ws_bytes=need - 1) == SHAPE
    assert dispatch(lib, ws=P + 65536 + 16) == ALIGN
    assert lib.fgq_quant_dispatch_workspace_bytes(0, 8, 32, 7168) == 0
    # routing counts of 256-pair blocks (rounded to 256 bytes), then 4 bytes per token tile
    assert lib.fgq_quant_dispatch_workspace_bytes(4096, 8, 32, 0) == 2 * (4096 * 8 // 256) * 32 * 4
    assert lib.fgq_quant_dispatch_workspace_bytes(4096, 8, 32, 7168) == 2 * (4096 * 8 // 256) * 32 * 4 + 4096 * 56 * 4
    assert lib.fgq_quant_dispatch_workspace_bytes(5, 1, 3, 128) == 256 + 5 * 4
    assert lib.fgq_quant_dispatch_workspace_bytes(-1, 8, 32, 7168) == 0
    assert lib.fgq_quant_dispatch_workspace_bytes(4096, 8, 32, 200) == 0


# ---- power-of-two (E8M0) scale variants: byte scales, no alignment rule on them

def test_quant_e8m0_validation(lib):
    a8 = lib.fgq_quant_act_1x128_e8m0
    assert a8(P, 256, -1, 256, Q, 256, S, 2, 1, None) == SHAPE
    assert a8(P, 256, 4, 100, Q, 256, S, 2, 1, None) == UNSUP
    assert a8(P, 256, 0, 256, Q, 256, S, 2, 1, None) == OK
    assert a8(P, 256, 4, 256, Q, 256, 0, 2, 1, None) == NULL
    assert a8(P, 256, 4, 256, Q + 8, 256, S + 1, 2, 1, None) == ALIGN    # the codes, not the bytes
    assert a8(P, 256, 4, 256, Q, 256, S + 1, -1, 1, None) == STRIDE     # byte scales pass the alignment check
    assert act(lib, s=S + 1, s_sm=-1) == ALIGN                           # binary32 scales do not
    w8 = lib.fgq_quant_w_128x128_e8m0
    assert w8(P, 256, 256 * 128, 2, 100, 256, Q, 256, 256 * 128, S, 2, 1, 2, None) == UNSUP
    assert w8(P, 256, 256 * 128, 0, 128, 256, Q, 256, 256 * 128, S, 2, 1, 2, None) == OK
    assert w8(P, 256, 256 * 128, 2, 128, 256, Q, 256, 256 * 128, S + 3, -2, 1, 2, None) == STRIDE
    f8 = lib.fgq_fused_rmsnorm_quant_e8m0
    assert f8(P, 256, 0, ctypes.c_float(1e-6), 4, 256, Q, 256, S, 2, 1, None) == NULL
    assert f8(P, 32768, Q, ctypes.c_float(1e-6), 4, 32768, Q, 32768, S + 1, 256, 1, None) == UNSUP


def gemm8(lib, qa=P, lda=256, sa=S, sa_sm=2, sa_skb=1, qw=Q, ldw=256, sw=S, sw_snb=2, sw_skb=1, c=Q,
          ldc=256, M=4, N=256, K=256, acc=0, ws=0, ws_bytes=0):
    return lib.fgq_gemm_fp8_e8m0(qa, lda, sa, sa_sm, sa_skb, qw, ldw, sw, sw_snb, sw_skb, c, ldc,
                                 M, N, K, acc, ws, ws_bytes, None)


def test_gemm_e8m0_validation(lib):
    assert gemm8(lib, M=-1) == SHAPE
    assert gemm8(lib, acc=2) == UNSUP
    assert gemm8(lib, acc=-1) == UNSUP
    assert gemm8(lib, K=200) == UNSUP
    assert gemm8(lib, M=0) == OK
    assert gemm8(lib, sa=0) == NULL
    assert gemm8(lib, sw=0) == NULL
    assert gemm8(lib, c=Q + 2) == ALIGN
    assert gemm8(lib, sa=S + 1, sw=S + 3, lda=128) == STRIDE       # unaligned byte scales are fine
    assert gemm(lib, sa=S + 1, lda=128) == ALIGN                    # unaligned binary32 scales are not
    need = lib.fgq_gemm_workspace_bytes(64, 18432, 7168)
    assert gemm8(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168) == NULL      # no workspace
    assert gemm8(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168, ws=P, ws_bytes=need - 1) == SHAPE
    g8 = lib.fgq_grouped_gemm_fp8_e8m0
    assert g8(P, 256, S, 2, 1, Q, 256, 256 * 256, S, 2, 1, 4, S, 4, 100, Q, 256, 256, 256, 5, None) == UNSUP
    assert g8(P, 256, S, 2, 1, Q, 256, 256 * 256, S, 2, 1, 4, S, 0, 100, Q, 256, 256, 256, 1, None) == OK
    assert g8(P, 256, S, 2, 1, Q, 256, 256 * 256, S, 2, 1, 4, 0, 4, 100, Q, 256, 256, 256, 1, None) == NULL
    assert g8(P, 256, S + 1, 2, 1, Q, 256, 100 * 16, S + 1, 2, 1, 4, S, 4, 100, Q, 256, 256, 256, 0, None) == STRIDE
    assert lib.fgq_debug_mfma_e8m0_16x16x128(P, Q, 0, S, S, S, None) == NULL
    assert lib.fgq_debug_mfma_e8m0_16x16x128(P + 8, Q, S, S, S, S, None) == ALIGN


def test_dispatch_e8m0_validation(lib):
    d8 = lib.fgq_quant_dispatch_1x128_e8m0
    args = dict(x=P, ldx=256, T=4, K=256, ids=S, topk=2, E=3, q=Q, ldq=256, s=S + 1025, s_sm=1, s_skb=8,
                off=S + 2048, src=S + 3072, dest=S + 4096, ws=P + 65536, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(args, **kw)
        return d8(a["x"], a["ldx"], a["T"], a["K"], a["ids"], a["topk"], a["E"], a["q"], a["ldq"], a["s"], a["s_sm"],
                  a["s_skb"], a["off"], a["src"], a["dest"], a["ws"], a["ws_bytes"], None)
    assert call(T=-1) == SHAPE
    assert call(E=4097) == UNSUP
    assert call(off=0) == NULL
    assert call(ldq=128) == STRIDE          # an odd scale address passes the alignment check
    assert dispatch(lib, s=S + 1025, ldq=128) == ALIGN


def gemm16(lib, a=P, lda=256, qw=Q, ldw=256, sw=S, sw_snb=2, sw_skb=1, c=Q, ldc=256, M=4, N=256, K=256, mode=0,
           qa=0, ldq=256, sa=0, sa_sm=2, sa_skb=1, ws=0, ws_bytes=0):
    return lib.fgq_gemm_bf16a_fp8_blockscaled(a, lda, qw, ldw, sw, sw_snb, sw_skb, c, ldc, M, N, K, mode, qa, ldq,
                                              sa, sa_sm, sa_skb, ws, ws_bytes, None)


def test_gemm_bf16a_validation(lib):
    assert gemm16(lib, M=-1) == SHAPE
    assert gemm16(lib, mode=2) == UNSUP
    assert gemm16(lib, K=200) == UNSUP
    assert gemm16(lib, M=0) == OK
    assert gemm16(lib, a=0) == NULL
    assert gemm16(lib, qa=Q) == NULL                 # codes without scales
    assert gemm16(lib, sa=S) == NULL                 # scales without codes
    assert gemm16(lib, a=P + 8) == ALIGN
    assert gemm16(lib, qa=Q + 8, sa=S) == ALIGN
    assert gemm16(lib, lda=128) == STRIDE
    assert gemm16(lib, lda=(1 << 23) + 8) == UNSUP
    assert gemm16(lib, ldw=(1 << 24) + 16) == UNSUP
    assert gemm16(lib, lda=260) == STRIDE
    assert gemm16(lib, qa=Q, sa=S, ldq=264) == STRIDE
    assert gemm16(lib, lda=(1 << 23) + 8, K=256) == UNSUP
    need = lib.fgq_gemm_workspace_bytes(64, 18432, 7168)
    assert gemm16(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168) == NULL      # no workspace
    assert gemm16(lib, M=64, N=18432, K=7168, ldc=18432, lda=7168, ldw=7168, ws=P, ws_bytes=need - 1) == SHAPE


def test_gemm_noalloc_validation(lib):
    na = lib.fgq_gemm_fp8_blockscaled_noalloc

    def call(qa=P, lda=256, sa=S, qw=Q, ldw=256, sw=S, c=Q, ldc=256, M=4, N=256, K=256, mode=0):
        return na(qa, lda, sa, 2, 1, qw, ldw, sw, 2, 1, c, ldc, M, N, K, mode, None)
    assert call(M=-1) == SHAPE
    assert call(mode=2) == UNSUP
    assert call(N=100) == UNSUP
    assert call(K=0) == UNSUP
    assert call(M=0) == OK
    assert call(N=0) == OK
    assert call(qa=0) == NULL
    assert call(c=Q + 2) == ALIGN
    assert call(lda=128) == STRIDE
    assert call(lda=(1 << 24) + 16) == UNSUP
    assert lib.fgq_status_string(7)
