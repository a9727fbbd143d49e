"""The C ABI on the host: the library loads, exports every function the header
declares, sizes are right, and every argument check fires before any HIP call
(no kernel is launched here: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

from bitlinear_absmean_ternarise_bit_amd import abi
from bitlinear_absmean_ternarise_bit_amd.build import LIB_PATH, build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")
PROBE_HEADER = os.path.join(ROOT, "include", "bitlinear_probe.h")

P = ctypes.c_void_p
FAKE = P(4096)  # a non-null, 256-byte aligned address: never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build_library()
    return abi.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 26
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(abi.SIGNATURES)


def test_probe_library_is_separate(lib):
    """The attainable-peak probes live in their own library and header: the
    BitLinear library neither declares nor exports them."""
    probe = abi.load_probe()
    names = declared_functions(PROBE_HEADER)
    assert names == ["bitlinear_probe_mfma_bf16", "bitlinear_probe_mfma_i8", "bitlinear_probe_stream"]
    for n in names:
        assert hasattr(probe, n), n
        assert n not in abi.SIGNATURES
        with pytest.raises(AttributeError):
            getattr(lib, n)
    assert set(names) == set(abi.PROBE_SIGNATURES)


def test_sizes(lib):
    assert lib.bitlinear_padded_k(1) == 64
    assert lib.bitlinear_padded_k(64) == 64
    assert lib.bitlinear_padded_k(65) == 128
    assert lib.bitlinear_padded_k(0) == 0
    assert lib.bitlinear_packed_bytes(2048, 2048) == 2048 * 2048 // 4  # 0.25 byte per weight
    assert lib.bitlinear_packed_bytes(3, 100) == 3 * 128 // 4
    assert lib.bitlinear_packed_bytes(0, 5) == 0
    assert 0 < lib.bitlinear_quantize_workspace_bytes() < 128 * 1024
    assert lib.bitlinear_forward_workspace_bytes(10, 100) >= 10 * 128 + 80
    assert lib.bitlinear_forward_workspace_bytes(10, 100) % 256 == 0
    assert lib.bitlinear_max_decode_m() == 16
    assert lib.bitlinear_max_decode_codes() == 65536


def test_r3_sizes(lib):
    assert lib.bitlinear_r3_padded_k(1) == 80
    assert lib.bitlinear_r3_padded_k(80) == 80
    assert lib.bitlinear_r3_padded_k(81) == 160
    assert lib.bitlinear_r3_padded_k(0) == 0
    assert lib.bitlinear_r3_packed_bytes(2048, 2080) == 2048 * 2080 // 5  # 1.6 bits per weight
    assert lib.bitlinear_r3_packed_bytes(3, 100) == 3 * 160 // 5
    assert lib.bitlinear_r3_packed_bytes(5, 0) == 0


def test_r3_checks(lib):
    ws = lib.bitlinear_quantize_workspace_bytes()
    f = lib.bitlinear_quantize_weights_r3
    assert f(None, 4, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_NULL
    assert f(FAKE, 4, 4, None, FAKE, FAKE, ws, None) == abi.ERR_NULL
    assert f(FAKE, 0, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 1 << 13, 1 << 19, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 4, 4, P(4104), FAKE, FAKE, ws, None) == abi.ERR_ALIGN
    assert f(FAKE, 4, 4, FAKE, FAKE, FAKE, ws - 1, None) == abi.ERR_WORKSPACE
    g = lib.bitlinear_forward_r3
    #   L, X, dt, M, K, packed, N, gamma, Y, acc, stream
    assert g(1, None, 0, 1, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_NULL
    assert g(1, FAKE, 0, 1, 64, FAKE, 8, FAKE, None, None, None) == abi.ERR_NULL
    assert g(0, FAKE, 0, 1, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_SHAPE
    assert g(1, FAKE, 0, 17, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_SHAPE   # M > 16
    assert g(1, FAKE, 0, 16, 4081, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_SHAPE  # codes > LDS
    assert g(1, FAKE, 2, 1, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_DTYPE
    assert g(1, FAKE, 0, 1, 64, P(4104), 8, FAKE, FAKE, None, None) == abi.ERR_ALIGN
    assert g(1, FAKE, 0, 1, 64, FAKE, 8, FAKE, FAKE, P(4098), None) == abi.ERR_ALIGN


def test_lut_checks(lib):
    assert lib.bitlinear_lut_workspace_bytes(3, 8, 100) == lib.bitlinear_forward_workspace_bytes(24, 100)
    assert lib.bitlinear_lut_workspace_bytes(1, 17, 100) == 0   # at most 16 tokens
    assert lib.bitlinear_lut_workspace_bytes(0, 1, 100) == 0
    f = lib.bitlinear_forward_lut
    ws = lib.bitlinear_lut_workspace_bytes(2, 4, 64)
    #   L, X, dt, M, K, packed, N, gamma, Y, acc, ws, ws_bytes, stream
    args = [2, FAKE, 1, 4, 64, FAKE, 8, FAKE, FAKE, None, FAKE, ws, None]

    def call(**kw):
        a = list(args)
        names = ["L", "X", "dt", "M", "K", "packed", "N", "gamma", "Y", "acc", "ws", "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(X=None) == abi.ERR_NULL
    assert call(packed=None) == abi.ERR_NULL
    assert call(Y=None) == abi.ERR_NULL
    assert call(L=0) == abi.ERR_SHAPE
    assert call(M=0) == abi.ERR_SHAPE
    assert call(M=17) == abi.ERR_SHAPE
    assert call(N=0) == abi.ERR_SHAPE
    assert call(K=(1 << 20) + 1) == abi.ERR_SHAPE
    assert call(dt=7) == abi.ERR_DTYPE
    assert call(X=P(4097)) == abi.ERR_ALIGN
    assert call(packed=P(4104)) == abi.ERR_ALIGN
    assert call(acc=P(4098)) == abi.ERR_ALIGN
    assert call(ws=None) == abi.ERR_WORKSPACE
    assert call(wsb=ws - 1) == abi.ERR_WORKSPACE
    assert call(ws=P(4096 + 16)) == abi.ERR_ALIGN


def test_backward_checks(lib):
    assert lib.bitlinear_ste_mask_bytes(3, 33) == 3 * 2 * 4
    assert lib.bitlinear_ste_mask_bytes(5, 64) == 5 * 2 * 4
    assert lib.bitlinear_ste_mask_bytes(0, 64) == 0
    pt = lib.bitlinear_pack_transposed
    #   W, N, K, gamma, packedT, mask, stream
    assert pt(None, 4, 4, FAKE, FAKE, FAKE, None) == abi.ERR_NULL
    assert pt(FAKE, 4, 4, FAKE, None, None, None) == abi.ERR_NULL  # neither output
    assert pt(FAKE, 0, 4, FAKE, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert pt(FAKE, 4, 4, FAKE, P(4104), None, None) == abi.ERR_ALIGN
    assert pt(FAKE, 4, 4, FAKE, None, P(4098), None) == abi.ERR_ALIGN
    bw = lib.bitlinear_backward
    ws = lib.bitlinear_backward_workspace_bytes(4, 8, 8)
    #   dY, M, N, K, packedT, gamma, Xq, gamma_a, mask, dX, dW, ws, ws_bytes, stream
    args = [FAKE, 4, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]

    def call(**kw):
        a = list(args)
        names = ["dY", "M", "N", "K", "pT", "g", "Xq", "ga", "mask", "dX", "dW", "ws", "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return bw(*a)

    assert call(dY=None) == abi.ERR_NULL
    assert call(dX=None, dW=None) == abi.ERR_NULL
    assert call(pT=None) == abi.ERR_NULL                 # dX needs the transposed codes
    assert call(mask=None) == abi.ERR_NULL               # dW needs the range mask
    assert call(M=0) == abi.ERR_SHAPE
    assert call(mask=P(4098)) == abi.ERR_ALIGN
    assert call(ws=None) == abi.ERR_WORKSPACE
    assert call(wsb=ws - 1) == abi.ERR_WORKSPACE


def test_ffn_checks(lib):
    f = lib.bitlinear_ffn_forward
    ws = lib.bitlinear_ffn_workspace_bytes(1, 4, 64, 128)
    assert ws >= 4 * 128 * 4
    assert lib.bitlinear_ffn_workspace_bytes(0, 4, 64, 128) == 0
    #   L, X, dt, M, D, F, Do, pu, gu, pd, gd, Y, hidden, path, ws, ws_bytes, stream
    args = [1, FAKE, 0, 4, 64, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, ws, None]

    def call(**kw):
        a = list(args)
        names = ["L", "X", "dt", "M", "D", "F", "Do", "pu", "gu", "pd", "gd", "Y", "hid", "path", "ws",
                 "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(X=None) == abi.ERR_NULL
    assert call(pd=None) == abi.ERR_NULL
    assert call(Y=None) == abi.ERR_NULL
    assert call(L=0) == abi.ERR_SHAPE
    assert call(F=0) == abi.ERR_SHAPE
    assert call(Do=-1) == abi.ERR_SHAPE
    assert call(dt=5) == abi.ERR_DTYPE
    assert call(path=9) == abi.ERR_ARG
    assert call(pu=P(4104)) == abi.ERR_ALIGN
    assert call(hid=P(4100)) == abi.ERR_ALIGN
    assert call(M=17, path=1) == abi.ERR_SHAPE            # decode forced beyond 16 tokens
    assert call(ws=None) == abi.ERR_WORKSPACE            # hidden layer needs the workspace
    assert call(wsb=4 * 128 * 4 - 1) == abi.ERR_WORKSPACE     # decode path: the hidden layer ...
    assert call(wsb=4 * 128 * 4 + 256) == abi.ERR_WORKSPACE   # ... and the codes of its rows
    assert call(hid=FAKE, ws=None) == abi.ERR_WORKSPACE      # codes even with a caller hidden buffer
    assert call(path=2, wsb=4 * 128 * 4) == abi.ERR_WORKSPACE  # prefill also holds activation codes
    assert call(ws=P(4096 + 16)) == abi.ERR_ALIGN


def test_status_strings(lib):
    for s in range(-7, 1):
        assert abi.status_string(s)
    assert abi.status_string(-99) == "unknown status"


def test_quantize_weights_checks(lib):
    ws = lib.bitlinear_quantize_workspace_bytes()
    f = lib.bitlinear_quantize_weights
    assert f(None, 4, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_NULL
    assert f(FAKE, 4, 4, None, FAKE, FAKE, ws, None) == abi.ERR_NULL
    assert f(FAKE, 4, 4, FAKE, None, FAKE, ws, None) == abi.ERR_NULL
    assert f(FAKE, 0, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 4, -1, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 4, (1 << 20) + 1, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 1 << 13, 1 << 19, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE  # N*K >= 2^32
    # packed matrices of 2 GiB or more: N * padded_k(K) / 4 >= 2^31 (rows of K = 1 pad to 64)
    assert f(FAKE, 1 << 28, 1, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 1 << 27, 1, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(FAKE, 1 << 27, 64, FAKE, FAKE, FAKE, ws, None) == abi.ERR_SHAPE
    assert f(P(4100), 4, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_ALIGN
    assert f(FAKE, 4, 4, P(4104), FAKE, FAKE, ws, None) == abi.ERR_ALIGN
    assert f(FAKE, 4, 4, FAKE, P(4098), FAKE, ws, None) == abi.ERR_ALIGN
    assert f(FAKE, 4, 4, FAKE, FAKE, None, ws, None) == abi.ERR_WORKSPACE
    assert f(FAKE, 4, 4, FAKE, FAKE, FAKE, ws - 1, None) == abi.ERR_WORKSPACE
    assert f(FAKE, 4, 4, FAKE, FAKE, P(4100), ws, None) == abi.ERR_ALIGN


def test_quantize_activations_checks(lib):
    f = lib.bitlinear_quantize_activations
    assert f(None, 0, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_NULL
    assert f(FAKE, 0, 2, 8, FAKE, None, FAKE, None) == abi.ERR_NULL
    assert f(FAKE, 2, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_DTYPE
    assert f(FAKE, -1, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_DTYPE
    assert f(FAKE, 0, 0, 8, FAKE, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(FAKE, 0, 2, 0, FAKE, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(P(4098), 0, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_ALIGN  # f32 needs 4 bytes
    assert f(P(4097), 1, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_ALIGN  # bf16 needs 2 bytes
    assert f(FAKE, 0, 2, 8, P(4100), FAKE, FAKE, None) == abi.ERR_ALIGN


def test_forward_checks(lib):
    f = lib.bitlinear_forward_ex
    wsb = lib.bitlinear_forward_workspace_bytes(64, 128)
    args = dict(X=FAKE, dt=0, M=64, K=128, packed=FAKE, N=32, gamma=FAKE, Y=FAKE, acc=None,
                path=0, ws=FAKE, wsb=wsb)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["X"], a["dt"], a["M"], a["K"], a["packed"], a["N"], a["gamma"], a["Y"], a["acc"],
                 a["path"], a["ws"], a["wsb"], None)

    assert call(X=None) == abi.ERR_NULL
    assert call(packed=None) == abi.ERR_NULL
    assert call(gamma=None) == abi.ERR_NULL
    assert call(Y=None) == abi.ERR_NULL
    assert call(M=0) == abi.ERR_SHAPE
    assert call(N=0) == abi.ERR_SHAPE
    assert call(K=0) == abi.ERR_SHAPE
    assert call(dt=7) == abi.ERR_DTYPE
    assert call(path=3) == abi.ERR_ARG
    assert call(packed=P(4104)) == abi.ERR_ALIGN
    assert call(Y=P(4098)) == abi.ERR_ALIGN
    assert call(acc=P(4098)) == abi.ERR_ALIGN
    # prefill path (M > 16) needs the workspace
    assert call(ws=None) == abi.ERR_WORKSPACE
    assert call(wsb=wsb - 1) == abi.ERR_WORKSPACE
    assert call(ws=P(4096 + 16)) == abi.ERR_ALIGN
    # forcing decode beyond its limits
    assert call(path=1) == abi.ERR_SHAPE  # M = 64 > 16
    assert call(M=16, K=4096, path=1) == abi.ERR_SHAPE  # 16 * (4096 + 16) > 65536
    g = lib.bitlinear_forward
    assert g(FAKE, 0, 64, 128, FAKE, 32, FAKE, FAKE, None, 0, None) == abi.ERR_WORKSPACE


def test_forward_quantized_checks(lib):
    f = lib.bitlinear_forward_quantized
    assert f(None, FAKE, FAKE, 4, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_NULL
    assert f(FAKE, FAKE, None, 4, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_NULL
    assert f(FAKE, FAKE, FAKE, 0, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_SHAPE
    assert f(P(4104), FAKE, FAKE, 4, 64, FAKE, 8, FAKE, FAKE, None, None) == abi.ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 64, FAKE, 8, FAKE, FAKE, P(4098), None) == abi.ERR_ALIGN


def test_forward_batched_checks(lib):
    f = lib.bitlinear_forward_batched
    assert f(0, FAKE, 1, 1, 2048, FAKE, 2048, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(4, None, 1, 1, 2048, FAKE, 2048, FAKE, FAKE, None) == abi.ERR_NULL
    assert f(4, FAKE, 1, 17, 2048, FAKE, 2048, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(4, FAKE, 5, 1, 2048, FAKE, 2048, FAKE, FAKE, None) == abi.ERR_DTYPE
    assert f(4, FAKE, 1, 1, 2048, P(4100), 2048, FAKE, FAKE, None) == abi.ERR_ALIGN


def test_probe_checks(lib):
    probe = abi.load_probe()
    s, m = probe.bitlinear_probe_stream, probe.bitlinear_probe_mfma_i8
    assert s(None, FAKE, 1 << 20, 32, None, None) == abi.ERR_NULL
    assert s(FAKE, None, 1 << 20, 32, None, None) == abi.ERR_NULL       # neither dst nor out
    assert s(FAKE, FAKE, (1 << 20) + 16, 32, None, None) == abi.ERR_SHAPE  # not a multiple of 32 KiB per block
    assert s(FAKE, FAKE, 1 << 20, 0, None, None) == abi.ERR_SHAPE
    assert s(FAKE, FAKE, 1 << 32, 1, None, None) == abi.ERR_SHAPE       # a slice of 2^32 bytes
    assert s(P(4100), FAKE, 1 << 20, 32, None, None) == abi.ERR_ALIGN
    assert m(1, 1, None, None) == abi.ERR_NULL
    assert m(0, 1, FAKE, None) == abi.ERR_SHAPE
    assert m(1, 0, FAKE, None) == abi.ERR_SHAPE
    h = probe.bitlinear_probe_mfma_bf16
    assert h(1, 1, None, None) == abi.ERR_NULL
    assert h(0, 1, FAKE, None) == abi.ERR_SHAPE
    assert h(1, 0, FAKE, None) == abi.ERR_SHAPE
    assert h(1, 1, P(4098), None) == abi.ERR_ALIGN


def test_header_documents_citations_and_conventions():
    text = open(HEADER).read()
    for fn in declared_functions():
        assert fn in text
    assert "PMV" in text and "DEVICE pointers" in text


def test_size_queries_saturate_to_zero(lib):
    """Size queries take any int64: out-of-range arguments (< 1 or > 2^40) and
    products that would not fit in size_t give 0 rather than a wrapped value."""
    huge, neg = (1 << 63) - 1, -(1 << 63)
    for v in (0, -1, neg, huge, (1 << 40) + 1):
        assert lib.bitlinear_padded_k(v) == 0
        assert lib.bitlinear_r3_padded_k(v) == 0
        assert lib.bitlinear_packed_bytes(v, 64) == 0 and lib.bitlinear_packed_bytes(64, v) == 0
        assert lib.bitlinear_r3_packed_bytes(v, 80) == 0 and lib.bitlinear_r3_packed_bytes(80, v) == 0
        assert lib.bitlinear_forward_workspace_bytes(v, 64) == 0
        assert lib.bitlinear_forward_workspace_bytes(64, v) == 0
        assert lib.bitlinear_ste_mask_bytes(v, 64) == 0 and lib.bitlinear_ste_mask_bytes(64, v) == 0
        assert lib.bitlinear_backward_workspace_bytes(v, 64, 64) == 0
        assert lib.bitlinear_backward_workspace_bytes(64, v, 64) == 0
        assert lib.bitlinear_backward_workspace_bytes(64, 64, v) == 0
        assert lib.bitlinear_ffn_workspace_bytes(v, 8, 64, 64) == 0
        assert lib.bitlinear_ffn_workspace_bytes(1, v, 64, 64) == 0
        assert lib.bitlinear_lut_workspace_bytes(v, 8, 64) == 0
    t = 1 << 40
    assert lib.bitlinear_padded_k(t) == t
    assert lib.bitlinear_packed_bytes(t, t) == 0          # 2^78 bytes: does not fit size_t
    assert lib.bitlinear_backward_workspace_bytes(t, t, t) == 0
    assert lib.bitlinear_packed_bytes(t, 64) == t * 16


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="a GPU is present: valid arguments would launch kernels on it")
def test_launch_without_a_device_returns_err_hip(lib):
    """With no GPU in the machine, calls whose arguments pass every check reach
    the launch, which fails; the failure comes back as BITLINEAR_ERR_HIP (never
    an abort).  The pointers are never dereferenced: nothing runs."""
    ws = lib.bitlinear_quantize_workspace_bytes()
    assert lib.bitlinear_quantize_weights(FAKE, 4, 4, FAKE, FAKE, FAKE, ws, None) == abi.ERR_HIP
    assert lib.bitlinear_quantize_activations(FAKE, 1, 2, 8, FAKE, FAKE, FAKE, None) == abi.ERR_HIP
    # decode path (M <= 16) and prefill path (M > 16) of the forward
    assert lib.bitlinear_forward(FAKE, 0, 1, 64, FAKE, 16, FAKE, FAKE, None, 0, None) == abi.ERR_HIP
    wsb = lib.bitlinear_forward_workspace_bytes(64, 128)
    assert lib.bitlinear_forward(FAKE, 1, 64, 128, FAKE, 32, FAKE, FAKE, FAKE, wsb, None) == abi.ERR_HIP
    assert lib.bitlinear_forward_batched(4, FAKE, 1, 1, 2048, FAKE, 2048, FAKE, FAKE, None) == abi.ERR_HIP
    assert lib.bitlinear_forward_quantized(FAKE, FAKE, FAKE, 4, 64, FAKE, 8, FAKE, FAKE, None,
                                           None) == abi.ERR_HIP


def test_forward_noalloc_checks(lib):
    """The allocation-free forward checks its arguments like the forward, and
    rejects a prefill problem whose workspace exceeds its scratch array before
    any HIP call."""
    f = lib.bitlinear_forward_noalloc
    assert f(None, 0, 64, 128, FAKE, 32, FAKE, FAKE, None) == abi.ERR_NULL
    assert f(FAKE, 0, 64, 128, FAKE, 32, FAKE, None, None) == abi.ERR_NULL
    assert f(FAKE, 0, 0, 128, FAKE, 32, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(FAKE, 0, 1, 1, FAKE, 1 << 28, FAKE, FAKE, None) == abi.ERR_SHAPE
    assert f(FAKE, 4, 64, 128, FAKE, 32, FAKE, FAKE, None) == abi.ERR_DTYPE
    assert f(FAKE, 0, 64, 128, P(4104), 32, FAKE, FAKE, None) == abi.ERR_ALIGN
    # 16384 tokens of K = 8192: 128 MiB of codes, more than the 80 MiB array
    assert lib.bitlinear_forward_workspace_bytes(16384, 8192) > abi.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, 1, 16384, 8192, FAKE, 64, FAKE, FAKE, None) == abi.ERR_WORKSPACE
    # the largest problems of the two prefill workloads fit
    assert lib.bitlinear_forward_workspace_bytes(8192, 8192) <= abi.NOALLOC_SCRATCH_BYTES
    assert lib.bitlinear_forward_workspace_bytes(16384, 4096) <= abi.NOALLOC_SCRATCH_BYTES
    m = re.search(r"#define BITLINEAR_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", open(HEADER).read())
    assert m and int(m.group(1)) << 20 == abi.NOALLOC_SCRATCH_BYTES
