"""BitNet b1.58 BitLinear forward on MI355X (gfx950).

A thin torch-facing binding over the C ABI in ``include/bitlinear.h``: these
functions only check and marshal arguments (device pointers, sizes, the
current HIP stream); every step of the computation runs in the HIP kernels of
``libbitlinear.so``.  There is no CPU fallback: without the built library or a
GPU the calls raise.

    packed, gamma = quantize_weights(W)           # W: float32 [N, K] on the GPU
    Y = forward(X, packed, gamma, K)              # X: float32/bfloat16 [M, K] -> float32 [M, N]
"""
from __future__ import annotations

from . import abi
from .abi import BitLinearError

__all__ = [
    "BitLinearError",
    "padded_k",
    "packed_words",
    "quantize_weights",
    "quantize_activations",
    "forward",
    "forward_batched",
    "forward_quantized",
    "forward_noalloc",
    "max_decode_m",
    "decode_fits",
    "ffn_forward",
    "pack_transposed",
    "backward",
    "r3_padded_k",
    "r3_row_bytes",
    "r3_decode_fits",
    "quantize_weights_r3",
    "forward_r3",
]


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes_void(torch.cuda.current_stream(t.device).cuda_stream)


def ctypes_void(v):
    import ctypes
    return ctypes.c_void_p(v)


def _ptr(t):
    import ctypes
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def padded_k(K: int) -> int:
    return int(abi.load().bitlinear_padded_k(K))


def packed_words(K: int) -> int:
    """uint32 words per packed row."""
    return padded_k(K) // 16


def max_decode_m() -> int:
    return int(abi.load().bitlinear_max_decode_m())


def decode_fits(M: int, K: int, N: int) -> bool:
    """Whether the decode kernel takes an M x K activation against N weight rows."""
    lib = abi.load()
    return (M <= lib.bitlinear_max_decode_m()
            and M * (padded_k(K) + 16) <= lib.bitlinear_max_decode_codes()
            and M * N < (1 << 29))


def _x_dtype(X):
    torch = _torch()
    if X.dtype == torch.float32:
        return abi.F32
    if X.dtype == torch.bfloat16:
        return abi.BF16
    raise ValueError("X must be float32 or bfloat16")


def quantize_weights(W, out_packed=None, out_gamma=None, workspace=None):
    """AbsMean ternarisation + 2-bit packing of a float32 [N, K] GPU tensor.

    Returns (packed int32 [N, padded_k(K) // 16] holding uint32 words, gamma float32 [1]);
    ``out_packed`` / ``out_gamma`` / ``workspace`` may be given to avoid allocations.
    """
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a float32 [N, K] tensor")
    lib = abi.load()
    N, K = W.shape
    packed = out_packed if out_packed is not None else torch.empty(
        (N, packed_words(K)), dtype=torch.int32, device=W.device)
    gamma = out_gamma if out_gamma is not None else torch.empty((1,), dtype=torch.float32,
                                                                device=W.device)
    if packed.shape != (N, packed_words(K)) or packed.element_size() != 4 or gamma.numel() < 1:
        raise ValueError("output buffers have the wrong shape")
    _require_cuda(packed, "out_packed")
    if workspace is not None:
        _require_cuda(workspace, "workspace")
        ws = workspace
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        ws_bytes = lib.bitlinear_quantize_workspace_bytes()
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=W.device)
    abi.check("bitlinear_quantize_weights",
              lib.bitlinear_quantize_weights(_ptr(W), N, K, _ptr(packed), _ptr(gamma), _ptr(ws),
                                             ws_bytes, _stream(W)))
    return packed, gamma


def quantize_activations(X):
    """Per-token AbsMax INT8 codes: (Xq int8 [M, padded_k(K)], gamma_a float32 [M], rowsum int32 [M])."""
    torch = _torch()
    _require_cuda(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    lib = abi.load()
    M, K = X.shape
    Xq = torch.empty((M, padded_k(K)), dtype=torch.int8, device=X.device)
    ga = torch.empty((M,), dtype=torch.float32, device=X.device)
    rs = torch.empty((M,), dtype=torch.int32, device=X.device)
    abi.check("bitlinear_quantize_activations",
              lib.bitlinear_quantize_activations(_ptr(X), _x_dtype(X), M, K, _ptr(Xq), _ptr(ga),
                                                 _ptr(rs), _stream(X)))
    return Xq, ga, rs


_PATHS = {"auto": abi.PATH_AUTO, "decode": abi.PATH_DECODE, "prefill": abi.PATH_PREFILL}


def forward(X, packed, gamma, K: int | None = None, path: str = "auto", return_acc: bool = False,
            out=None, workspace=None):
    """Y = dequant(A_q x W_q^T) for X [M, K] (float32 or bfloat16) -> float32 [M, N].

    ``path`` forces the decode or prefill kernels; ``return_acc`` also returns
    the exact INT32 accumulator [M, N].
    """
    torch = _torch()
    _require_cuda(X, "X")
    _require_cuda(packed, "packed")
    _require_cuda(gamma, "gamma")
    if X.dim() != 2 or packed.dim() != 2:
        raise ValueError("X must be [M, K] and packed [N, words]")
    M, Kx = X.shape
    K = Kx if K is None else K
    if K != Kx:
        raise ValueError("K does not match X")
    N = packed.shape[0]
    if packed.shape[1] != packed_words(K) or packed.element_size() != 4:
        raise ValueError("packed does not hold padded_k(K) // 16 32-bit words per row")
    lib = abi.load()
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=X.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=X.device) if return_acc else None
    ws_bytes = 0
    ws = workspace
    if ws is None and not (path == "decode" or (path == "auto" and decode_fits(M, K, N))):
        ws_bytes = lib.bitlinear_forward_workspace_bytes(M, K)
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=X.device)
    elif ws is not None:
        ws_bytes = ws.numel() * ws.element_size()
    abi.check("bitlinear_forward_ex",
              lib.bitlinear_forward_ex(_ptr(X), _x_dtype(X), M, K, _ptr(packed), N, _ptr(gamma),
                                       _ptr(Y), _ptr(acc), _PATHS[path], _ptr(ws), ws_bytes,
                                       _stream(X)))
    return (Y, acc) if return_acc else Y


def forward_noalloc(X, packed, gamma, K: int | None = None, out=None):
    """bitlinear_forward_noalloc: the same forward with the library's own
    per-GPU scratch array as the prefill workspace (the C call allocates
    nothing; pass ``out`` to allocate nothing here either).  Calls that overlap
    on one GPU share that array and must be serialised."""
    torch = _torch()
    _require_cuda(X, "X")
    _require_cuda(packed, "packed")
    _require_cuda(gamma, "gamma")
    if X.dim() != 2 or packed.dim() != 2:
        raise ValueError("X must be [M, K] and packed [N, words]")
    M, Kx = X.shape
    K = Kx if K is None else K
    if K != Kx:
        raise ValueError("K does not match X")
    N = packed.shape[0]
    if packed.shape[1] != packed_words(K) or packed.element_size() != 4:
        raise ValueError("packed does not hold padded_k(K) // 16 32-bit words per row")
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=X.device)
    if Y.shape != (M, N) or Y.dtype != torch.float32:
        raise ValueError("out must be float32 [M, N]")
    _require_cuda(Y, "out")
    lib = abi.load()
    abi.check("bitlinear_forward_noalloc",
              lib.bitlinear_forward_noalloc(_ptr(X), _x_dtype(X), M, K, _ptr(packed), N, _ptr(gamma),
                                            _ptr(Y), _stream(X)))
    return Y


def forward_quantized(Xq, gamma_a, rowsum, packed, gamma, K: int, return_acc: bool = False, out=None):
    """Contraction + rescale from activation codes (as quantize_activations returns them)."""
    torch = _torch()
    for t, nm in ((Xq, "Xq"), (gamma_a, "gamma_a"), (rowsum, "rowsum"), (packed, "packed"),
                  (gamma, "gamma")):
        _require_cuda(t, nm)
    M = Xq.shape[0]
    if Xq.dtype != torch.int8 or Xq.shape[1] != padded_k(K):
        raise ValueError("Xq must be int8 [M, padded_k(K)]")
    N = packed.shape[0]
    if packed.shape[1] != packed_words(K):
        raise ValueError("packed does not hold padded_k(K) // 16 words per row")
    lib = abi.load()
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device) if return_acc else None
    abi.check("bitlinear_forward_quantized",
              lib.bitlinear_forward_quantized(_ptr(Xq), _ptr(gamma_a), _ptr(rowsum), M, K,
                                              _ptr(packed), N, _ptr(gamma), _ptr(Y), _ptr(acc),
                                              _stream(Xq)))
    return (Y, acc) if return_acc else Y


def forward_batched(X, packed, gamma, K: int | None = None, out=None):
    """L decode forwards in one launch: X [L, M, K], packed [L, N, words], gamma [L] -> Y [L, M, N]."""
    torch = _torch()
    for t, nm in ((X, "X"), (packed, "packed"), (gamma, "gamma")):
        _require_cuda(t, nm)
    if X.dim() != 3 or packed.dim() != 3:
        raise ValueError("X must be [L, M, K] and packed [L, N, words]")
    L, M, Kx = X.shape
    K = Kx if K is None else K
    if K != Kx or packed.shape[0] != L or gamma.numel() != L:
        raise ValueError("inconsistent batched shapes")
    N = packed.shape[1]
    if packed.shape[2] != packed_words(K):
        raise ValueError("packed does not hold padded_k(K) // 16 words per row")
    lib = abi.load()
    Y = out if out is not None else torch.empty((L, M, N), dtype=torch.float32, device=X.device)
    abi.check("bitlinear_forward_batched",
              lib.bitlinear_forward_batched(L, _ptr(X), _x_dtype(X), M, K, _ptr(packed), N,
                                            _ptr(gamma), _ptr(Y), _stream(X)))
    return Y


# ---- radix-3 weights (five per byte) --------------------------------------

def r3_padded_k(K: int) -> int:
    return int(abi.load().bitlinear_r3_padded_k(K))


def r3_row_bytes(K: int) -> int:
    """Bytes per radix-3 packed row."""
    return r3_padded_k(K) // 5


def r3_decode_fits(M: int, K: int, N: int) -> bool:
    lib = abi.load()
    return (M <= lib.bitlinear_max_decode_m()
            and M * (r3_padded_k(K) + 16) <= lib.bitlinear_max_decode_codes()
            and M * N < (1 << 29))


def quantize_weights_r3(W, out_packed=None, out_gamma=None, workspace=None):
    """AbsMean ternarisation of a float32 [N, K] GPU tensor, packed five weights per byte.

    Returns (packed uint8 [N, r3_row_bytes(K)], gamma float32 [1]); gamma and the
    ternary codes are bit-identical to :func:`quantize_weights`.
    """
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a float32 [N, K] tensor")
    lib = abi.load()
    N, K = W.shape
    packed = out_packed if out_packed is not None else torch.empty(
        (N, r3_row_bytes(K)), dtype=torch.uint8, device=W.device)
    gamma = out_gamma if out_gamma is not None else torch.empty((1,), dtype=torch.float32,
                                                                device=W.device)
    if packed.shape != (N, r3_row_bytes(K)) or packed.element_size() != 1 or gamma.numel() < 1:
        raise ValueError("output buffers have the wrong shape")
    _require_cuda(packed, "out_packed")
    if workspace is not None:
        _require_cuda(workspace, "workspace")
        ws = workspace
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        ws_bytes = lib.bitlinear_quantize_workspace_bytes()
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=W.device)
    abi.check("bitlinear_quantize_weights_r3",
              lib.bitlinear_quantize_weights_r3(_ptr(W), N, K, _ptr(packed), _ptr(gamma), _ptr(ws),
                                                ws_bytes, _stream(W)))
    return packed, gamma


def forward_r3(X, packed, gamma, K: int | None = None, return_acc: bool = False, out=None):
    """Decode forward over radix-3 weights.

    X [M, K] with packed [N, r3_row_bytes(K)] and gamma [1], or X [L, M, K] with
    packed [L, N, r3_row_bytes(K)] and gamma [L] (L layers in one launch).
    Returns Y float32 [M, N] / [L, M, N] (and the INT32 accumulators if asked).
    """
    torch = _torch()
    for t, nm in ((X, "X"), (packed, "packed"), (gamma, "gamma")):
        _require_cuda(t, nm)
    batched = X.dim() == 3
    if batched:
        if packed.dim() != 3:
            raise ValueError("X [L, M, K] needs packed [L, N, bytes]")
        L, M, Kx = X.shape
        N = packed.shape[1]
        if packed.shape[0] != L or gamma.numel() != L:
            raise ValueError("inconsistent batched shapes")
    else:
        if X.dim() != 2 or packed.dim() != 2:
            raise ValueError("X must be [M, K] and packed [N, bytes]")
        L = 1
        M, Kx = X.shape
        N = packed.shape[0]
    K = Kx if K is None else K
    if K != Kx:
        raise ValueError("K does not match X")
    if packed.shape[-1] != r3_row_bytes(K) or packed.element_size() != 1:
        raise ValueError("packed does not hold r3_row_bytes(K) bytes per row")
    lib = abi.load()
    shape = (L, M, N) if batched else (M, N)
    Y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=X.device)
    acc = torch.empty(shape, dtype=torch.int32, device=X.device) if return_acc else None
    abi.check("bitlinear_forward_r3",
              lib.bitlinear_forward_r3(L, _ptr(X), _x_dtype(X), M, K, _ptr(packed), N, _ptr(gamma),
                                       _ptr(Y), _ptr(acc), _stream(X)))
    return (Y, acc) if return_acc else Y


# ---- LUT contraction (comparison variant) ----------------------------------

def lut_workspace_bytes(L: int, M: int, K: int) -> int:
    return int(abi.load().bitlinear_lut_workspace_bytes(L, M, K))


def forward_lut(X, packed, gamma, K: int | None = None, return_acc: bool = False, out=None, workspace=None):
    """Decode forward through 81-entry LUTs over 2-bit weights (a comparison to ``forward``).

    X [M, K] with packed [N, words] and gamma [1], or X [L, M, K] with
    packed [L, N, words] and gamma [L].  Returns Y float32 [M, N] / [L, M, N]
    (and the INT32 accumulators if asked).
    """
    torch = _torch()
    for t, nm in ((X, "X"), (packed, "packed"), (gamma, "gamma")):
        _require_cuda(t, nm)
    batched = X.dim() == 3
    if batched:
        if packed.dim() != 3:
            raise ValueError("X [L, M, K] needs packed [L, N, words]")
        L, M, Kx = X.shape
        N = packed.shape[1]
        if packed.shape[0] != L or gamma.numel() != L:
            raise ValueError("inconsistent batched shapes")
    else:
        if X.dim() != 2 or packed.dim() != 2:
            raise ValueError("X must be [M, K] and packed [N, words]")
        L = 1
        M, Kx = X.shape
        N = packed.shape[0]
    K = Kx if K is None else K
    if K != Kx:
        raise ValueError("K does not match X")
    if packed.shape[-1] != packed_words(K):
        raise ValueError("packed does not hold padded_k(K) // 16 words per row")
    lib = abi.load()
    ws_bytes = int(lib.bitlinear_lut_workspace_bytes(L, M, K))
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=X.device)
    shape = (L, M, N) if batched else (M, N)
    Y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=X.device)
    acc = torch.empty(shape, dtype=torch.int32, device=X.device) if return_acc else None
    abi.check("bitlinear_forward_lut",
              lib.bitlinear_forward_lut(L, _ptr(X), _x_dtype(X), M, K, _ptr(packed), N, _ptr(gamma),
                                        _ptr(Y), _ptr(acc), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(X)))
    return (Y, acc) if return_acc else Y


# ---- the BitNet FFN block --------------------------------------------------

def ffn_forward(X, up, down, path: str = "auto", return_hidden: bool = False, out=None, workspace=None):
    """Y = BitLinear_down(ReLU^2(BitLinear_up(X))).

    ``up`` = (packed [F, words(D)], gamma [1]) and ``down`` = (packed [D_out, words(F)],
    gamma [1]) as :func:`quantize_weights` returns them, with X [M, D]; or X
    [L, M, D] with packed [L, ...] and gamma [L] for L layers.  Returns Y float32
    [(L,) M, D_out] (and the hidden ReLU^2 activations [(L,) M, F] if asked).
    """
    torch = _torch()
    (pu, gu), (pd, gd) = up, down
    for t, nm in ((X, "X"), (pu, "packed_up"), (gu, "gamma_up"), (pd, "packed_down"), (gd, "gamma_down")):
        _require_cuda(t, nm)
    batched = X.dim() == 3
    if batched:
        L, M, D = X.shape
        F, Do = pu.shape[1], pd.shape[1]
        if pu.dim() != 3 or pd.dim() != 3 or pu.shape[0] != L or pd.shape[0] != L or gu.numel() != L \
                or gd.numel() != L:
            raise ValueError("inconsistent batched shapes")
    else:
        L = 1
        M, D = X.shape
        F, Do = pu.shape[0], pd.shape[0]
    if pu.shape[-1] != packed_words(D) or pd.shape[-1] != packed_words(F):
        raise ValueError("packed weights do not match D and F")
    lib = abi.load()
    shape = (L, M, Do) if batched else (M, Do)
    Y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=X.device)
    hid = torch.empty((L, M, F) if batched else (M, F), dtype=torch.float32, device=X.device) \
        if return_hidden else None
    if workspace is None:
        ws_bytes = lib.bitlinear_ffn_workspace_bytes(L, M, D, F)
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=X.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    abi.check("bitlinear_ffn_forward",
              lib.bitlinear_ffn_forward(L, _ptr(X), _x_dtype(X), M, D, F, Do, _ptr(pu), _ptr(gu), _ptr(pd),
                                        _ptr(gd), _ptr(Y), _ptr(hid), _PATHS[path], _ptr(workspace), ws_bytes,
                                        _stream(X)))
    return (Y, hid) if return_hidden else Y


# ---- backward with the straight-through estimator ---------------------------

def pack_transposed(W, gamma, out=None, mask_out=None):
    """What the backward needs from W (once per weight update): the codes of
    W^T ([K, padded_k(N) // 16] words, for dX) and the range mask (int32
    [N, ceil(K / 32)] bit words, for dW); gamma from quantize_weights(W)."""
    torch = _torch()
    _require_cuda(W, "W")
    _require_cuda(gamma, "gamma")
    N, K = W.shape
    lib = abi.load()
    packedT = out if out is not None else torch.empty((K, packed_words(N)), dtype=torch.int32, device=W.device)
    mask = mask_out if mask_out is not None else torch.empty((N, (K + 31) // 32), dtype=torch.int32,
                                                             device=W.device)
    abi.check("bitlinear_pack_transposed",
              lib.bitlinear_pack_transposed(_ptr(W), N, K, _ptr(gamma), _ptr(packedT), _ptr(mask), _stream(W)))
    return packedT, mask


def backward(dY, packedT, gamma, Xq, gamma_a, mask, K: int, need_dx: bool = True, need_dw: bool = True,
             workspace=None):
    """STE gradients (dX [M, K], dW [N, K], float32) of the forward from dY (bfloat16 [M, N]).

    ``Xq``/``gamma_a``: the forward's activation codes (quantize_activations);
    ``packedT``/``mask``: pack_transposed(W, gamma); K: the weights' columns.
    """
    torch = _torch()
    for t, nm in ((dY, "dY"), (gamma, "gamma")):
        _require_cuda(t, nm)
    if dY.dtype != torch.bfloat16:
        raise ValueError("dY must be bfloat16")
    M, N = dY.shape
    lib = abi.load()
    dX = torch.empty((M, K), dtype=torch.float32, device=dY.device) if need_dx else None
    dW = torch.empty((N, K), dtype=torch.float32, device=dY.device) if need_dw else None
    if workspace is None:
        workspace = torch.empty((lib.bitlinear_backward_workspace_bytes(M, N, K),), dtype=torch.uint8,
                                device=dY.device)
    abi.check("bitlinear_backward",
              lib.bitlinear_backward(_ptr(dY), M, N, K, _ptr(packedT), _ptr(gamma), _ptr(Xq), _ptr(gamma_a),
                                     _ptr(mask), _ptr(dX), _ptr(dW), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(dY)))
    return dX, dW
