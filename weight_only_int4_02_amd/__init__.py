"""MI355X (gfx950) W4A16 group-quantized GEMM:  Y = X . dequant(Q)^T.

A thin ctypes binding over libw4a16.so (C ABI in include/w4a16.h).  It only
marshals arguments: torch supplies device memory and the current HIP stream,
and every step of the computation runs in the library's HIP kernels.  There is
no CPU fallback: if the library is missing the calls raise.

    codes  uint8  [N, K] (values 0..15)   -> pack()    -> qpacked int32 [N, K/8]
    zeros  uint8  [N, G]                  -> pack()    -> zpacked int32 [N, ceil(G/8)]
    (qpacked, scales fp16 [N, G], zpacked) -> repack()  -> PackedWeight (device layout)
    X fp16 [M, K], PackedWeight           -> gemm()    -> Y fp16 [M, N]
    (qpacked, scales, zpacked)            -> dequant() -> W fp16 [N, K]
    W fp16 [N, K]                         -> quantize() -> (qpacked, scales, zpacked)

uint32 bit patterns are carried in int32 tensors.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_ALIGN = -1, -2, -3, -4
ERR_WORKSPACE, ERR_ARCH, ERR_HIP, ERR_FLAGS = -5, -6, -7, -8

SYMMETRIC = 0x1
PARTIAL_LAST_GROUP = 0x2
BF16 = 0x4
PATH_SMALL_M = 0x10
PATH_LARGE_M = 0x20

# Every symbol include/w4a16.h declares.
EXPORTS = (
    "w4a16_status_str", "w4a16_last_hip_error", "w4a16_device_check",
    "w4a16_pack", "w4a16_check_pack_args",
    "w4a16_repack_size", "w4a16_repack", "w4a16_check_repack_args",
    "w4a16_dequant", "w4a16_check_dequant_args",
    "w4a16_quantize", "w4a16_check_quantize_args",
    "w4a16_gemm_workspace_size", "w4a16_gemm_kernel", "w4a16_gemm", "w4a16_check_gemm_args",
    "w4a16_stream_read", "w4a16_gemm_noalloc",
)

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class W4A16ArgumentError(W4A16Error, ValueError):
    pass


def lib():
    """The loaded libw4a16.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m weight_only_int4_02_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        SZ = ctypes.c_size_t
        PSZ = ctypes.POINTER(ctypes.c_size_t)
        L.w4a16_status_str.argtypes = [I32]
        L.w4a16_status_str.restype = ctypes.c_char_p
        L.w4a16_last_hip_error.argtypes = []
        L.w4a16_last_hip_error.restype = ctypes.c_char_p
        L.w4a16_device_check.argtypes = []
        L.w4a16_pack.argtypes = [P, I64, I64, P, P]
        L.w4a16_check_pack_args.argtypes = [P, I64, I64, P]
        L.w4a16_repack_size.argtypes = [I64, I64, I32, U32, PSZ, PSZ, PSZ]
        L.w4a16_repack.argtypes = [P, P, P, I64, I64, I32, U32, P, P, P, P]
        L.w4a16_check_repack_args.argtypes = [P, P, P, I64, I64, I32, U32, P, P, P]
        L.w4a16_dequant.argtypes = [P, P, P, I64, I64, I32, U32, P, P]
        L.w4a16_check_dequant_args.argtypes = [P, P, P, I64, I64, I32, U32, P]
        L.w4a16_quantize.argtypes = [P, I64, I64, I32, U32, P, P, P, P]
        L.w4a16_check_quantize_args.argtypes = [P, I64, I64, I32, U32, P, P, P]
        L.w4a16_gemm_workspace_size.argtypes = [I64, I64, I64, I32, U32, PSZ]
        PI32 = ctypes.POINTER(ctypes.c_int32)
        L.w4a16_gemm_kernel.argtypes = [I64, I64, I64, I32, U32, PI32, PI32]
        L.w4a16_gemm.argtypes = [P, I64, I64, P, P, P, I64, I32, U32, P, P, SZ, P]
        L.w4a16_check_gemm_args.argtypes = [P, I64, I64, P, P, P, I64, I32, U32, P, P, SZ]
        L.w4a16_stream_read.argtypes = [P, SZ, P, SZ, P, SZ, U32, P, P]
        L.w4a16_gemm_noalloc.argtypes = [P, I64, I64, P, P, P, I64, I32, U32, P, P]
        for name in EXPORTS:
            if name not in ("w4a16_status_str", "w4a16_last_hip_error"):
                getattr(L, name).restype = I32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().w4a16_status_str(status).decode()


def _raise(status: int, what: str):
    if status == OK:
        return
    msg = f"{what}: {status_str(status)}"
    if status == ERR_HIP:
        msg += f" [{lib().w4a16_last_hip_error().decode()}]"
    if status in (ERR_HIP, ERR_ARCH):
        raise W4A16Error(status, msg)
    raise W4A16ArgumentError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _need16(t: torch.Tensor, name: str, ndim=None) -> bool:
    """A 16-bit float tensor (fp16 or bf16); returns True for bf16."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16:
        _need(t, name, torch.bfloat16, ndim)
        return True
    _need(t, name, torch.float16, ndim)
    return False


def flags_of(symmetric: bool = False, partial: bool = False) -> int:
    return (SYMMETRIC if symmetric else 0) | (PARTIAL_LAST_GROUP if partial else 0)


def device_check() -> None:
    _raise(lib().w4a16_device_check(), "w4a16_device_check")


def pack(codes: torch.Tensor) -> torch.Tensor:
    """uint8 [R, C] device codes -> int32 [R, ceil(C/8)] packed words."""
    _need(codes, "codes", torch.uint8, 2)
    R, C = codes.shape
    out = torch.empty((R, (C + 7) // 8), dtype=torch.int32, device=codes.device)
    _raise(lib().w4a16_pack(_ptr(codes), R, C, _ptr(out), _stream()), "w4a16_pack")
    return out


@dataclass
class PackedWeight:
    """A weight in the device layout, owned by torch tensors."""
    q: torch.Tensor            # uint8 bytes of q_dev
    s: torch.Tensor            # fp16 s_dev
    z: Optional[torch.Tensor]  # int32 z_dev, None when symmetric
    N: int
    K: int
    g: int
    flags: int

    @property
    def symmetric(self) -> bool:
        return bool(self.flags & SYMMETRIC)


def repack_size(N: int, K: int, g: int, flags: int):
    q, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _raise(lib().w4a16_repack_size(N, K, g, flags, ctypes.byref(q), ctypes.byref(s),
                                   ctypes.byref(z)), "w4a16_repack_size")
    return q.value, s.value, z.value


def repack(qpacked: torch.Tensor, scales: torch.Tensor, zpacked: Optional[torch.Tensor],
           K: int, g: int, symmetric: bool = False, partial: bool = False) -> PackedWeight:
    _need(qpacked, "qpacked", torch.int32, 2)
    bf = _need16(scales, "scales", 2)
    N = qpacked.shape[0]
    G = -(-K // g)
    if qpacked.shape[1] != -(-K // 8) or tuple(scales.shape) != (N, G):
        raise ValueError("qpacked must be [N, K/8] and scales [N, ceil(K/g)]")
    if not symmetric:
        _need(zpacked, "zpacked", torch.int32, 2)
        if tuple(zpacked.shape) != (N, -(-G // 8)):
            raise ValueError("zpacked must be [N, ceil(G/8)]")
    flags = flags_of(symmetric, partial) | (BF16 if bf else 0)
    qb, sb, zb = repack_size(N, K, g, flags)
    dev = qpacked.device
    q = torch.empty(qb, dtype=torch.uint8, device=dev)
    s = torch.empty(sb // 2, dtype=scales.dtype, device=dev)
    z = None if symmetric else torch.empty(zb // 4, dtype=torch.int32, device=dev)
    _raise(lib().w4a16_repack(_ptr(qpacked), _ptr(scales), _ptr(None if symmetric else zpacked),
                              N, K, g, flags, _ptr(q), _ptr(s), _ptr(z), _stream()),
           "w4a16_repack")
    return PackedWeight(q, s, z, N, K, g, flags)


def dequant(qpacked: torch.Tensor, scales: torch.Tensor, zpacked: Optional[torch.Tensor],
            K: int, g: int, symmetric: bool = False, partial: bool = False) -> torch.Tensor:
    _need(qpacked, "qpacked", torch.int32, 2)
    bf = _need16(scales, "scales", 2)
    N = qpacked.shape[0]
    G = -(-K // g)
    if qpacked.shape[1] != -(-K // 8) or tuple(scales.shape) != (N, G):
        raise ValueError("qpacked must be [N, K/8] and scales [N, ceil(K/g)]")
    if not symmetric:
        _need(zpacked, "zpacked", torch.int32, 2)
        if tuple(zpacked.shape) != (N, -(-G // 8)):
            raise ValueError("zpacked must be [N, ceil(G/8)]")
    W = torch.empty((N, K), dtype=scales.dtype, device=qpacked.device)
    flags = flags_of(symmetric, partial) | (BF16 if bf else 0)
    _raise(lib().w4a16_dequant(_ptr(qpacked), _ptr(scales), _ptr(None if symmetric else zpacked),
                               N, K, g, flags, _ptr(W), _stream()),
           "w4a16_dequant")
    return W


def quantize(W: torch.Tensor, g: int, symmetric: bool = False, partial: bool = False,
             out=None):
    """Round-to-nearest group quantization of an fp16 weight W [N, K] on the
    device -> (qpacked int32 [N, K/8], scales fp16 [N, G], zpacked int32
    [N, ceil(G/8)] or None when symmetric), the canonical formats repack()
    takes.  partial: allow K % g != 0 (a partial last group).  out: the three
    output tensors to fill instead of new ones."""
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    G = -(-K // g)
    dev = W.device
    if out is not None:
        qp, sc, zp = out
        _need(qp, "qpacked", torch.int32, 2)
        _need(sc, "scales", torch.float16, 2)
        if tuple(qp.shape) != (N, -(-K // 8)) or tuple(sc.shape) != (N, G):
            raise ValueError("out tensors must be [N, K/8] and [N, ceil(K/g)]")
        if not symmetric:
            _need(zp, "zpacked", torch.int32, 2)
            if tuple(zp.shape) != (N, -(-G // 8)):
                raise ValueError("zpacked out must be [N, ceil(G/8)]")
    else:
        qp = torch.empty((N, -(-K // 8)), dtype=torch.int32, device=dev)
        sc = torch.empty((N, G), dtype=torch.float16, device=dev)
        zp = None if symmetric else torch.empty((N, -(-G // 8)), dtype=torch.int32, device=dev)
    _raise(lib().w4a16_quantize(_ptr(W), N, K, g, flags_of(symmetric, partial), _ptr(qp),
                                _ptr(sc), _ptr(zp), _stream()), "w4a16_quantize")
    return qp, sc, zp


def workspace_size(M: int, N: int, K: int, g: int, flags: int) -> int:
    b = ctypes.c_size_t()
    _raise(lib().w4a16_gemm_workspace_size(M, N, K, g, flags, ctypes.byref(b)),
           "w4a16_gemm_workspace_size")
    return b.value


def gemm_kernel(M: int, N: int, K: int, g: int, flags: int):
    """("small_m" or "large_m", K splits) of the kernel w4a16_gemm runs for
    this problem (pure host)."""
    path, splits = ctypes.c_int32(), ctypes.c_int32()
    _raise(lib().w4a16_gemm_kernel(M, N, K, g, flags, ctypes.byref(path), ctypes.byref(splits)),
           "w4a16_gemm_kernel")
    return ("small_m" if path.value == 0 else "large_m"), splits.value


_workspaces = {}
# Workspaces replaced by larger ones stay allocated: a HIP graph captured
# with an older one still writes to it on every replay.
_retired_workspaces = []


def _cached_workspace(device, nbytes: int) -> torch.Tensor:
    """A workspace of at least nbytes for (device, current stream), kept for
    later calls: w4a16_gemm overwrites the partial sums it reads in the same
    call, and calls on one stream never overlap.  A workspace that is
    outgrown is kept alive (not freed), since graphs captured with it keep
    using it."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired_workspaces.append(ws)
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def new_workspace(device, nbytes: int) -> torch.Tensor:
    """A workspace for callers that manage their own (e.g. to capture calls
    into a HIP graph); calls that may run at the same time need separate ones."""
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def _check_packed(w: PackedWeight) -> None:
    """The device-layout tensors of w hold at least the bytes its shape needs
    (the kernels read them through bare pointers)."""
    qb, sb, zb = repack_size(w.N, w.K, w.g, w.flags & (SYMMETRIC | PARTIAL_LAST_GROUP | BF16))
    _need(w.q, "w.q", torch.uint8)
    _need(w.s, "w.s", torch.bfloat16 if w.flags & BF16 else torch.float16)
    if w.q.numel() < qb or w.s.numel() * 2 < sb:
        raise ValueError("PackedWeight tensors are smaller than its shape needs")
    if not (w.flags & SYMMETRIC):
        _need(w.z, "w.z", torch.int32)
        if w.z.numel() * 4 < zb:
            raise ValueError("PackedWeight zero words are smaller than its shape needs")


def gemm(X: torch.Tensor, w: PackedWeight, path: Optional[str] = None,
         out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [M, N] = X [M, K] . dequant(w)^T, in fp16, or in bf16 when X and the
    weight's scales are bfloat16.

    path: None (chosen by M), "small_m" or "large_m" (forces a kernel)."""
    bf = _need16(X, "X", 2)
    M, K = X.shape
    if K != w.K:
        raise ValueError(f"X has K={K}, the weight K={w.K}")
    if bf != bool(w.flags & BF16):
        raise TypeError("X and the weight's scales must both be fp16 or both bf16")
    flags = w.flags
    if path == "small_m":
        flags |= PATH_SMALL_M
    elif path == "large_m":
        flags |= PATH_LARGE_M
    elif path is not None:
        raise ValueError("path must be None, 'small_m' or 'large_m'")
    _check_packed(w)
    if out is None:
        out = torch.empty((M, w.N), dtype=X.dtype, device=X.device)
    else:
        _need(out, "out", X.dtype, 2)
        if tuple(out.shape) != (M, w.N):
            raise ValueError("out must be [M, N]")
    wsb = workspace_size(M, w.N, K, w.g, flags)
    if wsb and workspace is None:
        workspace = _cached_workspace(X.device, wsb)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _raise(lib().w4a16_gemm(_ptr(X), M, K, _ptr(w.q), _ptr(w.s), _ptr(w.z), w.N, w.g, flags,
                            _ptr(out), _ptr(workspace), ws_bytes, _stream()), "w4a16_gemm")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def gemm_noalloc(X: torch.Tensor, w: PackedWeight, path: Optional[str] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm() through w4a16_gemm_noalloc: the split-K partial sums go to the
    library's static scratch (NOALLOC_SCRATCH_BYTES per GPU) instead of a
    workspace, so the call itself allocates nothing (pass `out` to avoid the
    output allocation here too).  Calls on one GPU share that scratch: calls
    that may overlap must be ordered by the caller."""
    bf = _need16(X, "X", 2)
    M, K = X.shape
    if K != w.K:
        raise ValueError(f"X has K={K}, the weight K={w.K}")
    if bf != bool(w.flags & BF16):
        raise TypeError("X and the weight's scales must both be fp16 or both bf16")
    flags = w.flags
    if path == "small_m":
        flags |= PATH_SMALL_M
    elif path == "large_m":
        flags |= PATH_LARGE_M
    elif path is not None:
        raise ValueError("path must be None, 'small_m' or 'large_m'")
    _check_packed(w)
    if out is None:
        out = torch.empty((M, w.N), dtype=X.dtype, device=X.device)
    else:
        _need(out, "out", X.dtype, 2)
        if tuple(out.shape) != (M, w.N):
            raise ValueError("out must be [M, N]")
    _raise(lib().w4a16_gemm_noalloc(_ptr(X), M, K, _ptr(w.q), _ptr(w.s), _ptr(w.z), w.N, w.g,
                                    flags, _ptr(out), _stream()), "w4a16_gemm_noalloc")
    return out


def stream_read(tensors, sink: torch.Tensor, key: int = 0x9E3779B9) -> None:
    """Measurement only: reads the bytes of up to three device tensors once
    (no arithmetic); sink (int32, >= 1 element) is written only if the xor of
    everything read equals key."""
    if not 1 <= len(tensors) <= 3:
        raise ValueError("one to three tensors")
    _need(sink, "sink", torch.int32)
    args = []
    for t in list(tensors) + [None] * (3 - len(tensors)):
        if t is None:
            args += [None, 0]
        else:
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("stream_read takes contiguous device tensors")
            args += [_ptr(t), t.numel() * t.element_size()]
    _raise(lib().w4a16_stream_read(*args, key, _ptr(sink), _stream()), "w4a16_stream_read")


def quantized_weight(codes: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
                     g: int, partial: bool = False) -> PackedWeight:
    """codes uint8 [N, K], scales fp16 or bf16 [N, G], zeros uint8 [N, G] or None
    (symmetric) -> PackedWeight, all on the device (pack + repack)."""
    K = codes.shape[1]
    qp = pack(codes)
    zp = None if zeros is None else pack(zeros)
    return repack(qp, scales, zp, K, g, symmetric=zeros is None, partial=partial)
