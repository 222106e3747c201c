"""Python binding of libgnf4 (ctypes): argument marshalling only.

Every step of the path runs in the HIP library; this module checks tensor
placement, allocates outputs with torch (device memory is torch's), passes raw
device pointers and torch's current HIP stream, and raises on a non-OK status.
There is no fallback: if the library is missing or a call fails, it raises.

Names follow the C ABI in include/gnf4.h: route, grouped_gemm, combine,
dequant, quantize, nf4_codebook, last_error, build_id.
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgnf4.so")

NF4, NF4_DQ, MXFP4 = 0, 1, 2
FORMATS = {"nf4": NF4, "nf4_dq": NF4_DQ, "mxfp4": MXFP4}
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "DEVICE"}

# Every entry point declared in include/gnf4.h.
EXPORTS = ("gnf4_route", "gnf4_route_workspace_bytes", "gnf4_route_noalloc", "gnf4_route_logits", "gnf4_route_grouped_gemm",
           "gnf4_route_logits_grouped_gemm", "gnf4_grouped_gemm",
           "gnf4_grouped_gemm_swiglu", "gnf4_grouped_gemm_combine",
           "gnf4_grouped_gemm_dx", "gnf4_swiglu", "gnf4_combine",
           "gnf4_dequant", "gnf4_dequant_experts_bf16", "gnf4_quantize", "gnf4_nf4_codebook",
           "gnf4_nf4_codebook_bf16", "gnf4_read_probe",
           "gnf4_expert_cache_state_words", "gnf4_expert_cache_copies_words",
           "gnf4_expert_cache_reset", "gnf4_expert_cache_stage", "gnf4_expert_cache_fill",
           "gnf4_last_error",
           "gnf4_build_id")


class Gnf4Error(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed with %s: %s" % (what, STATUS.get(status, status), last_error()))
        self.status = status


class CWeights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("scales2", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libgnf4.so (built in-tree by bit_mixture_experts_topk_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgnf4.so is not built; run `python -m bit_mixture_experts_topk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
        Z = ctypes.c_size_t
        L.gnf4_route_workspace_bytes.argtypes = [I, I, I]
        L.gnf4_route_workspace_bytes.restype = Z
        L.gnf4_route.argtypes = [P, I, I, I, P, P, P, P, P, P, P, P, Z, S]
        L.gnf4_route_logits.argtypes = [P, I, I, I, P, P, P, P, P, P, P, P, P, P, Z, S]
        L.gnf4_route_noalloc.argtypes = [P, I, I, I, P, P, P, P, P, P, P, S]
        L.gnf4_swiglu.argtypes = [P, I, I, P, S]
        L.gnf4_grouped_gemm.argtypes = [ctypes.POINTER(CWeights), P, I, P, P, P, P, I, I, P, S]
        L.gnf4_grouped_gemm_swiglu.argtypes = [ctypes.POINTER(CWeights), P, I, P, P, P, P, I, I, P, S]
        L.gnf4_route_grouped_gemm.argtypes = [P, I, I, P, P, P, P, P, P, P, P, Z,
                                              ctypes.POINTER(CWeights), P, P, P, S]
        L.gnf4_grouped_gemm_combine.argtypes = [ctypes.POINTER(CWeights), P, P, P, P, P, P, P, I, I,
                                                P, P, S]
        L.gnf4_route_logits_grouped_gemm.argtypes = [P, I, I, P, P, P, P, P, P, P, P, P, P, Z,
                                                     ctypes.POINTER(CWeights), P, P, P, S]
        L.gnf4_grouped_gemm_dx.argtypes = [ctypes.POINTER(CWeights), P, P, I, I, P, S]
        L.gnf4_combine.argtypes = [P, P, P, I, I, I, P, S]
        L.gnf4_dequant.argtypes = [ctypes.POINTER(CWeights), I, P, S]
        L.gnf4_dequant_experts_bf16.argtypes = [ctypes.POINTER(CWeights), P, P, I, P, S]
        L.gnf4_quantize.argtypes = [I, P, I, I, P, P, P, S]
        L.gnf4_expert_cache_state_words.argtypes = [I, I]
        L.gnf4_expert_cache_state_words.restype = ctypes.c_size_t
        L.gnf4_expert_cache_copies_words.argtypes = [I, I, I, I]
        L.gnf4_expert_cache_copies_words.restype = ctypes.c_size_t
        L.gnf4_expert_cache_reset.argtypes = [P, I, I, S]
        L.gnf4_expert_cache_stage.argtypes = [P, I, I, I, I, P, P, P, S]
        L.gnf4_expert_cache_fill.argtypes = [ctypes.POINTER(CWeights), ctypes.POINTER(CWeights), P, I, S]
        L.gnf4_nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
        L.gnf4_nf4_codebook.restype = None
        L.gnf4_nf4_codebook_bf16.argtypes = [ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_float)]
        L.gnf4_nf4_codebook_bf16.restype = None
        L.gnf4_read_probe.argtypes = [P, ctypes.c_size_t, I, P, S]
        L.gnf4_last_error.restype = ctypes.c_char_p
        L.gnf4_build_id.restype = ctypes.c_char_p
        for name in ("gnf4_route", "gnf4_grouped_gemm", "gnf4_combine", "gnf4_dequant", "gnf4_quantize"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def last_error():
    return lib().gnf4_last_error().decode()


def build_id():
    return lib().gnf4_build_id().decode()


def nf4_codebook():
    buf = (ctypes.c_float * 16)()
    lib().gnf4_nf4_codebook(buf)
    return [buf[i] for i in range(16)]


def nf4_codebook_bf16():
    """(bf16 bits of the 16 NF4 operand values, their scale s): the values
    are bf16(s * c[q]) and the kernels scale partial sums by absmax / s."""
    buf = (ctypes.c_uint16 * 16)()
    sc = ctypes.c_float()
    lib().gnf4_nf4_codebook_bf16(buf, ctypes.byref(sc))
    return [buf[i] for i in range(16)], sc.value


def _check(status, what):
    if status != 0:
        raise Gnf4Error(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))
    return t


@dataclass
class PackedWeights:
    """Packed experts of one projection: W [E, N, K] in a 4-bit format."""
    format: int
    E: int
    N: int
    K: int
    codes: torch.Tensor                  # uint8 [E, N, K/2]
    scales: torch.Tensor                 # float32 / int8 / uint8 per format
    scales2: Optional[torch.Tensor] = None

    def cstruct(self):
        return CWeights(self.format, self.E, self.N, self.K, self.codes.data_ptr(),
                        self.scales.data_ptr(),
                        self.scales2.data_ptr() if self.scales2 is not None else None)

    def nbytes(self):
        n = self.codes.numel() + self.scales.numel() * self.scales.element_size()
        if self.scales2 is not None:
            n += self.scales2.numel() * 4
        return n


def empty_packed(fmt, E, N, K, device="cuda", pin_memory=False):
    """Uninitialised packed weights; device="cpu", pin_memory=True gives pinned
    host memory (the host side of the expert streaming cache)."""
    fmt = FORMATS.get(fmt, fmt)
    kw = dict(device=device, pin_memory=pin_memory)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, **kw)
    scales2 = None
    if fmt == MXFP4:
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, **kw)
    elif fmt == NF4:
        scales = torch.empty((E, N, K // 64), dtype=torch.float32, **kw)
    else:
        scales = torch.empty((E, N, K // 64), dtype=torch.int8, **kw)
        nb = E * N * (K // 64)
        scales2 = torch.empty(((nb + 255) // 256,), dtype=torch.float32, **kw)
    return PackedWeights(fmt, E, N, K, codes, scales, scales2)


def quantize(fmt, W, out=None):
    """Pack float32 W [E, N, K] (CUDA) with gnf4_quantize."""
    fmt = FORMATS.get(fmt, fmt)
    _dev(W, torch.float32, "W")
    E, N, K = W.shape
    pw = out if out is not None else empty_packed(fmt, E, N, K, W.device)
    _check(lib().gnf4_quantize(fmt, _ptr(W), E * N, K, _ptr(pw.codes), _ptr(pw.scales),
                               _ptr(pw.scales2), _stream()), "gnf4_quantize")
    return pw


def quantize_into(fmt, W, pw, e0):
    """Pack float32 W [n, N, K] into experts [e0, e0 + n) of pw."""
    fmt = FORMATS.get(fmt, fmt)
    _dev(W, torch.float32, "W")
    n, N, K = W.shape
    if fmt == NF4_DQ:
        raise ValueError("NF4_DQ groups span experts; quantize the whole layer at once")
    codes = pw.codes[e0:e0 + n]
    scales = pw.scales[e0:e0 + n]
    _check(lib().gnf4_quantize(fmt, _ptr(W), n * N, K, _ptr(codes), _ptr(scales), None, _stream()),
           "gnf4_quantize")


def route_workspace_bytes(T, k, E):
    return int(lib().gnf4_route_workspace_bytes(T, k, E))


def route_buffers(T, k, E, device="cuda"):
    """Output buffers for route(): counts, offsets, perm, inv, active,
    n_active, bad, and the route's workspace (empty when none is needed)."""
    i32 = dict(dtype=torch.int32, device=device)
    ws = route_workspace_bytes(T, k, E)
    return {"counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
            "perm": torch.empty(max(T * k, 1), **i32), "inv": torch.empty(max(T * k, 1), **i32),
            "active": torch.empty(E, **i32), "n_active": torch.empty(1, **i32),
            "bad": torch.empty(1, **i32),
            "workspace": torch.empty(max(ws, 16), dtype=torch.uint8, device=device)}


def _ws(r):
    """(pointer, bytes) of a route dict's workspace."""
    w = r.get("workspace")
    return (None, 0) if w is None else (_ptr(w), w.numel())


def route(topk_ids, E, out=None):
    """Route int32 topk_ids [T, k] (CUDA) over E experts; returns a dict of tensors."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    r = dict(out) if out is not None else route_buffers(T, k, E, topk_ids.device)
    _check(lib().gnf4_route(_ptr(topk_ids), T, k, E, _ptr(r["counts"]), _ptr(r["offsets"]),
                            _ptr(r["perm"]), _ptr(r["inv"]), _ptr(r["active"]),
                            _ptr(r["n_active"]), _ptr(r["bad"]), *_ws(r), _stream()), "gnf4_route")
    r["perm"] = r["perm"][:T * k]
    r["inv"] = r["inv"][:T * k]
    return r


def route_noalloc(topk_ids, E, out=None):
    """route() through gnf4_route_noalloc: the library's static workspace,
    no workspace argument (out's "workspace" entry, if any, is not used)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    r = dict(out) if out is not None else route_buffers(T, k, E, topk_ids.device)
    _check(lib().gnf4_route_noalloc(_ptr(topk_ids), T, k, E, _ptr(r["counts"]), _ptr(r["offsets"]),
                                    _ptr(r["perm"]), _ptr(r["inv"]), _ptr(r["active"]),
                                    _ptr(r["n_active"]), _ptr(r["bad"]), _stream()),
           "gnf4_route_noalloc")
    r["perm"] = r["perm"][:T * k]
    r["inv"] = r["inv"][:T * k]
    return r


def route_grouped_gemm(topk_ids, w, X, out=None, Y=None, H=None, swiglu=False):
    """route() then grouped_gemm(gather=1) (or grouped_gemm_swiglu when
    swiglu), one launch for a single token; returns (route dict, Y or H)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    if not (X.is_cuda and X.is_contiguous() and X.element_size() == 2):
        raise ValueError("X must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    T, k = topk_ids.shape
    r = dict(out) if out is not None else route_buffers(T, k, w.E, topk_ids.device)
    if swiglu:
        if H is None:
            H = torch.empty((max(T * k, 1), w.N // 2), dtype=torch.int16, device=X.device)
        res = H
    else:
        if Y is None:
            Y = torch.empty((max(T * k, 1), w.N), dtype=torch.float32, device=X.device)
        res = Y
    cw = w.cstruct()
    _check(lib().gnf4_route_grouped_gemm(_ptr(topk_ids), T, k, _ptr(r["counts"]), _ptr(r["offsets"]),
                                         _ptr(r["perm"]), _ptr(r["inv"]), _ptr(r["active"]),
                                         _ptr(r["n_active"]), _ptr(r["bad"]), *_ws(r), ctypes.byref(cw),
                                         _ptr(X), None if swiglu else _ptr(Y),
                                         _ptr(H) if swiglu else None, _stream()),
           "gnf4_route_grouped_gemm")
    r["perm"] = r["perm"][:T * k]
    r["inv"] = r["inv"][:T * k]
    return r, res


def route_logits_grouped_gemm(logits, k, w, X, out=None, Y=None, H=None, swiglu=False):
    """route_logits() then grouped_gemm(gather=1) (or grouped_gemm_swiglu),
    one launch for a single token; returns (route dict with topk_ids and
    topk_w, Y or H)."""
    _dev(logits, torch.float32, "logits")
    if not (X.is_cuda and X.is_contiguous() and X.element_size() == 2):
        raise ValueError("X must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    T, E = logits.shape
    r = dict(out) if out is not None else route_buffers(T, k, E, logits.device)
    if "topk_ids" not in r:
        r["topk_ids"] = torch.empty((max(T, 1), k), dtype=torch.int32, device=logits.device)
        r["topk_w"] = torch.empty((max(T, 1), k), dtype=torch.float32, device=logits.device)
    if swiglu:
        if H is None:
            H = torch.empty((max(T * k, 1), w.N // 2), dtype=torch.int16, device=X.device)
        res = H
    else:
        if Y is None:
            Y = torch.empty((max(T * k, 1), w.N), dtype=torch.float32, device=X.device)
        res = Y
    cw = w.cstruct()
    _check(lib().gnf4_route_logits_grouped_gemm(
        _ptr(logits), T, k, _ptr(r["topk_ids"]), _ptr(r["topk_w"]), _ptr(r["counts"]),
        _ptr(r["offsets"]), _ptr(r["perm"]), _ptr(r["inv"]), _ptr(r["active"]), _ptr(r["n_active"]),
        _ptr(r["bad"]), *_ws(r), ctypes.byref(cw), _ptr(X), None if swiglu else _ptr(Y),
        _ptr(H) if swiglu else None, _stream()), "gnf4_route_logits_grouped_gemm")
    r["perm"] = r["perm"][:T * k]
    r["inv"] = r["inv"][:T * k]
    r["topk_ids"] = r["topk_ids"][:T]
    r["topk_w"] = r["topk_w"][:T]
    return r, res


def route_logits(logits, k, out=None):
    """Top-k of float32 router logits [T, E] (CUDA) with softmax weights, then
    route; returns the route dict plus "topk_ids" [T, k] and "topk_w" [T, k]."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    r = dict(out) if out is not None else route_buffers(T, k, E, logits.device)
    if "topk_ids" not in r:
        r["topk_ids"] = torch.empty((max(T, 1), k), dtype=torch.int32, device=logits.device)
        r["topk_w"] = torch.empty((max(T, 1), k), dtype=torch.float32, device=logits.device)
    _check(lib().gnf4_route_logits(_ptr(logits), T, k, E, _ptr(r["topk_ids"]), _ptr(r["topk_w"]),
                                   _ptr(r["counts"]), _ptr(r["offsets"]), _ptr(r["perm"]),
                                   _ptr(r["inv"]), _ptr(r["active"]), _ptr(r["n_active"]),
                                   _ptr(r["bad"]), *_ws(r), _stream()), "gnf4_route_logits")
    r["perm"] = r["perm"][:T * k]
    r["inv"] = r["inv"][:T * k]
    r["topk_ids"] = r["topk_ids"][:T]
    r["topk_w"] = r["topk_w"][:T]
    return r


def swiglu(Y, I, H=None):
    """H [rows, I] bf16 bits (int16) = bf16(silu(Y[:, :I]) * Y[:, I:2I])."""
    _dev(Y, torch.float32, "Y")
    rows = Y.shape[0]
    if Y.shape[1] != 2 * I:
        raise ValueError("Y must have 2*I columns")
    if H is None:
        H = torch.empty((max(rows, 1), I), dtype=torch.int16, device=Y.device)
    _check(lib().gnf4_swiglu(_ptr(Y), rows, I, _ptr(H), _stream()), "gnf4_swiglu")
    return H


def grouped_gemm(w, X, gather, r, T, k, Y=None):
    """Y [T*k, N] float32 = grouped GEMM of bf16 X over the routed rows."""
    if not (X.is_cuda and X.is_contiguous() and X.element_size() == 2):
        raise ValueError("X must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    if Y is None:
        Y = torch.empty((max(T * k, 1), w.N), dtype=torch.float32, device=X.device)
    cw = w.cstruct()
    _check(lib().gnf4_grouped_gemm(ctypes.byref(cw), _ptr(X), gather, _ptr(r["offsets"]),
                                   _ptr(r["perm"]), _ptr(r["active"]), _ptr(r["n_active"]),
                                   T, k, _ptr(Y), _stream()), "gnf4_grouped_gemm")
    return Y


def grouped_gemm_swiglu(w, X, gather, r, T, k, H=None):
    """H [T*k, N/2] bf16 bits (int16) = SwiGLU of the grouped GEMM, fused."""
    if not (X.is_cuda and X.is_contiguous() and X.element_size() == 2):
        raise ValueError("X must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    if H is None:
        H = torch.empty((max(T * k, 1), w.N // 2), dtype=torch.int16, device=X.device)
    cw = w.cstruct()
    _check(lib().gnf4_grouped_gemm_swiglu(ctypes.byref(cw), _ptr(X), gather, _ptr(r["offsets"]),
                                          _ptr(r["perm"]), _ptr(r["active"]), _ptr(r["n_active"]),
                                          T, k, _ptr(H), _stream()), "gnf4_grouped_gemm_swiglu")
    return H


def grouped_gemm_combine(w, X, r, topk_w, T, k, out=None, Y=None):
    """grouped_gemm(gather=0) then combine: out [T, N] float32; one launch for
    a single token. Y is the [T*k, N] intermediate of the two-launch path
    (allocated here when needed)."""
    if not (X.is_cuda and X.is_contiguous() and X.element_size() == 2):
        raise ValueError("X must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    _dev(topk_w, torch.float32, "topk_w")
    if out is None:
        out = torch.empty((max(T, 1), w.N), dtype=torch.float32, device=X.device)
    if Y is None and not (T == 1 and w.K <= 8192):
        Y = torch.empty((max(T * k, 1), w.N), dtype=torch.float32, device=X.device)
    cw = w.cstruct()
    _check(lib().gnf4_grouped_gemm_combine(ctypes.byref(cw), _ptr(X), _ptr(r["offsets"]), _ptr(r["perm"]),
                                           _ptr(r["inv"]), _ptr(r["active"]), _ptr(r["n_active"]),
                                           _ptr(topk_w), T, k, _ptr(Y), _ptr(out), _stream()),
           "gnf4_grouped_gemm_combine")
    return out


def grouped_gemm_dx(w, dY, r, T, k, dA=None):
    """dA [T*k, K] float32 = dY [T*k, N] (bf16 bits, routed order) times the
    dequantized weights of each row's expert: the input gradient of
    grouped_gemm with frozen weights. Rows past the routed ones are left as
    they are (uninitialised when dA is allocated here)."""
    if not (dY.is_cuda and dY.is_contiguous() and dY.element_size() == 2):
        raise ValueError("dY must be a contiguous bf16 (or 16-bit bit pattern) CUDA tensor")
    if dA is None:
        dA = torch.empty((max(T * k, 1), w.K), dtype=torch.float32, device=dY.device)
    cw = w.cstruct()
    _check(lib().gnf4_grouped_gemm_dx(ctypes.byref(cw), _ptr(dY), _ptr(r["offsets"]), T, k,
                                      _ptr(dA), _stream()), "gnf4_grouped_gemm_dx")
    return dA


def token_grad(dA, r, T, k, out=None):
    """dX [T, K] float32: the sum of each token's k routed copies of dA (the
    gradient through the gather of a first projection), via gnf4_combine
    with unit weights."""
    ones = torch.ones((max(T, 1), k), dtype=torch.float32, device=dA.device)
    return combine(dA, r["inv"], ones, T, k, out=out)


def combine(Y, inv, topk_w, T, k, out=None):
    _dev(Y, torch.float32, "Y")
    _dev(topk_w, torch.float32, "topk_w")
    N = Y.shape[1]
    if out is None:
        out = torch.empty((max(T, 1), N), dtype=torch.float32, device=Y.device)
    _check(lib().gnf4_combine(_ptr(Y), _ptr(inv), _ptr(topk_w), T, k, N, _ptr(out), _stream()),
           "gnf4_combine")
    return out


def dequant_experts_bf16(w, experts, count, max_experts, out=None):
    """bf16 bits (int16) [max_experts, N, K] of the listed experts (device
    int32 experts[], count[1]); slots past *count are left untouched."""
    _dev(experts, torch.int32, "experts")
    _dev(count, torch.int32, "count")
    if out is None:
        out = torch.zeros((max(max_experts, 1), w.N, w.K), dtype=torch.int16, device=w.codes.device)
    cw = w.cstruct()
    _check(lib().gnf4_dequant_experts_bf16(ctypes.byref(cw), _ptr(experts), _ptr(count), max_experts,
                                           _ptr(out), _stream()), "gnf4_dequant_experts_bf16")
    return out


def read_probe(buf, nbytes=None, workgroups=0, sink=None):
    """Read nbytes (default: all) of the CUDA tensor buf once (the achievable
    HBM read rate; over more than 256 MB it also evicts the Infinity Cache)."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous CUDA tensor")
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    _check(lib().gnf4_read_probe(_ptr(buf), n, workgroups, _ptr(sink), _stream()), "gnf4_read_probe")
    return sink


def dequant(w, e):
    out = torch.empty((w.N, w.K), dtype=torch.float32, device=w.codes.device)
    cw = w.cstruct()
    _check(lib().gnf4_dequant(ctypes.byref(cw), e, _ptr(out), _stream()), "gnf4_dequant")
    return out


# ------------------------------------------------ expert streaming cache

def expert_cache_state(E, S):
    """A reset residency state for S slots over E experts (device int32)."""
    n = lib().gnf4_expert_cache_state_words(E, S)
    if n == 0:
        raise ValueError("invalid cache shape E=%d S=%d" % (E, S))
    state = torch.empty((n,), dtype=torch.int32, device="cuda")
    expert_cache_reset(state, E, S)
    return state


def expert_cache_reset(state, E, S):
    _dev(state, torch.int32, "state")
    _check(lib().gnf4_expert_cache_reset(_ptr(state), E, S, _stream()), "gnf4_expert_cache_reset")


def expert_cache_copies_words(T, k, E, S):
    return int(lib().gnf4_expert_cache_copies_words(T, k, E, S))


def expert_cache_stage(topk_ids, E, S, state, slot_ids=None, copies=None):
    """Residency decision for int32 topk_ids [T, k]: (slot_ids [T, k], copies)."""
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(state, torch.int32, "state")
    T, k = topk_ids.shape
    if slot_ids is None:
        slot_ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    if copies is None:
        copies = torch.empty((max(expert_cache_copies_words(T, k, E, S), 1),), dtype=torch.int32,
                             device="cuda")
    _check(lib().gnf4_expert_cache_stage(_ptr(topk_ids), T, k, E, S, _ptr(state), _ptr(slot_ids),
                                         _ptr(copies), _stream()), "gnf4_expert_cache_stage")
    return slot_ids, copies


def expert_cache_fill(host_w, cache_w, copies, max_copies):
    """Copy the listed experts of host_w (pinned host memory) into cache_w."""
    _dev(copies, torch.int32, "copies")
    hw, cw = host_w.cstruct(), cache_w.cstruct()
    _check(lib().gnf4_expert_cache_fill(ctypes.byref(hw), ctypes.byref(cw), _ptr(copies), max_copies,
                                        _stream()), "gnf4_expert_cache_fill")
