"""Thin ctypes binding of libgdr.so (C ABI in include/gdr.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels of libgdr.so.  PyTorch provides device memory and the stream.  There
is no fallback: if the library is missing or cannot be loaded, every call
raises.

Entry points (same names as the C ABI):
  gdr_chunk_fwd_workspace_size(desc) -> bytes
  gdr_chunk_fwd_segment_chunks(desc) -> chunks per stream in one segment
  gdr_chunk_fwd(q, k, v, log_alpha, b, w, gamma=None, z=None, S0=None, ...)
      -> (o, S_T)
  gdr_chunk_fwd_gated(q, k, v, log_alpha, b, w, g, ...) -> (y, S_T)
  ChunkCall(...) and its .intra() / .scan(): gdr_chunk_fwd_intra / _scan
  ChunkCall(...).static(): gdr_chunk_fwd_static (no workspace, no allocation)
  gdr_chunk_fwd_varlen_workspace_size(desc, n_seqs) -> bytes
  gdr_chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, ...) -> (o, S_T)
  gdr_decode_step(S, q, k, v, log_alpha, b, w, gamma=None, z=None, ...) -> o
  gdr_status_string(code) -> str
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_WORKSPACE, GDR_ERR_HIP = range(5)
GDR_BF16, GDR_F32 = 0, 1
PER_CHANNEL, PER_TOKEN, ONES, ZEROS = 0, 1, 2, 3
SYMBOLS = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_chunk_fwd_gated", "gdr_chunk_fwd_intra",
           "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd", "gdr_chunk_bwd_varlen_workspace_size",
           "gdr_chunk_bwd_varlen", "gdr_output_gate_bwd_workspace_size", "gdr_output_gate_bwd",
           "gdr_chunk_fwd_scan", "gdr_chunk_fwd_varlen_workspace_size", "gdr_chunk_fwd_varlen",
           "gdr_decode_step", "gdr_status_string", "gdr_version", "gdr_gate_proj_workspace_size",
           "gdr_gate_proj", "gdr_chunk_fwd_static", "gdr_chunk_fwd_segment_chunks", "gdr_check_inputs")
# counters of gdr_check_inputs, in order
CHECK_NAMES = ("q", "k", "v", "log_alpha", "b", "w", "z", "gamma")


class GdrDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("chunk", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("normalize_qk", ctypes.c_int), ("scale", ctypes.c_float),
                ("alpha_mode", ctypes.c_int), ("b_mode", ctypes.c_int),
                ("w_mode", ctypes.c_int)]


class GdrGateDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("d_model", ctypes.c_int),
                ("H", ctypes.c_int), ("d", ctypes.c_int), ("rank", ctypes.c_int * 5),
                ("out_dtype", ctypes.c_int)]


class GdrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {gdr_status_string(code)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdr.so; raise (never fall back) if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m channel_wise_gated_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(GdrDesc)
    lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_fwd_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdr_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdr_chunk_fwd_gated.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                        vp, vp, vp, sz, vp]
    lib.gdr_chunk_fwd_segment_chunks.restype = ctypes.c_int
    lib.gdr_chunk_fwd_segment_chunks.argtypes = [dp, ctypes.POINTER(ctypes.c_int)]
    lib.gdr_chunk_fwd_static.restype = ctypes.c_int
    lib.gdr_chunk_fwd_static.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdr_chunk_fwd_intra.restype = ctypes.c_int
    lib.gdr_chunk_fwd_intra.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdr_chunk_fwd_scan.restype = ctypes.c_int
    lib.gdr_chunk_fwd_scan.argtypes = [dp, vp, vp, vp, vp, sz, vp]
    lib.gdr_chunk_fwd_varlen_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_fwd_varlen_workspace_size.argtypes = [dp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.gdr_chunk_fwd_varlen.restype = ctypes.c_int
    lib.gdr_chunk_fwd_varlen.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, sz, vp]
    lib.gdr_decode_step.restype = ctypes.c_int
    lib.gdr_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    gp = ctypes.POINTER(GdrGateDesc)
    lib.gdr_gate_proj_workspace_size.restype = ctypes.c_int
    lib.gdr_gate_proj_workspace_size.argtypes = [gp, ctypes.POINTER(sz)]
    lib.gdr_gate_proj.restype = ctypes.c_int
    lib.gdr_gate_proj.argtypes = [gp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_bwd_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [dp] + [vp] * 21 + [sz, vp]
    lib.gdr_chunk_bwd_varlen_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_bwd_varlen_workspace_size.argtypes = [dp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.gdr_chunk_bwd_varlen.restype = ctypes.c_int
    lib.gdr_chunk_bwd_varlen.argtypes = [dp, ctypes.c_int, vp] + [vp] * 21 + [sz, vp]
    lib.gdr_output_gate_bwd_workspace_size.restype = ctypes.c_int
    lib.gdr_output_gate_bwd_workspace_size.argtypes = [dp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.gdr_output_gate_bwd.restype = ctypes.c_int
    lib.gdr_output_gate_bwd.argtypes = [dp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.gdr_check_inputs.restype = ctypes.c_int
    lib.gdr_check_inputs.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_version.restype = ctypes.c_int
    lib.gdr_version.argtypes = []
    _lib = lib
    return lib


def gdr_status_string(code: int) -> str:
    return load().gdr_status_string(int(code)).decode()


def make_desc(B, H, T, dk, dv, chunk=64, in_dtype=GDR_BF16, out_dtype=GDR_F32,
              normalize_qk=1, scale=1.0, alpha_mode=PER_CHANNEL, b_mode=PER_CHANNEL,
              w_mode=PER_CHANNEL) -> GdrDesc:
    return GdrDesc(int(B), int(H), int(T), int(dk), int(dv), int(chunk), int(in_dtype),
                   int(out_dtype), int(normalize_qk), float(scale), int(alpha_mode),
                   int(b_mode), int(w_mode))


def gdr_chunk_fwd_workspace_size(desc: GdrDesc) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_workspace_size")
    return int(n.value)


def gdr_chunk_fwd_segment_chunks(desc: GdrDesc) -> int:
    """Chunks per stream in one segment of gdr_chunk_fwd (see gdr.h)."""
    n = ctypes.c_int(0)
    rc = load().gdr_chunk_fwd_segment_chunks(ctypes.byref(desc), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_segment_chunks")
    return int(n.value)


# ----------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gate(g, full_ndim: int, name: str):
    """(mode, tensor-or-None) from a gate argument: tensor with the full rank
    (per channel), one dim less (per token), or the scalar 1 / 0 / None."""
    if g is None:
        return ONES, None
    if isinstance(g, (int, float)):
        if g == 1:
            return ONES, None
        if g == 0:
            return ZEROS, None
        raise ValueError(f"{name}: scalar gates must be 0 or 1")
    if g.dim() == full_ndim:
        return PER_CHANNEL, g
    if g.dim() == full_ndim - 1:
        return PER_TOKEN, g
    raise ValueError(f"{name}: rank {g.dim()} does not fit")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _contig(t):
    if t is None or isinstance(t, (int, float)):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t


# ----------------------------------------------------------------- validation
# Every tensor argument is checked before anything is launched: its shape
# against the call's sizes, its dtype against what the kernels read it as,
# its layout, and its device.  The C ABI checks pointers, sizes and
# alignment, but a pointer carries neither a dtype nor an extent.
_FLOAT = (torch.bfloat16, torch.float32)
_F32 = (torch.float32,)


def _req(t, name, shape, dtypes):
    """A required tensor argument: exact shape, one of `dtypes`, contiguous."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtypes):
    """An optional tensor argument (None passes)."""
    return None if t is None else _req(t, name, shape, dtypes)


def _rank(t, name, ndim):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{name} must be a {ndim}-d tensor")
    return t


def _gate_arg(g, name, full_shape, dtypes):
    """(mode, tensor) of a gate given per channel (full_shape), per token
    (full_shape without its last dim) or as the scalar 1 / 0 / None."""
    mode, t = _gate(g, len(full_shape), name)
    if t is not None:
        _req(t, name, full_shape if mode == PER_CHANNEL else full_shape[:-1], dtypes)
    return mode, t


def _log_alpha_arg(la, full_shape):
    if isinstance(la, (int, float)):
        if la != 0:
            raise ValueError("scalar log_alpha must be 0")
        return ONES, None
    if la is None:
        raise ValueError("log_alpha must be a tensor or 0")
    return _gate_arg(la, "log_alpha", full_shape, _F32)


def _same_device(ref, named):
    """Every tensor on the GPU device of `ref`."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, not {ref.device}")
    for name, t in named.items():
        if isinstance(t, torch.Tensor) and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _workspace_arg(ws, need, device):
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws


def _cu_seqlens_arg(cu, T):
    if not isinstance(cu, torch.Tensor) or cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 offsets")
    if not cu.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    return cu


class ChunkCall:
    """Marshalled arguments of one chunkwise forward (pointers, descriptor,
    outputs and workspace), so that the call -- or either of its two phases --
    can be issued repeatedly without re-marshalling."""

    def __init__(self, q, k, v, log_alpha, b, w, gamma=None, z=None, S0=None, *, chunk=64,
                 out_dtype=torch.float32, normalize_qk=True, scale=1.0, o=None, S_T=None,
                 workspace=None, _gated=False):
        B, H, T, dk = _rank(q, "q", 4).shape
        dv = _rank(v, "v", 4).shape[-1]
        dt = (_req(q, "q", (B, H, T, dk), _FLOAT).dtype,)
        _req(k, "k", (B, H, T, dk), dt)
        _req(v, "v", (B, H, T, dv), dt)
        amode, la = _log_alpha_arg(log_alpha, (B, H, T, dk))
        bmode, bt = _gate_arg(b, "b", (B, H, T, dk), dt)
        wmode, wt = _gate_arg(w, "w", (B, H, T, dv), dt)
        _opt(gamma, "gamma", (H, dk), _F32)
        _opt(z, "z", (B, H, T, dk), dt)
        _opt(S0, "S0", (B, H, dk, dv), _F32)
        if out_dtype not in _FLOAT:
            raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
        if not _gated:
            _opt(o, "o", (B, H, T, dv), (out_dtype,))
        _opt(S_T, "S_T", (B, H, dk, dv), _F32)
        od = GDR_BF16 if out_dtype == torch.bfloat16 else GDR_F32
        self.desc = make_desc(B, H, T, dk, dv, chunk, _dtype_code(q), od, int(bool(normalize_qk)),
                              scale, amode, bmode, wmode)
        need = gdr_chunk_fwd_workspace_size(self.desc)
        if workspace is not None:
            _workspace_arg(workspace, need, q.device)
        _same_device(q, dict(k=k, v=v, log_alpha=la, b=bt, w=wt, gamma=gamma, z=z, S0=S0, o=o, S_T=S_T,
                             workspace=workspace))
        if o is None:
            o = torch.empty((B, H, T, dv), dtype=out_dtype, device=q.device)
        if S_T is None:
            S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
        workspace = _workspace_arg(workspace, need, q.device)
        self.o, self.S_T, self.workspace = o, S_T, workspace
        self._keep = (q, k, v, la, bt, wt, gamma, z, S0)   # keep the inputs alive
        self.ptrs = [_ptr(t) for t in self._keep]
        self.out_ptrs = (_ptr(S0), _ptr(o), _ptr(S_T))
        self.ws = (_ptr(workspace), workspace.numel())

    def __call__(self, stream=None):
        """gdr_chunk_fwd: both phases."""
        S0p, op, sTp = self.out_ptrs
        rc = load().gdr_chunk_fwd(ctypes.byref(self.desc), *self.ptrs[:8], S0p, op, sTp,
                                  *self.ws, _stream(stream))
        if rc != GDR_OK:
            raise GdrError(rc, "gdr_chunk_fwd")
        return self.o, self.S_T

    def static(self, stream=None):
        """gdr_chunk_fwd_static: the whole call with the library's static
        scratch instead of the workspace (no device allocation)."""
        S0p, op, sTp = self.out_ptrs
        rc = load().gdr_chunk_fwd_static(ctypes.byref(self.desc), *self.ptrs[:8], S0p, op, sTp, _stream(stream))
        if rc != GDR_OK:
            raise GdrError(rc, "gdr_chunk_fwd_static")
        return self.o, self.S_T

    def intra(self, stream=None):
        """gdr_chunk_fwd_intra: token inputs -> per-chunk maps in the workspace."""
        rc = load().gdr_chunk_fwd_intra(ctypes.byref(self.desc), *self.ptrs[:8], *self.ws,
                                        _stream(stream))
        if rc != GDR_OK:
            raise GdrError(rc, "gdr_chunk_fwd_intra")

    def scan(self, stream=None):
        """gdr_chunk_fwd_scan: workspace and S0 -> o and S_T."""
        S0p, op, sTp = self.out_ptrs
        rc = load().gdr_chunk_fwd_scan(ctypes.byref(self.desc), S0p, op, sTp, *self.ws,
                                       _stream(stream))
        if rc != GDR_OK:
            raise GdrError(rc, "gdr_chunk_fwd_scan")
        return self.o, self.S_T


def gdr_chunk_fwd(q, k, v, log_alpha, b, w, gamma=None, z=None, S0=None, *, chunk=64,
                  out_dtype=torch.float32, normalize_qk=True, scale=1.0, o=None, S_T=None,
                  workspace=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunkwise forward over whole sequences; see gdr_chunk_fwd in gdr.h.

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (bf16 or fp32, same dtype); log_alpha: fp32
    [B,H,T,dk] or [B,H,T] or 0; b, w: per channel, per token or the scalars
    1 / 0; gamma [H,dk] fp32; z [B,H,T,dk]; S0 [B,H,dk,dv] fp32.
    Returns (o [B,H,T,dv] out_dtype, S_T [B,H,dk,dv] fp32).
    """
    load()
    call = ChunkCall(q, k, v, log_alpha, b, w, gamma, z, S0, chunk=chunk, out_dtype=out_dtype,
                     normalize_qk=normalize_qk, scale=scale, o=o, S_T=S_T, workspace=workspace)
    return call(stream)


def gdr_chunk_fwd_gated(q, k, v, log_alpha, b, w, g, gamma=None, z=None, S0=None, norm_weight=None,
                        eps=1e-6, *, chunk=64, out_dtype=torch.float32, normalize_qk=True, scale=1.0,
                        y=None, S_T=None, workspace=None, stream=None, o=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunkwise forward with the fused output gate; see gdr_chunk_fwd_gated in gdr.h.

    Arguments as gdr_chunk_fwd, plus g [B,H,T,dv] (input dtype), norm_weight
    [H,dv] fp32 or None, eps.  Returns (y [B,T,H,dv] out_dtype, S_T).  With
    `o` (an fp32 [B,H,T,dv] tensor) o itself is written there as well.
    """
    lib = load()
    call = ChunkCall(q, k, v, log_alpha, b, w, gamma, z, S0, chunk=chunk, out_dtype=out_dtype,
                     normalize_qk=normalize_qk, scale=scale, o=None, S_T=S_T, workspace=workspace,
                     _gated=True)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    _req(g, "g", (B, H, T, dv), (q.dtype,))
    _opt(norm_weight, "norm_weight", (H, dv), _F32)
    _opt(y, "y", (B, T, H, dv), (out_dtype,))
    _opt(o, "o", (B, H, T, dv), _F32)
    _same_device(q, dict(g=g, norm_weight=norm_weight, y=y, o=o))
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    S0p, _, sTp = call.out_ptrs
    rc = lib.gdr_chunk_fwd_gated(ctypes.byref(call.desc), *call.ptrs[:8], S0p, _ptr(g), _ptr(norm_weight),
                                 float(eps), _ptr(y), _ptr(o), sTp, *call.ws, _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_gated")
    return y, call.S_T


GATE_ORDER = ("f", "b", "g", "w", "q")


def make_gate_desc(B, T, d_model, H, d, ranks, out_dtype=GDR_BF16) -> GdrGateDesc:
    return GdrGateDesc(int(B), int(T), int(d_model), int(H), int(d), (ctypes.c_int * 5)(*map(int, ranks)),
                       int(out_dtype))


def pack_gate_up(w_up) -> torch.Tensor:
    """The five up-projection weights (dict gate -> [H*d, r] bf16) packed one
    after the other in gate order, as gdr_gate_proj reads them."""
    return torch.cat([_contig(w_up[n]).reshape(-1) for n in GATE_ORDER]).contiguous()


def gdr_gate_proj(x, w_down, w_up, bias, ranks, H, d, *, out_dtype=torch.bfloat16, gates=GATE_ORDER,
                  outs=None, workspace=None, stream=None) -> dict:
    """The five-gate low-rank projection; see gdr_gate_proj in gdr.h.

    x [B,T,d_model] bf16; w_down [R,d_model] bf16; w_up: dict gate -> [H*d, r]
    bf16 (packed here in gate order) or the packed tensor from pack_gate_up;
    bias [5,H*d] fp32 or None.  Returns a dict gate -> [B,H,T,d] tensor for
    the gates in `gates` ("f": log alpha fp32; the others out_dtype), written
    into `outs` (same keys) when given.
    """
    lib = load()
    B, T, dm = _rank(x, "x", 3).shape
    bf = (torch.bfloat16,)
    _req(x, "x", (B, T, dm), bf)
    if len(ranks) != 5:
        raise ValueError("ranks: five gate ranks (f, b, g, w, q)")
    R = sum(int(r) for r in ranks)
    _req(w_down, "w_down", (R, dm), bf)
    if isinstance(w_up, torch.Tensor):
        wu = _req(w_up, "w_up", (H * d * R,), bf)
    else:
        for name, r in zip(GATE_ORDER, ranks):
            _req(w_up.get(name), f"w_up['{name}']", (H * d, int(r)), bf)
        wu = pack_gate_up(w_up)
    _opt(bias, "bias", (5, H * d), _F32)
    if out_dtype not in _FLOAT:
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    _same_device(x, dict(w_down=w_down, w_up=wu, bias=bias, workspace=workspace))
    desc = make_gate_desc(B, T, dm, H, d, ranks, GDR_BF16 if out_dtype == torch.bfloat16 else GDR_F32)
    n = ctypes.c_size_t(0)
    rc = lib.gdr_gate_proj_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_gate_proj_workspace_size")
    workspace = _workspace_arg(workspace, int(n.value), x.device)
    if outs is not None:
        gates = tuple(outs)
        for name, t in outs.items():
            want = torch.float32 if name == "f" else out_dtype
            if (name not in GATE_ORDER or tuple(t.shape) != (B, H, T, d) or t.dtype != want
                    or not t.is_contiguous() or t.device != x.device):
                raise ValueError(f"gdr_gate_proj: output '{name}' must be a contiguous [B,H,T,d] {want} "
                                 f"tensor on {x.device}")
    outs = dict(outs or {})
    for name in GATE_ORDER:
        if name in gates and name not in outs:
            outs[name] = torch.empty((B, H, T, d), device=x.device,
                                     dtype=torch.float32 if name == "f" else out_dtype)
    ptr = lambda name: _ptr(outs.get(name))
    rc = lib.gdr_gate_proj(ctypes.byref(desc), _ptr(x), _ptr(w_down), _ptr(wu), _ptr(bias), ptr("f"), ptr("b"),
                           ptr("g"), ptr("w"), ptr("q"), _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_gate_proj")
    return outs


BWD_OUTPUTS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dgamma", "dz", "dS0")


def gdr_chunk_bwd(q, k, v, log_alpha, b, w, dO, gamma=None, z=None, S0=None, dS_T=None, *,
                  normalize_qk=True, scale=1.0, workspace=None, stream=None, outputs=BWD_OUTPUTS,
                  cu_seqlens=None) -> dict:
    """Backward of gdr_chunk_fwd; see gdr_chunk_bwd in gdr.h.

    Arguments as gdr_chunk_fwd, plus dO [B,H,T,dv] (its dtype is the
    descriptor's out_dtype) and dS_T [B,H,dk,dv] fp32 or None.  Returns a dict
    of fp32 gradients: dq, dk, dv, dS0; dlog_alpha, db, dw shaped as their
    gate (None for a constant gate); dgamma [H,dk] (None without gamma); dz
    (None without z).  Gradients not named in `outputs` are passed as NULL
    (not computed into memory) and returned as None.  With `cu_seqlens` (device
    int32 [N+1]) the tensors are a packed batch as in gdr_chunk_fwd_varlen
    (gdr_chunk_bwd_varlen): B = 1, S0 / dS_T / dS0 are [N,H,dk,dv].
    """
    unknown = set(outputs) - set(BWD_OUTPUTS)
    if unknown:
        raise ValueError(f"unknown outputs {sorted(unknown)}")
    lib = load()
    B, H, T, dk = _rank(q, "q", 4).shape
    dv = _rank(v, "v", 4).shape[-1]
    dt = (_req(q, "q", (B, H, T, dk), _FLOAT).dtype,)
    _req(k, "k", (B, H, T, dk), dt)
    _req(v, "v", (B, H, T, dv), dt)
    amode, la = _log_alpha_arg(log_alpha, (B, H, T, dk))
    bmode, bt = _gate_arg(b, "b", (B, H, T, dk), dt)
    wmode, wt = _gate_arg(w, "w", (B, H, T, dv), dt)
    nseq = 0
    if cu_seqlens is not None:
        cu_seqlens = _cu_seqlens_arg(cu_seqlens, T)
        nseq = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("a packed batch (cu_seqlens) has B = 1")
    _opt(gamma, "gamma", (H, dk), _F32)
    _opt(z, "z", (B, H, T, dk), dt)
    _opt(S0, "S0", (nseq or B, H, dk, dv), _F32)
    _req(dO, "dO", (B, H, T, dv), _FLOAT)
    _opt(dS_T, "dS_T", (nseq or B, H, dk, dv), _F32)
    _same_device(q, dict(k=k, v=v, log_alpha=la, b=bt, w=wt, gamma=gamma, z=z, S0=S0, dO=dO, dS_T=dS_T,
                         cu_seqlens=cu_seqlens, workspace=workspace))
    od = GDR_BF16 if dO.dtype == torch.bfloat16 else GDR_F32
    desc = make_desc(B, H, T, dk, dv, 64, _dtype_code(q), od, int(bool(normalize_qk)), scale, amode, bmode, wmode)
    n = ctypes.c_size_t(0)
    if nseq:
        rc = lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), nseq, ctypes.byref(n))
    else:
        rc = lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_bwd_workspace_size")
    dev = q.device
    workspace = _workspace_arg(workspace, int(n.value), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gshape = lambda mode, d: (B, H, T, d) if mode == PER_CHANNEL else ((B, H, T) if mode == PER_TOKEN else None)
    out = {"dq": torch.empty(B, H, T, dk, **f32), "dk": torch.empty(B, H, T, dk, **f32),
           "dv": torch.empty(B, H, T, dv, **f32), "dS0": torch.empty(nseq or B, H, dk, dv, **f32)}
    for name, mode, d in (("dlog_alpha", amode, dk), ("db", bmode, dk), ("dw", wmode, dv)):
        shp = gshape(mode, d)
        out[name] = torch.empty(*shp, **f32) if shp else None
    out["dgamma"] = torch.empty(H, dk, **f32) if gamma is not None else None
    out["dz"] = torch.empty(B, H, T, dk, **f32) if z is not None else None
    for name in BWD_OUTPUTS:
        if name not in outputs:
            out[name] = None
    tail = (_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bt), _ptr(wt), _ptr(gamma), _ptr(z), _ptr(S0), _ptr(dO),
            _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
            _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dgamma"]), _ptr(out["dz"]), _ptr(out["dS0"]),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if nseq:
        rc = lib.gdr_chunk_bwd_varlen(ctypes.byref(desc), nseq, _ptr(cu_seqlens), *tail)
    else:
        rc = lib.gdr_chunk_bwd(ctypes.byref(desc), *tail)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_bwd_varlen" if nseq else "gdr_chunk_bwd")
    return out


def gdr_decode_step(S, q, k, v, log_alpha, b, w, gamma=None, z=None, *, out_dtype=torch.float32,
                    normalize_qk=True, scale=1.0, o=None, stream=None) -> torch.Tensor:
    """One decode step; S [B,H,dk,dv] fp32 is updated in place; returns o [B,H,dv].

    q, k, z: [B,H,dk]; v: [B,H,dv]; log_alpha [B,H,dk] / [B,H] / 0; b, w per
    channel [B,H,d], per token [B,H] or the scalars 1 / 0.
    """
    lib = load()
    B, H, dk = _rank(q, "q", 3).shape
    dv = _rank(v, "v", 3).shape[-1]
    dt = (_req(q, "q", (B, H, dk), _FLOAT).dtype,)
    _req(k, "k", (B, H, dk), dt)
    _req(v, "v", (B, H, dv), dt)
    _req(S, "S", (B, H, dk, dv), _F32)
    amode, la = _log_alpha_arg(log_alpha, (B, H, dk))
    bmode, bt = _gate_arg(b, "b", (B, H, dk), dt)
    wmode, wt = _gate_arg(w, "w", (B, H, dv), dt)
    _opt(gamma, "gamma", (H, dk), _F32)
    _opt(z, "z", (B, H, dk), dt)
    if out_dtype not in _FLOAT:
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    _opt(o, "o", (B, H, dv), (out_dtype,))
    _same_device(q, dict(S=S, k=k, v=v, log_alpha=la, b=bt, w=wt, gamma=gamma, z=z, o=o))
    od = GDR_BF16 if out_dtype == torch.bfloat16 else GDR_F32
    desc = make_desc(B, H, 1, dk, dv, 64, _dtype_code(q), od, int(bool(normalize_qk)), scale,
                     amode, bmode, wmode)
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
    rc = lib.gdr_decode_step(ctypes.byref(desc), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                             _ptr(bt), _ptr(wt), _ptr(gamma), _ptr(z), _ptr(o), _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_decode_step")
    return o


def gdr_check_inputs(q, k, v, log_alpha, b, w, gamma=None, z=None, *, counts=None, stream=None) -> torch.Tensor:
    """The opt-in precondition check: per input tensor, the number of its
    elements that are NaN or +-inf (and for log_alpha also > 0 or < -30), as
    a device int64 tensor of 8 counts in the order of CHECK_NAMES, written on
    the stream.  Arguments as gdr_chunk_fwd ([B,H,T,d] head-major; gates per
    channel, per token or the scalars 1 / 0); `counts` may be given (int64,
    8 elements, on the inputs' device)."""
    lib = load()
    B, H, T, dk = _rank(q, "q", 4).shape
    dv = _rank(v, "v", 4).shape[-1]
    dt = (_req(q, "q", (B, H, T, dk), _FLOAT).dtype,)
    _req(k, "k", (B, H, T, dk), dt)
    _req(v, "v", (B, H, T, dv), dt)
    amode, la = _log_alpha_arg(log_alpha, (B, H, T, dk))
    bmode, bt = _gate_arg(b, "b", (B, H, T, dk), dt)
    wmode, wt = _gate_arg(w, "w", (B, H, T, dv), dt)
    _opt(gamma, "gamma", (H, dk), _F32)
    _opt(z, "z", (B, H, T, dk), dt)
    _opt(counts, "counts", (len(CHECK_NAMES),), (torch.int64,))
    _same_device(q, dict(k=k, v=v, log_alpha=la, b=bt, w=wt, gamma=gamma, z=z, counts=counts))
    desc = make_desc(B, H, T, dk, dv, 64, _dtype_code(q), GDR_F32, 1, 1.0, amode, bmode, wmode)
    if counts is None:
        counts = torch.empty(len(CHECK_NAMES), dtype=torch.int64, device=q.device)
    rc = lib.gdr_check_inputs(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bt), _ptr(wt),
                              _ptr(gamma), _ptr(z), _ptr(counts), _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_check_inputs")
    return counts


def gdr_chunk_fwd_varlen_workspace_size(desc: GdrDesc, n_seqs: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(desc), int(n_seqs), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_varlen_workspace_size")
    return int(n.value)


def gdr_chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, gamma=None, z=None, S0=None, *,
                         chunk=64, out_dtype=torch.float32, normalize_qk=True, scale=1.0, o=None,
                         S_T=None, workspace=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunkwise forward of a packed batch of sequences of different lengths;
    see gdr_chunk_fwd_varlen in gdr.h.

    q, k: [1,H,T,dk], v: [1,H,T,dv], z [1,H,T,dk], gates [1,H,T,d] / [1,H,T] /
    scalars, all packed along T; cu_seqlens: int32 device tensor [N+1]
    (cu_seqlens[N] = T); gamma [H,dk]; S0 [N,H,dk,dv] fp32.
    Returns (o [1,H,T,dv], S_T [N,H,dk,dv]).
    """
    lib = load()
    Bq, H, T, dk = _rank(q, "q", 4).shape
    dv = _rank(v, "v", 4).shape[-1]
    if Bq != 1:
        raise ValueError("a packed batch has B = 1")
    dt = (_req(q, "q", (Bq, H, T, dk), _FLOAT).dtype,)
    cu = _cu_seqlens_arg(cu_seqlens, T)
    n_seqs = cu.numel() - 1
    _req(k, "k", (Bq, H, T, dk), dt)
    _req(v, "v", (Bq, H, T, dv), dt)
    amode, la = _log_alpha_arg(log_alpha, (Bq, H, T, dk))
    bmode, bt = _gate_arg(b, "b", (Bq, H, T, dk), dt)
    wmode, wt = _gate_arg(w, "w", (Bq, H, T, dv), dt)
    _opt(gamma, "gamma", (H, dk), _F32)
    _opt(z, "z", (Bq, H, T, dk), dt)
    _opt(S0, "S0", (n_seqs, H, dk, dv), _F32)
    if out_dtype not in _FLOAT:
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    _opt(o, "o", (Bq, H, T, dv), (out_dtype,))
    _opt(S_T, "S_T", (n_seqs, H, dk, dv), _F32)
    _same_device(q, dict(cu_seqlens=cu, k=k, v=v, log_alpha=la, b=bt, w=wt, gamma=gamma, z=z, S0=S0, o=o,
                         S_T=S_T, workspace=workspace))
    od = GDR_BF16 if out_dtype == torch.bfloat16 else GDR_F32
    desc = make_desc(Bq, H, T, dk, dv, chunk, _dtype_code(q), od, int(bool(normalize_qk)), scale,
                     amode, bmode, wmode)
    if o is None:
        o = torch.empty((Bq, H, T, dv), dtype=out_dtype, device=q.device)
    if S_T is None:
        S_T = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    need = gdr_chunk_fwd_varlen_workspace_size(desc, n_seqs)
    workspace = _workspace_arg(workspace, need, q.device)
    ptrs = [_ptr(t) for t in (q, k, v, la, bt, wt, gamma, z)]
    rc = lib.gdr_chunk_fwd_varlen(ctypes.byref(desc), n_seqs, _ptr(cu), *ptrs, _ptr(S0), _ptr(o),
                                  _ptr(S_T), _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_varlen")
    return o, S_T


def gdr_output_gate_bwd(o, g, dy, norm_weight=None, eps=1e-6, *, stream=None) -> dict:
    """Backward of the fused output gate; see gdr_output_gate_bwd in gdr.h.

    o [B,H,T,dv] fp32, g [B,H,T,dv] (bf16 or fp32), dy [B,T,H,dv] (bf16 or
    fp32, token-major), norm_weight [H,dv] fp32 or None.  Returns fp32 d_o and
    dg [B,H,T,dv] and d_norm_weight [H,dv] (None without a weight).
    """
    lib = load()
    B, H, T, dv = _rank(o, "o", 4).shape
    _req(o, "o", (B, H, T, dv), _F32)
    _req(g, "g", (B, H, T, dv), _FLOAT)
    _req(dy, "dy", (B, T, H, dv), _FLOAT)
    _opt(norm_weight, "norm_weight", (H, dv), _F32)
    _same_device(o, dict(g=g, dy=dy, norm_weight=norm_weight))
    desc = make_desc(B, H, T, dv, dv, 64, _dtype_code(g), GDR_BF16 if dy.dtype == torch.bfloat16 else GDR_F32,
                     1, 1.0, PER_CHANNEL, PER_CHANNEL, PER_CHANNEL)
    f32 = dict(dtype=torch.float32, device=o.device)
    out = {"d_o": torch.empty(B, H, T, dv, **f32), "dg": torch.empty(B, H, T, dv, **f32),
           "d_norm_weight": torch.empty(H, dv, **f32) if norm_weight is not None else None}
    n = ctypes.c_size_t(0)
    rc = lib.gdr_output_gate_bwd_workspace_size(ctypes.byref(desc), int(norm_weight is not None), ctypes.byref(n))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_output_gate_bwd_workspace_size")
    ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=o.device)
    rc = lib.gdr_output_gate_bwd(ctypes.byref(desc), _ptr(o), _ptr(g), _ptr(norm_weight), float(eps), _ptr(dy),
                                 _ptr(out["d_o"]), _ptr(out["dg"]), _ptr(out["d_norm_weight"]), _ptr(ws),
                                 ws.numel(), _stream(stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_output_gate_bwd")
    return out
