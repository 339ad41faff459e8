"""Thin Python binding of libattn.so (include/attn.h): argument marshalling only.

Every step of the forward, backward and decoding passes runs in the library's HIP kernels.  torch is used only to hold
device memory and to name the current HIP stream.  There is no fallback: if the library is not
built, or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os

# ATTN_LIB_PATH selects another build of the same library (the tests load the race-check and
# AddressSanitizer debug builds this way, each in a process of its own).
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# variant bits and codes, as in include/attn.h
ATTN_MASK_NONE = 0
ATTN_MASK_CAUSAL = 1
ATTN_MASK_SLIDING_WINDOW = 2
ATTN_MASK_DOCUMENT = 3
ATTN_MOD_ALIBI = 1 << 4
ATTN_MOD_SOFTCAP = 1 << 5
ATTN_PREC_FP8 = 1 << 6
ATTN_O_BF16 = 0
ATTN_O_F32 = 1
ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED_DEVICE = -2
ATTN_ERR_LAUNCH = -3
ATTN_ERR_WORKSPACE = -4
ATTN_ERR_COMPILE = -5
ATTN_MODF_SCORE = 1
ATTN_MODF_MASK = 2
ATTN_MODF_MAX_FIRST = 4

MASK_BITS = {"none": ATTN_MASK_NONE, "causal": ATTN_MASK_CAUSAL,
             "window": ATTN_MASK_SLIDING_WINDOW, "document": ATTN_MASK_DOCUMENT}

ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of attn_fwd_noalloc

EXPORTS = ("attn_fwd", "attn_fwd_noalloc", "attn_workspace_size", "attn_tile_shape", "attn_block_table",
           "attn_block_table_host", "attn_bwd", "attn_bwd_workspace_size", "attn_decode",
           "attn_decode_workspace_size", "attn_quantize_fp8", "attn_mod_create",
           "attn_mod_destroy", "attn_mod_workspace_size", "attn_fwd_mod", "attn_fwd_mod_cached",
           "attn_strerror",
           "attn_last_error")


class attn_params(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p), ("doc_offsets", ctypes.c_void_p),
                ("max_docs", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("timing_events", ctypes.c_void_p)]


_lib = None


class AttnError(RuntimeError):
    def __init__(self, code, detail):
        self.code = code
        super().__init__(f"{detail} (code {code})")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               f"(or make -C exact_io_aware_21_amd/csrc)")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_u32, c_vp, c_f = ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float
        P = ctypes.POINTER(attn_params)
        L.attn_fwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_f,
                               c_u32, P, c_vp]
        L.attn_fwd.restype = c_int
        L.attn_fwd_noalloc.argtypes = L.attn_fwd.argtypes
        L.attn_fwd_noalloc.restype = c_int
        L.attn_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_u32]
        L.attn_workspace_size.restype = ctypes.c_size_t
        L.attn_tile_shape.argtypes = [c_int, c_u32, ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
        L.attn_tile_shape.restype = c_int
        L.attn_block_table.argtypes = [c_int, c_int, c_int, c_int, c_u32, P, c_vp, c_vp, c_vp, c_vp]
        L.attn_block_table.restype = c_int
        L.attn_block_table_host.argtypes = [c_int, c_int, c_int, c_int, c_u32, P, c_vp, c_vp, c_vp]
        L.attn_block_table_host.restype = c_int
        L.attn_bwd.argtypes = [c_vp] * 9 + [c_int, c_int, c_int, c_int, c_f, c_u32, P, c_vp]
        L.attn_bwd.restype = c_int
        L.attn_bwd_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_u32]
        L.attn_bwd_workspace_size.restype = ctypes.c_size_t
        L.attn_decode.argtypes = [c_vp] * 7 + [c_int] * 7 + [c_f, c_u32, P, c_vp]
        L.attn_decode.restype = c_int
        L.attn_decode_workspace_size.argtypes = [c_int] * 6
        L.attn_decode_workspace_size.restype = ctypes.c_size_t
        L.attn_quantize_fp8.argtypes = [c_vp, c_vp, c_vp] + [c_int] * 5 + [c_vp]
        L.attn_quantize_fp8.restype = c_int
        L.attn_mod_create.argtypes = [ctypes.c_char_p, c_u32, c_int,
                                       ctypes.POINTER(c_vp), c_vp, ctypes.c_size_t]
        L.attn_mod_create.restype = c_int
        L.attn_mod_destroy.argtypes = [c_vp]
        L.attn_mod_destroy.restype = None
        L.attn_mod_workspace_size.argtypes = [c_vp, c_int, c_int, c_int]
        L.attn_mod_workspace_size.restype = ctypes.c_size_t
        L.attn_fwd_mod.argtypes = [c_vp] * 6 + [c_int] * 3 + [c_f, c_vp, P, c_vp]
        L.attn_fwd_mod.restype = c_int
        L.attn_fwd_mod_cached.argtypes = L.attn_fwd_mod.argtypes
        L.attn_fwd_mod_cached.restype = c_int
        L.attn_strerror.argtypes = [c_int]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc):
    if rc != ATTN_OK:
        L = lib()
        raise AttnError(rc, f"{L.attn_strerror(rc).decode()}: {L.attn_last_error().decode()}")


def variant_bits(mask="none", alibi=False, softcap=False, fp8=False) -> int:
    v = MASK_BITS[mask]
    if alibi:
        v |= ATTN_MOD_ALIBI
    if softcap:
        v |= ATTN_MOD_SOFTCAP
    if fp8:
        v |= ATTN_PREC_FP8
    return v


def attn_tile_shape(d: int, variant: int):
    Br, Bc = ctypes.c_int(), ctypes.c_int()
    _check(lib().attn_tile_shape(d, variant, ctypes.byref(Br), ctypes.byref(Bc)))
    return Br.value, Bc.value


def attn_workspace_size(B: int, H: int, N: int, d: int, variant: int) -> int:
    return int(lib().attn_workspace_size(B, H, N, d, variant))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_device(dev, **tensors):
    """Every named tensor (None skipped) lives on the GPU `dev`.  The library receives raw
    device addresses and cannot tell a host pointer or another GPU's memory from its own, so this
    is the only guard against a kernel reading the wrong memory."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device} while the inputs are on {dev}")


def _check_aux(dev, B, H, variant, alibi_slopes, doc_offsets, workspace):
    """alibi_slopes: contiguous fp32 with at least H values; doc_offsets: contiguous int32
    [B, max_docs + 1]; workspace: contiguous; all on `dev`."""
    import torch
    _on_device(dev, alibi_slopes=alibi_slopes, doc_offsets=doc_offsets, workspace=workspace)
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32
                                     or not alibi_slopes.is_contiguous()
                                     or alibi_slopes.numel() < H):
        raise ValueError(f"alibi_slopes must be a contiguous fp32 tensor of >= {H} values")
    if doc_offsets is not None and (doc_offsets.dtype != torch.int32
                                    or not doc_offsets.is_contiguous()
                                    or doc_offsets.dim() != 2 or doc_offsets.shape[0] != B
                                    or doc_offsets.shape[1] < 2):
        raise ValueError(f"doc_offsets must be a contiguous int32 [B={B}, max_docs + 1] tensor")
    if (variant & 0xF) == ATTN_MASK_DOCUMENT and doc_offsets is None:
        raise ValueError("the document mask needs doc_offsets")
    if (variant & ATTN_MOD_ALIBI) and alibi_slopes is None:
        raise ValueError("ATTN_MOD_ALIBI needs alibi_slopes")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def make_params(window=0, softcap=0.0, alibi_slopes=None, doc_offsets=None, o_dtype=ATTN_O_BF16,
                workspace=None):
    p = attn_params()
    p.window = int(window)
    p.softcap = float(softcap)
    p.alibi_slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    if doc_offsets is not None:
        p.doc_offsets = doc_offsets.data_ptr()
        p.max_docs = doc_offsets.shape[-1] - 1
    p.o_dtype = int(o_dtype)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p


def alloc_workspace(B, H, N, d, variant, device="cuda"):
    """A workspace tensor of the size attn_fwd needs (allocated by torch, outside any call)."""
    import torch
    n = attn_workspace_size(B, H, N, d, variant)
    if n == 0:
        raise AttnError(ATTN_ERR_INVALID_ARG, "invalid shape for attn_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _fwd_args(q, k, v, o, lse, variant, window, softcap, alibi_slopes, doc_offsets, workspace,
              timing_events):
    """Checks the forward arguments; returns (B, H, N, d, params, keepalive)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} must be a contiguous bf16 [B,H,N,d] tensor")
    if o.dtype not in (torch.bfloat16, torch.float32) or not o.is_contiguous() \
            or tuple(o.shape) != (B, H, N, d):
        raise ValueError("o must be a contiguous bf16/fp32 [B,H,N,d] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, N)):
        raise ValueError("lse must be a contiguous fp32 [B,H,N] tensor")
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse)
    _check_aux(q.device, B, H, variant, alibi_slopes, doc_offsets, workspace)
    p = make_params(window, softcap, alibi_slopes, doc_offsets,
                    ATTN_O_F32 if o.dtype == torch.float32 else ATTN_O_BF16, workspace)
    ev = None
    if timing_events is not None:
        if not (timing_events[0].cuda_event and timing_events[1].cuda_event):
            raise ValueError("timing events must have been recorded once before use")
        ev = (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)
        p.timing_events = ctypes.cast(ev, ctypes.c_void_p)
    return B, H, N, d, p, ev


def attn_fwd(q, k, v, o, lse, scale, variant, window=0, softcap=0.0, alibi_slopes=None,
             doc_offsets=None, workspace=None, stream=None, timing_events=None):
    """Calls attn_fwd on torch tensors q, k, v ([B,H,N,d] bf16), o (bf16 or fp32), lse (fp32 or
    None).  alibi_slopes: fp32 [H]; doc_offsets: int32 [B, max_docs+1]; workspace: uint8 tensor
    of at least attn_workspace_size bytes (allocated here when None); timing_events: optional
    pair of torch.cuda.Event(enable_timing=True), each recorded once beforehand (torch creates
    the underlying event on its first record), recorded again around the main kernel."""
    B, H, N, d, p, _ev = _fwd_args(q, k, v, o, lse, variant, window, softcap, alibi_slopes,
                                   doc_offsets, workspace, timing_events)
    if workspace is None:
        workspace = alloc_workspace(B, H, N, d, variant, q.device)
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                          float(scale), variant, ctypes.byref(p), _stream(stream)))
    return o, lse


def attn_fwd_noalloc(q, k, v, o, lse, scale, variant, window=0, softcap=0.0, alibi_slopes=None,
                     doc_offsets=None, stream=None, timing_events=None):
    """Calls attn_fwd_noalloc: attn_fwd with the library's static scratch as the workspace, for
    callers that cannot allocate (no workspace argument; shapes whose workspace would exceed
    ATTN_NOALLOC_SCRATCH_BYTES are refused).  Calls that can overlap on one GPU race."""
    B, H, N, d, p, _ev = _fwd_args(q, k, v, o, lse, variant, window, softcap, alibi_slopes,
                                   doc_offsets, None, timing_events)
    _check(lib().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                  float(scale), variant, ctypes.byref(p), _stream(stream)))
    return o, lse


class FwdPlan:
    """attn_fwd (or, with noalloc=True, attn_fwd_noalloc) on fixed buffers, for loops that run
    the forward pass many times on the same tensors: the arguments are checked and marshalled
    once, here, and each call is then one C call (which still validates its arguments).  The
    tensors must stay alive and keep their storage while the plan is used; their contents may
    change between calls.  stream=None means the current stream at each call (so a call made
    under graph capture goes to the capturing stream)."""

    def __init__(self, q, k, v, o, lse, scale, variant, window=0, softcap=0.0, alibi_slopes=None,
                 doc_offsets=None, workspace=None, stream=None, noalloc=False):
        if noalloc and workspace is not None:
            raise ValueError("attn_fwd_noalloc takes no workspace")
        B, H, N, d, p, _ = _fwd_args(q, k, v, o, lse, variant, window, softcap, alibi_slopes,
                                     doc_offsets, workspace, None)
        if not noalloc and workspace is None:
            workspace = alloc_workspace(B, H, N, d, variant, q.device)
            p.workspace = workspace.data_ptr()
            p.workspace_bytes = workspace.numel() * workspace.element_size()
        self._keep = (q, k, v, o, lse, alibi_slopes, doc_offsets, workspace)
        self._p = p
        self._ev = None
        self._fn = lib().attn_fwd_noalloc if noalloc else lib().attn_fwd
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                      variant, ctypes.byref(p))
        self._stream = None if stream is None else _stream(stream)

    @staticmethod
    def events(timing_events):
        """A pair of torch.cuda.Event(enable_timing=True), each recorded once beforehand,
        marshalled for __call__ (prepare them before a timed loop)."""
        if not (timing_events[0].cuda_event and timing_events[1].cuda_event):
            raise ValueError("timing events must have been recorded once before use")
        return (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)

    def __call__(self, timing_events=None):
        """One forward pass; timing_events: None, a pair of events as for attn_fwd, or the
        result of events() for that pair."""
        p = self._p
        if timing_events is None:
            p.timing_events = None
        else:
            if not isinstance(timing_events, ctypes.Array):
                timing_events = self.events(timing_events)
            self._ev = timing_events
            p.timing_events = ctypes.addressof(timing_events)
        _check(self._fn(*self._args, self._stream if self._stream is not None else _stream(None)))


def attn_bwd_workspace_size(B: int, H: int, N: int, d: int, variant: int) -> int:
    return int(lib().attn_bwd_workspace_size(B, H, N, d, variant))


def alloc_bwd_workspace(B, H, N, d, variant, device="cuda"):
    """A workspace tensor of the size attn_bwd needs (allocated by torch, outside any call)."""
    import torch
    n = attn_bwd_workspace_size(B, H, N, d, variant)
    if n == 0:
        raise AttnError(ATTN_ERR_INVALID_ARG, "invalid shape for attn_bwd_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale, variant, window=0, softcap=0.0,
             alibi_slopes=None, doc_offsets=None, workspace=None, stream=None, timing_events=None):
    """Calls attn_bwd: q, k, v, dout bf16 [B,H,N,d]; o the forward output and dq, dk, dv the
    gradients, all of one dtype (bf16 or fp32); lse fp32 [B,H,N] from the forward."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} must be a contiguous bf16 [B,H,N,d] tensor")
    for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dtype != o.dtype or o.dtype not in (torch.bfloat16, torch.float32) \
                or not t.is_contiguous() or tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} must be a contiguous [B,H,N,d] tensor of o's dtype "
                             f"(bf16 or fp32)")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be a contiguous fp32 [B,H,N] tensor")
    _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv)
    _check_aux(q.device, B, H, variant, alibi_slopes, doc_offsets, workspace)
    if workspace is None:
        workspace = alloc_bwd_workspace(B, H, N, d, variant, q.device)
    p = make_params(window, softcap, alibi_slopes, doc_offsets,
                    ATTN_O_F32 if o.dtype == torch.float32 else ATTN_O_BF16, workspace)
    ev = None
    if timing_events is not None:
        if not (timing_events[0].cuda_event and timing_events[1].cuda_event):
            raise ValueError("timing events must have been recorded once before use")
        ev = (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)
        p.timing_events = ctypes.cast(ev, ctypes.c_void_p)
    _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, N, d, float(scale), variant, ctypes.byref(p),
                          _stream(stream)))
    return dq, dk, dv


def attn_decode_workspace_size(B: int, H: int, Lq: int, d: int, page_size: int,
                               max_pages: int) -> int:
    return int(lib().attn_decode_workspace_size(B, H, Lq, d, page_size, max_pages))


def alloc_decode_workspace(B, H, Lq, d, page_size, max_pages, device="cuda"):
    """A workspace tensor of the size attn_decode needs (allocated by torch, outside any call)."""
    import torch
    n = attn_decode_workspace_size(B, H, Lq, d, page_size, max_pages)
    if n == 0:
        raise AttnError(ATTN_ERR_INVALID_ARG, "invalid shape for attn_decode_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_decode(q, k_cache, v_cache, page_table, seq_lens, o, lse, scale, causal=True,
                workspace=None, stream=None, timing_events=None):
    """Calls attn_decode: q bf16 [B,H,Lq,d]; k_cache, v_cache bf16 [n_pages,H,page,d];
    page_table int32 [B,max_pages]; seq_lens int32 [B]; o bf16 or fp32 [B,H,Lq,d]; lse fp32
    [B,H,Lq] or None."""
    import torch
    B, H, Lq, d = q.shape
    n_pages, Hc, page, dc = k_cache.shape
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B,H,Lq,d] tensor")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or \
                tuple(t.shape) != (n_pages, H, page, d):
            raise ValueError(f"{name} must be a contiguous bf16 [n_pages,H,page,d] tensor")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or \
            page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 [B,max_pages] tensor")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be an int32 [B] tensor")
    if o.dtype not in (torch.bfloat16, torch.float32) or not o.is_contiguous() or \
            tuple(o.shape) != (B, H, Lq, d):
        raise ValueError("o must be a contiguous bf16/fp32 [B,H,Lq,d] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, Lq)):
        raise ValueError("lse must be a contiguous fp32 [B,H,Lq] tensor")
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
               seq_lens=seq_lens, o=o, lse=lse, workspace=workspace)
    max_pages = page_table.shape[1]
    if workspace is None:
        workspace = alloc_decode_workspace(B, H, Lq, d, page, max_pages, q.device)
    p = make_params(o_dtype=ATTN_O_F32 if o.dtype == torch.float32 else ATTN_O_BF16,
                    workspace=workspace)
    ev = None
    if timing_events is not None:
        if not (timing_events[0].cuda_event and timing_events[1].cuda_event):
            raise ValueError("timing events must have been recorded once before use")
        ev = (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)
        p.timing_events = ctypes.cast(ev, ctypes.c_void_p)
    variant = ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    _check(lib().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                             _ptr(seq_lens), _ptr(o), _ptr(lse), B, H, Lq, d, page, max_pages,
                             n_pages, float(scale), variant, ctypes.byref(p), _stream(stream)))
    return o, lse


def attn_quantize_fp8(x, codes, scales, rows, stream=None):
    """Block quantization of x (bf16 [B,H,N,d]) into codes (uint8, same shape) and scales
    (fp32 [B,H,ceil(N/rows)])."""
    import torch
    B, H, N, d = x.shape
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [B,H,N,d] tensor")
    if codes.dtype != torch.uint8 or not codes.is_contiguous() or tuple(codes.shape) != (B, H, N, d):
        raise ValueError("codes must be a contiguous uint8 [B,H,N,d] tensor")
    nb = -(-N // rows)
    if scales.dtype != torch.float32 or not scales.is_contiguous() or \
            tuple(scales.shape) != (B, H, nb):
        raise ValueError("scales must be a contiguous fp32 [B,H,ceil(N/rows)] tensor")
    _on_device(x.device, x=x, codes=codes, scales=scales)
    _check(lib().attn_quantize_fp8(_ptr(x), _ptr(codes), _ptr(scales), B, H, N, d, rows,
                                   _stream(stream)))
    return codes, scales


def attn_block_table(B, H, N, d, variant, cls, kv_cnt, kv_list, window=0, doc_offsets=None,
                     stream=None):
    """Device block table into torch tensors cls (int8), kv_cnt (int32), kv_list (int32)."""
    import torch
    Br, Bc = attn_tile_shape(d, variant)
    n_qt, n_kt = -(-N // Br), -(-N // Bc)
    Bm = B if (variant & 0xF) == ATTN_MASK_DOCUMENT else 1
    for name, t, dt, shape in (("cls", cls, torch.int8, (Bm, n_qt, n_kt)),
                               ("kv_cnt", kv_cnt, torch.int32, (Bm, n_qt)),
                               ("kv_list", kv_list, torch.int32, (Bm, n_qt, n_kt))):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape}")
    _on_device(cls.device, cls=cls, kv_cnt=kv_cnt, kv_list=kv_list)
    _check_aux(cls.device, B, H, variant & 0xF, None, doc_offsets, None)
    p = make_params(window=window, doc_offsets=doc_offsets)
    _check(lib().attn_block_table(B, H, N, d, variant, ctypes.byref(p), _ptr(cls), _ptr(kv_cnt),
                                  _ptr(kv_list), _stream(stream)))


def attn_block_table_host(B, H, N, d, variant, window=0, doc_offsets=None):
    """The same table computed on the host by the library; returns numpy arrays."""
    import numpy as np
    Br, Bc = attn_tile_shape(d, variant)
    n_qt, n_kt = -(-N // Br), -(-N // Bc)
    Bm = B if (variant & 0xF) == ATTN_MASK_DOCUMENT else 1
    cls = np.zeros((Bm, n_qt, n_kt), dtype=np.int8)
    cnt = np.zeros((Bm, n_qt), dtype=np.int32)
    lst = np.zeros((Bm, n_qt, n_kt), dtype=np.int32)
    p = attn_params()
    p.window = int(window)
    offs = None
    if doc_offsets is not None:
        offs = np.ascontiguousarray(doc_offsets, dtype=np.int32)
        p.doc_offsets = offs.ctypes.data
        p.max_docs = offs.shape[-1] - 1
    _check(lib().attn_block_table_host(B, H, N, d, variant, ctypes.byref(p), cls.ctypes.data,
                                       cnt.ctypes.data, lst.ctypes.data))
    return cls, cnt, lst


class AttnMod:
    """A runtime-compiled score / mask modification (attn_mod_create).  `source` is HIP C++
    defining attn_score_mod and/or attn_mask_mod (see include/attn.h); `flags` names which.
    Compilation needs no GPU.  The compiler's messages are in `.log`."""

    def __init__(self, source: str, flags: int, d: int):
        self._h = None
        buf = ctypes.create_string_buffer(1 << 16)
        h = ctypes.c_void_p()
        rc = lib().attn_mod_create(source.encode(), flags, d, ctypes.byref(h), buf, len(buf))
        self.log = buf.value.decode(errors="replace")
        if rc != ATTN_OK:
            L = lib()
            raise AttnError(rc, f"{L.attn_strerror(rc).decode()}: {self.log or L.attn_last_error().decode()}")
        self._h, self.flags, self.d = h, flags, d

    def close(self):
        if self._h is not None:
            lib().attn_mod_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, B: int, H: int, N: int) -> int:
        return int(lib().attn_mod_workspace_size(self._h, B, H, N))

    def alloc_workspace(self, B, H, N, device="cuda"):
        import torch
        n = self.workspace_size(B, H, N)
        if n == 0:
            raise AttnError(ATTN_ERR_INVALID_ARG, "invalid shape for attn_mod_workspace_size")
        return torch.empty(n, dtype=torch.uint8, device=device)

    def fwd(self, q, k, v, o, lse, scale, mod_params=None, workspace=None, stream=None,
            timing_events=None, cached_table=False):
        """attn_fwd_mod on torch tensors: q, k, v bf16 [B,H,N,d]; o bf16 or fp32; lse fp32
        [B,H,N] or None; mod_params a device fp32 tensor or None.  cached_table=True calls
        attn_fwd_mod_cached, which reuses the block table an earlier call left in `workspace`
        (same mod, B, N and mod_params values)."""
        import torch
        if cached_table and workspace is None:
            raise ValueError("cached_table needs the workspace of an earlier call")
        B, H, N, d = q.shape
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != (B, H, N, d):
                raise ValueError(f"{name} must be a contiguous bf16 [B,H,N,d] tensor")
        if o.dtype not in (torch.bfloat16, torch.float32) or not o.is_contiguous() \
                or tuple(o.shape) != (B, H, N, d):
            raise ValueError("o must be a contiguous bf16/fp32 [B,H,N,d] tensor")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                                or tuple(lse.shape) != (B, H, N)):
            raise ValueError("lse must be a contiguous fp32 [B,H,N] tensor")
        if mod_params is not None and (mod_params.dtype != torch.float32
                                       or not mod_params.is_contiguous()):
            raise ValueError("mod_params must be a contiguous fp32 tensor")
        _on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, mod_params=mod_params,
                   workspace=workspace)
        if workspace is None:
            workspace = self.alloc_workspace(B, H, N, q.device)
        p = make_params(o_dtype=ATTN_O_F32 if o.dtype == torch.float32 else ATTN_O_BF16,
                        workspace=workspace)
        ev = None
        if timing_events is not None:
            if not (timing_events[0].cuda_event and timing_events[1].cuda_event):
                raise ValueError("timing events must have been recorded once before use")
            ev = (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)
            p.timing_events = ctypes.cast(ev, ctypes.c_void_p)
        fn = lib().attn_fwd_mod_cached if cached_table else lib().attn_fwd_mod
        _check(fn(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, float(scale),
                  _ptr(mod_params), ctypes.byref(p), _stream(stream)))
        return o, lse
