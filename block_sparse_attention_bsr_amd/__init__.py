"""Block-sparse (BSR, 128 x 128 tiles) softmax attention for AMD MI355X.

A thin binding over the C ABI in ``include/bsr_attn.h`` (``libbsr_attn.so``,
built in-tree by ``python -m block_sparse_attention_bsr_amd.build``). The
binding only marshals arguments: every step of the forward and backward runs
in the library's HIP kernels. PyTorch supplies device memory and the stream.
If the library is missing, every entry point raises; there is no fallback.

    s = bsr_attn_build_structure(row_ptr, col_idx)          # host, once per mask
    o, row_max, row_denom = bsr_attn_fwd(s, q, k, v)         # q, k, v: [B, H, S, D]
    dq, dk, dv = bsr_attn_bwd(s, q, k, v, o, do, row_max, row_denom)
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

import numpy as np
import torch

__all__ = [
    "BsrAttnError", "Structure", "bsr_attn_build_structure", "build_structure_from_mask",
    "bsr_attn_fwd", "bsr_attn_fwd_two_pass", "bsr_attn_bwd", "bsr_attn_bwd_ds", "bsr_attn_bwd_noalloc", "bsr_spmm", "timing_begin", "timing_end", "mfma_probe", "library", "LIBRARY_PATH",
]

LIBRARY_PATH = Path(__file__).resolve().parent / "libbsr_attn.so"
BLOCK = 128

_STATUS = {
    0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "WORKSPACE_TOO_SMALL", 4: "HIP", 5: "HOST_ALLOC",
}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class BsrAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"bsr_attn error {_STATUS.get(status, status)}: {message}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class _Info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_block_rows", "nnzb", "split_threshold", "n_row_items", "n_col_items", "n_row_merges",
        "n_col_merges", "n_row_slots", "n_col_slots", "max_row_blocks", "max_col_blocks",
        "fine_split_threshold", "fine_n_row_items")]


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None
# Callables run with a Structure just before its handle is destroyed (the
# operator library's registry of live structures uses this).
_destroy_hooks: list = []


def library() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIBRARY_PATH.exists():
            raise RuntimeError(
                f"{LIBRARY_PATH} is missing: build it with `python -m block_sparse_attention_bsr_amd.build`")
        L = ctypes.CDLL(str(LIBRARY_PATH))
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        L.bsr_attn_build_structure.argtypes = [i32, vp, vp, i32, i32, ctypes.POINTER(vp)]
        L.bsr_attn_build_structure.restype = i32
        L.bsr_attn_destroy_structure.argtypes = [vp]
        L.bsr_attn_destroy_structure.restype = None
        L.bsr_attn_structure_get_info.argtypes = [vp, ctypes.POINTER(_Info)]
        L.bsr_attn_structure_get_info.restype = i32
        L.bsr_attn_structure_plan_bytes.argtypes = [vp]
        L.bsr_attn_structure_plan_bytes.restype = sz
        L.bsr_attn_structure_pack.argtypes = [vp, vp, sz]
        L.bsr_attn_structure_pack.restype = i32
        L.bsr_attn_structure_bind_plan.argtypes = [vp, vp, sz]
        L.bsr_attn_structure_bind_plan.restype = i32
        L.bsr_attn_structure_unbind_plan.argtypes = [vp, vp]
        L.bsr_attn_structure_unbind_plan.restype = i32
        L.bsr_attn_workspace_bytes.argtypes = [vp, ctypes.POINTER(_Problem), ctypes.c_int]
        L.bsr_attn_workspace_bytes.restype = sz
        L.bsr_attn_fwd.argtypes = [vp, vp, ctypes.POINTER(_Problem)] + [vp] * 6 + [vp, sz, vp]
        L.bsr_attn_fwd.restype = i32
        L.bsr_attn_fwd_two_pass.argtypes = [vp, vp, ctypes.POINTER(_Problem)] + [vp] * 6 + [vp, sz, vp]
        L.bsr_attn_fwd_two_pass.restype = i32
        L.bsr_spmm_workspace_bytes.argtypes = [vp, i32]
        L.bsr_spmm_workspace_bytes.restype = sz
        L.bsr_spmm.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.bsr_spmm.restype = i32
        L.bsr_attn_bwd.argtypes = [vp, vp, ctypes.POINTER(_Problem)] + [vp] * 10 + [vp, sz, vp]
        L.bsr_attn_bwd.restype = i32
        L.bsr_attn_bwd_ds.argtypes = [vp, vp, ctypes.POINTER(_Problem)] + [vp] * 10 + [vp, sz, vp]
        L.bsr_attn_bwd_ds.restype = i32
        L.bsr_attn_bwd_noalloc.argtypes = [vp, vp, ctypes.POINTER(_Problem)] + [vp] * 10 + [vp]
        L.bsr_attn_bwd_noalloc.restype = i32
        L.bsr_attn_mfma_probe.argtypes = [i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
        L.bsr_attn_mfma_probe.restype = i32
        L.bsr_attn_timing_begin.argtypes = []
        L.bsr_attn_timing_begin.restype = i32
        L.bsr_attn_timing_end.argtypes = [ctypes.POINTER(_KernelTime), ctypes.c_int]
        L.bsr_attn_timing_end.restype = ctypes.c_int
        L.bsr_attn_last_error.argtypes = []
        L.bsr_attn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise BsrAttnError(status, library().bsr_attn_last_error().decode())


class Structure:
    """A built BSR structure: the host handle plus (lazily) its device plan."""

    def __init__(self, row_ptr, col_idx, block_size: int = BLOCK, split_threshold: int = 0):
        L = library()
        self.row_ptr = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int32))
        self.col_idx = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int32))
        # The C builder reads row_ptr[nb] + 1 entries of row_ptr and row_ptr[nb]
        # entries of col_idx: check the lengths it cannot see.
        if self.row_ptr.ndim != 1 or self.col_idx.ndim != 1:
            raise ValueError("row_ptr and col_idx must be one-dimensional")
        if self.row_ptr.size < 2:
            raise ValueError("row_ptr must hold nb + 1 >= 2 entries")
        if self.row_ptr[-1] != self.col_idx.size:
            raise ValueError(f"col_idx has {self.col_idx.size} entries but row_ptr[-1] = {int(self.row_ptr[-1])}")
        self.nb = len(self.row_ptr) - 1
        handle = ctypes.c_void_p()
        ci = self.col_idx.ctypes.data if self.col_idx.size else None
        _check(L.bsr_attn_build_structure(self.nb, self.row_ptr.ctypes.data, ci, block_size,
                                          split_threshold, ctypes.byref(handle)))
        self._h = handle
        info = _Info()
        _check(L.bsr_attn_structure_get_info(self._h, ctypes.byref(info)))
        self.info = {name: getattr(info, name) for name, _ in _Info._fields_}
        nbytes = L.bsr_attn_structure_plan_bytes(self._h)
        self.plan = np.zeros(nbytes // 4, dtype=np.int32)
        _check(L.bsr_attn_structure_pack(self._h, self.plan.ctypes.data, nbytes))
        self._device_plans = {}

    @property
    def handle(self):
        return self._h

    def device_plan(self, device) -> torch.Tensor:
        """The plan's copy on ``device``, uploaded and bound to the structure
        on first use (the library accepts only bound copies)."""
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        key = (device.type, device.index)
        if key not in self._device_plans:
            t = torch.from_numpy(self.plan).to(device)
            torch.cuda.synchronize(device)  # the copy has landed before any kernel can read it
            _check(library().bsr_attn_structure_bind_plan(self._h, t.data_ptr(), t.numel() * 4))
            self._device_plans[key] = t
        return self._device_plans[key]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            for hook in _destroy_hooks or ():  # registrations of the handle end before it is destroyed
                hook(self)
            _lib.bsr_attn_destroy_structure(h)
            self._h = None


def bsr_attn_build_structure(row_ptr, col_idx, block_size: int = BLOCK, split_threshold: int = 0) -> Structure:
    """Validate a BSR block structure and build its plan (host only).

    split_threshold: longest work item in stored blocks; longer rows and
    columns are split and their fp32 partials merged. 0 picks it from the
    mean line length (the rule in bsr_attn.h). The structure does not know
    the batch x head count, so a tiny structure run on few heads (a handful
    of block rows, one head) fills more of the GPU with a small explicit
    value such as 1, at the price of the merge launches."""
    return Structure(row_ptr, col_idx, block_size, split_threshold)


def build_structure_from_mask(block_mask, split_threshold: int = 0) -> Structure:
    """Structure of a boolean [nb, nb] block mask (True = stored block)."""
    bm = np.asarray(block_mask, dtype=bool)
    row_ptr = np.concatenate([[0], np.cumsum(bm.sum(axis=1))]).astype(np.int32)
    col_idx = np.nonzero(bm)[1].astype(np.int32)
    return Structure(row_ptr, col_idx, BLOCK, split_threshold)


def _problem(q: torch.Tensor, scale) -> _Problem:
    if q.dim() != 4:
        raise ValueError("operands must be [batch, heads, seq_len, head_dim]")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype} (float32, bfloat16 or float16)")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return _Problem(B, H, S, D, _DTYPES[q.dtype], float(scale))


def _check_operands(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t.device != ref.device or t.dtype != ref.dtype or t.shape != ref.shape:
            raise ValueError(f"{name} must match q in device, dtype and shape")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if ref.device.type != "cuda":
        raise ValueError("operands must be on a GPU device")


def _workspace(s: Structure, prob: _Problem, backward: int, device) -> tuple[torch.Tensor | None, int]:
    nbytes = library().bsr_attn_workspace_bytes(s.handle, ctypes.byref(prob), backward)
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _ptr(t):
    return None if t is None else t.data_ptr()


def bsr_attn_fwd(s: Structure, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale=None):
    """Forward: returns (O, row_max, row_denom); statistics are fp32 [B, H, S]."""
    _check_operands(q, q=q, k=k, v=v)
    prob = _problem(q, scale)
    o = torch.empty_like(q)
    row_max = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    row_denom = torch.empty_like(row_max)
    ws, nbytes = _workspace(s, prob, 0, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(library().bsr_attn_fwd(s.handle, s.device_plan(q.device).data_ptr(), ctypes.byref(prob),
                                  q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), row_max.data_ptr(),
                                  row_denom.data_ptr(), _ptr(ws), nbytes, stream))
    return o, row_max, row_denom


def bsr_attn_fwd_two_pass(s: Structure, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale=None):
    """The pages' two-pass forward (statistics pass, then output pass); same
    results as bsr_attn_fwd up to rounding."""
    _check_operands(q, q=q, k=k, v=v)
    prob = _problem(q, scale)
    o = torch.empty_like(q)
    row_max = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    row_denom = torch.empty_like(row_max)
    ws, nbytes = _workspace(s, prob, 0, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(library().bsr_attn_fwd_two_pass(s.handle, s.device_plan(q.device).data_ptr(), ctypes.byref(prob),
                                           q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                           row_max.data_ptr(), row_denom.data_ptr(), _ptr(ws), nbytes, stream))
    return o, row_max, row_denom


def _backward(entry: str, kind: int, s: Structure, q, k, v, o, do, row_max, row_denom, scale):
    _check_operands(q, q=q, k=k, v=v, o=o, do=do)
    for name, t in (("row_max", row_max), ("row_denom", row_denom)):
        if t.dtype != torch.float32 or t.shape != q.shape[:3] or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 [B, H, S] on q's device")
    prob = _problem(q, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws, nbytes = _workspace(s, prob, kind, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(getattr(library(), entry)(s.handle, s.device_plan(q.device).data_ptr(), ctypes.byref(prob),
                                     q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                     row_max.data_ptr(), row_denom.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), _ptr(ws), nbytes, stream))
    return dq, dk, dv


def bsr_attn_bwd(s: Structure, q, k, v, o, do, row_max, row_denom, scale=None):
    """Backward of <O, dO>: returns (dQ, dK, dV) in the operand dtype."""
    return _backward("bsr_attn_bwd", 1, s, q, k, v, o, do, row_max, row_denom, scale)


def bsr_attn_bwd_noalloc(s: Structure, q, k, v, o, do, row_max, row_denom, scale=None):
    """bsr_attn_bwd with the library's own fixed device workspace (no
    workspace allocation by the library; see bsr_attn.h for its limit and for
    why calls that overlap on one GPU race). Returns (dQ, dK, dV)."""
    _check_operands(q, q=q, k=k, v=v, o=o, do=do)
    for name, t in (("row_max", row_max), ("row_denom", row_denom)):
        if t.dtype != torch.float32 or t.shape != q.shape[:3] or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 [B, H, S] on q's device")
    prob = _problem(q, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(library().bsr_attn_bwd_noalloc(s.handle, s.device_plan(q.device).data_ptr(), ctypes.byref(prob),
                                          q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                          row_max.data_ptr(), row_denom.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                          dv.data_ptr(), stream))
    return dq, dk, dv


def bsr_attn_bwd_ds(s: Structure, q, k, v, o, do, row_max, row_denom, scale=None):
    """The same backward with dS stored by the dK/dV pass and dQ = dS K read
    from it (bf16 / fp16 only): returns (dQ, dK, dV) in the operand dtype."""
    return _backward("bsr_attn_bwd_ds", 2, s, q, k, v, o, do, row_max, row_denom, scale)


def bsr_spmm(s: Structure, blocks: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """C = A B for the block-sparse A whose stored blocks are ``blocks``
    [nnzb, 128, 128] (BSR order, the structure's) and dense ``b``
    [nb*128, n_cols]; returns C [nb*128, n_cols] in b's dtype."""
    if b.dim() != 2 or b.shape[0] != s.nb * BLOCK:
        raise ValueError("b must be [nb*128, n_cols]")
    if b.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {b.dtype} (float32, bfloat16 or float16)")
    nnzb = s.info["nnzb"]
    if blocks.shape != (nnzb, BLOCK, BLOCK) or blocks.dtype != b.dtype or blocks.device != b.device:
        raise ValueError("blocks must be [nnzb, 128, 128] in b's dtype, on b's device")
    for name, t in (("blocks", blocks), ("b", b)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if b.device.type != "cuda":
        raise ValueError("operands must be on a GPU device")
    n_cols = b.shape[1]
    c = torch.empty_like(b)
    nbytes = library().bsr_spmm_workspace_bytes(s.handle, n_cols)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=b.device) if nbytes else None
    stream = torch.cuda.current_stream(b.device).cuda_stream
    _check(library().bsr_spmm(s.handle, s.device_plan(b.device).data_ptr(), _DTYPES[b.dtype], n_cols,
                              blocks.data_ptr() if nnzb else None, b.data_ptr(), c.data_ptr(), _ptr(ws), nbytes,
                              stream))
    return c


def mfma_probe(dtype: torch.dtype, iters: int, sink: torch.Tensor) -> float:
    """Enqueue the MFMA-loop probe (matrix products on random register
    operands, two waves per SIMD on every CU) on the current stream of
    ``sink``'s device; returns its FLOPs. ``sink``: a one-element float32
    device tensor. Time it with events on the same stream."""
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    if sink.dtype != torch.float32 or sink.numel() < 1 or not sink.is_cuda:
        raise ValueError("sink must be a float32 tensor on a GPU")
    flops = ctypes.c_double()
    stream = torch.cuda.current_stream(sink.device).cuda_stream
    _check(library().bsr_attn_mfma_probe(_DTYPES[dtype], iters, sink.data_ptr(), stream, ctypes.byref(flops)))
    return flops.value


def timing_begin() -> None:
    """Start per-kernel event timing of fwd/bwd calls on this thread."""
    _check(library().bsr_attn_timing_begin())


def timing_end() -> dict:
    """Stop timing; {kernel name: (launches, total milliseconds)} (waits for the events)."""
    buf = (_KernelTime * 64)()
    n = library().bsr_attn_timing_end(buf, 64)
    if n < 0:
        raise BsrAttnError(4, library().bsr_attn_last_error().decode())
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, 64))}


from .autograd import block_sparse_attention  # noqa: E402  (uses the entry points above)

__all__.append("block_sparse_attention")
