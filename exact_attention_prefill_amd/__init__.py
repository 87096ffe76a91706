"""Python binding of the gfx950 attention library (libattn.so).

Same names and argument order as the two calls on page 3 of the pages
("Installation": ``prefill(q, k, v, causal, scale)`` and
``decode(q, k_cache, v_cache, seq_lens, scale)``).  This layer only marshals
arguments: it checks tensor metadata, passes device pointers and the current
HIP stream through ctypes, and turns a negative status into an exception.  Every
step of the computation runs in the library's HIP kernels; there is no fallback.
PyTorch supplies device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F16, ATTN_BF16 = 0, 1
ATTN_OK = 0
ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGNMENT, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = -1, -2, -3, -4, -5
DECODE_ROW_GRANULE = 32
DECODE_WGS_PER_CU = 8
DECODE_MIN_CHUNK = 64
DECODE_MFMA_LDS_BYTES = 163840
DECODE_SCRATCH_BYTES = 16777216

# Every symbol include/attn.h declares.
EXPORTS = (
    "attn_prefill",
    "attn_decode",
    "attn_decode_ex",
    "attn_decode_choose_split",
    "attn_decode_workspace_bytes",
    "attn_status_string",
    "attn_last_error",
    "attn_prefill_gqa",
    "attn_decode_gqa",
    "attn_decode_gqa_choose_split",
    "attn_prefill_ex",
    "attn_backward",
    "attn_backward_workspace_bytes",
    "attn_prefill_plan",
    "attn_build_id",
    "attn_decode_noalloc",
    "attn_decode_split",
    "attn_decode_merge",
    "attn_measure_read",
)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


class AttnValueError(AttnError, ValueError):
    pass


def lib() -> ctypes.CDLL:
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m exact_attention_prefill_amd.build` "
                "(the HIP library is the only implementation)"
            )
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        L.attn_prefill.restype = i
        L.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        L.attn_decode.restype = i
        L.attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        L.attn_decode_ex.restype = i
        L.attn_decode_choose_split.argtypes = [i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.attn_decode_choose_split.restype = i
        L.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
        L.attn_decode_workspace_bytes.restype = sz
        L.attn_status_string.argtypes = [i]
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_prefill_gqa.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        L.attn_prefill_gqa.restype = i
        L.attn_prefill_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        L.attn_prefill_ex.restype = i
        L.attn_backward.argtypes = [vp] * 9 + [i] * 7 + [f, vp, sz, vp]
        L.attn_backward.restype = i
        L.attn_backward_workspace_bytes.argtypes = [i, i, i]
        L.attn_backward_workspace_bytes.restype = sz
        L.attn_decode_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
        L.attn_decode_gqa.restype = i
        L.attn_decode_gqa_choose_split.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.attn_decode_gqa_choose_split.restype = i
        L.attn_prefill_plan.argtypes = [i] * 6 + [ctypes.POINTER(i)] * 4
        L.attn_prefill_plan.restype = i
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        L.attn_decode_noalloc.restype = i
        L.attn_decode_split.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
        L.attn_decode_split.restype = i
        L.attn_decode_merge.argtypes = [vp, sz, vp, i, i, i, i, i, i, vp]
        L.attn_decode_merge.restype = i
        L.attn_measure_read.argtypes = [vp, sz, i, vp, sz, vp]
        L.attn_measure_read.restype = i
        L.attn_build_id.argtypes = []
        L.attn_build_id.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != ATTN_OK:
        L = lib()
        detail = L.attn_last_error().decode() or L.attn_status_string(status).decode()
        cls = AttnValueError if status in (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGNMENT) else AttnError
        raise cls(status, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise AttnValueError(ATTN_ERR_INVALID_ARG, f"dtype {t.dtype} is not float16/bfloat16")


def _dev_tensor(t: torch.Tensor, name: str, dtype, shape) -> int:
    if not isinstance(t, torch.Tensor):
        raise AttnValueError(ATTN_ERR_INVALID_ARG, f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise AttnValueError(ATTN_ERR_INVALID_ARG, f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise AttnValueError(ATTN_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise AttnValueError(ATTN_ERR_INVALID_ARG, f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def prefill(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Exact attention for fp16/bf16 GPU tensors q (B, H, N, d) and k, v (B, Hkv, N, d);
    returns out shaped like q.  Hkv < H selects grouped K/V heads (query head h reads
    K/V head h // (H // Hkv)); Hkv must divide H.  ``lse``: True allocates and returns
    (out, lse), or a float32 GPU tensor (B, H, N) to fill; each row's natural-log
    log-sum-exp of the scaled scores."""
    if q.dim() != 4 or k.dim() != 4:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, "q, k, v must be (batch, heads, seq_len, d)")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    pq = _dev_tensor(q, "q", q.dtype, (B, H, N, d))
    pk = _dev_tensor(k, "k", q.dtype, (B, Hkv, N, d))
    pv = _dev_tensor(v, "v", q.dtype, (B, Hkv, N, d))
    po = _dev_tensor(out, "out", q.dtype, (B, H, N, d))
    if lse is not None and lse is not False:
        lse_t = torch.empty(B, H, N, dtype=torch.float32, device=q.device) if lse is True else lse
        pl = _dev_tensor(lse_t, "lse", torch.float32, (B, H, N))
        with torch.cuda.device(q.device):
            _check(lib().attn_prefill_ex(pq, pk, pv, po, pl, B, H, Hkv, N, d, dt, int(bool(causal)), float(scale),
                                         _stream(q.device)))
        return out, lse_t
    with torch.cuda.device(q.device):
        st = _stream(q.device)
        if Hkv == H:
            _check(lib().attn_prefill(pq, pk, pv, po, B, H, N, d, dt, int(bool(causal)), float(scale), st))
        else:
            _check(lib().attn_prefill_gqa(pq, pk, pv, po, B, H, Hkv, N, d, dt, int(bool(causal)), float(scale), st))
    return out


def backward(q, k, v, out, dout, lse, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
             workspace=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for out, lse = prefill(q, k, v, causal, scale, lse=True).

    q, out, dout (B, H, N, d); k, v (B, Hkv, N, d); lse float32 (B, H, N); all GPU tensors.
    """
    if q.dim() != 4 or k.dim() != 4:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, "q, k, v must be (batch, heads, seq_len, d)")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ptrs = [_dev_tensor(t, n, q.dtype, (B, H, N, d)) for t, n in ((q, "q"),)]
    ptrs += [_dev_tensor(t, n, q.dtype, (B, Hkv, N, d)) for t, n in ((k, "k"), (v, "v"))]
    ptrs += [_dev_tensor(t, n, q.dtype, (B, H, N, d)) for t, n in ((out, "out"), (dout, "dout"))]
    ptrs += [_dev_tensor(lse, "lse", torch.float32, (B, H, N))]
    ptrs += [_dev_tensor(dq, "dq", q.dtype, (B, H, N, d))]
    ptrs += [_dev_tensor(t, n, q.dtype, (B, Hkv, N, d)) for t, n in ((dk, "dk"), (dv, "dv"))]
    wp, wb = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    with torch.cuda.device(q.device):
        _check(lib().attn_backward(*ptrs, B, H, Hkv, N, d, dt, int(bool(causal)), float(scale), wp, wb,
                                   _stream(q.device)))
    return dq, dk, dv


def backward_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib().attn_backward_workspace_bytes(B, H, N))


def decode(q, k_cache, v_cache, seq_lens, scale: float | None = None, out=None, chunk: int = 0, workspace=None,
           validate: bool = False):
    """One query row per (b, h) over the first seq_lens[b] cache rows.

    q (B, H, 1, d); caches (B, Hkv, max_len, d) with Hkv dividing H (grouped K/V heads
    when Hkv < H); seq_lens int32 GPU tensor (B,).
    ``chunk``/``workspace`` select attn_decode_ex (0 = automatic chunk; workspace a
    GPU tensor of at least decode_workspace_bytes bytes).  ``validate`` checks on the
    host that every length lies in [1, max_len] (a device-to-host copy).
    """
    if q.dim() != 4 or q.shape[2] != 1:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, "q must be (batch, heads, 1, d)")
    B, H, _, d = q.shape
    if k_cache.dim() != 4:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, "k_cache must be (batch, heads, max_len, d)")
    Hkv, max_len = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    pq = _dev_tensor(q, "q", q.dtype, (B, H, 1, d))
    pk = _dev_tensor(k_cache, "k_cache", q.dtype, (B, Hkv, max_len, d))
    pv = _dev_tensor(v_cache, "v_cache", q.dtype, (B, Hkv, max_len, d))
    pl = _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    po = _dev_tensor(out, "out", q.dtype, (B, H, 1, d))
    if validate:
        lens = seq_lens.cpu()
        if int(lens.min()) < 1 or int(lens.max()) > max_len:
            raise AttnValueError(ATTN_ERR_INVALID_ARG, f"seq_lens must lie in [1, {max_len}]")
    with torch.cuda.device(q.device):
        st = _stream(q.device)
        wp, wb = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        if workspace is not None and workspace.device.type != "cuda":
            raise AttnValueError(ATTN_ERR_INVALID_ARG, "workspace must be a GPU tensor")
        if Hkv != H:
            _check(lib().attn_decode_gqa(pq, pk, pv, pl, po, B, H, Hkv, max_len, d, dt, float(scale), int(chunk),
                                         wp or None, wb, st))
        elif chunk == 0 and workspace is None:
            _check(lib().attn_decode(pq, pk, pv, pl, po, B, H, max_len, d, dt, float(scale), st))
        else:
            _check(lib().attn_decode_ex(pq, pk, pv, pl, po, B, H, max_len, d, dt, float(scale), int(chunk),
                                        wp or None, wb, st))
    return out


def decode_noalloc(q, k_cache, v_cache, seq_lens, out, scale: float | None = None, chunk: int = 0):
    """attn_decode_noalloc: decode into ``out`` with the partials in the library's device
    scratch array (no allocation by the library, none here: ``out`` is required).
    Shapes as for decode; grouped K/V heads when k_cache has fewer heads than q."""
    if q.dim() != 4 or q.shape[2] != 1 or k_cache.dim() != 4:
        raise AttnValueError(ATTN_ERR_INVALID_ARG, "q must be (batch, heads, 1, d), caches (batch, heads, max_len, d)")
    B, H, _, d = q.shape
    Hkv, max_len = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    pq = _dev_tensor(q, "q", q.dtype, (B, H, 1, d))
    pk = _dev_tensor(k_cache, "k_cache", q.dtype, (B, Hkv, max_len, d))
    pv = _dev_tensor(v_cache, "v_cache", q.dtype, (B, Hkv, max_len, d))
    pl = _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    po = _dev_tensor(out, "out", q.dtype, (B, H, 1, d))
    with torch.cuda.device(q.device):
        _check(lib().attn_decode_noalloc(pq, pk, pv, pl, po, B, H, Hkv, max_len, d, dt, float(scale), int(chunk),
                                         _stream(q.device)))
    return out


def decode_split(q, k_cache, v_cache, seq_lens, scale, chunk: int, workspace):
    """attn_decode_split: the split pass alone; leaves the (m, l, acc) partials in
    ``workspace`` (a GPU tensor of at least decode_workspace_bytes bytes)."""
    B, H, _, d = q.shape
    Hkv, max_len = k_cache.shape[1], k_cache.shape[2]
    pq = _dev_tensor(q, "q", q.dtype, (B, H, 1, d))
    pk = _dev_tensor(k_cache, "k_cache", q.dtype, (B, Hkv, max_len, d))
    pv = _dev_tensor(v_cache, "v_cache", q.dtype, (B, Hkv, max_len, d))
    pl = _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    with torch.cuda.device(q.device):
        _check(lib().attn_decode_split(pq, pk, pv, pl, B, H, Hkv, max_len, d, _dtype_code(q), float(scale), int(chunk),
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(q.device)))


def decode_merge(workspace, out, max_len: int, chunk: int):
    """attn_decode_merge: the merge pass alone, from the partials decode_split left in
    ``workspace``, into ``out`` (B, H, 1, d)."""
    B, H, _, d = out.shape
    po = _dev_tensor(out, "out", out.dtype, (B, H, 1, d))
    with torch.cuda.device(out.device):
        _check(lib().attn_decode_merge(workspace.data_ptr(), workspace.numel() * workspace.element_size(), po, B, H,
                                       max_len, d, _dtype_code(out), int(chunk), _stream(out.device)))
    return out


def measure_read(buf, waves: int, sink):
    """attn_measure_read: a plain streaming read of the GPU tensor ``buf`` by ``waves``
    single-wave workgroups (measurement only); ``sink`` a GPU tensor of waves * 256 bytes."""
    with torch.cuda.device(buf.device):
        _check(lib().attn_measure_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(waves), sink.data_ptr(),
                                       sink.numel() * sink.element_size(), _stream(buf.device)))


def decode_choose_split(B: int, H: int, max_len: int, d: int, num_cus: int):
    """(chunk, n_split) the automatic decode split picks for a device with num_cus CUs."""
    c, n = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().attn_decode_choose_split(B, H, max_len, d, num_cus, ctypes.byref(c), ctypes.byref(n)))
    return c.value, n.value


def decode_gqa_choose_split(B: int, Hq: int, Hkv: int, max_len: int, d: int, num_cus: int):
    """(chunk, n_split) the automatic decode split picks with grouped K/V heads."""
    c, n = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().attn_decode_gqa_choose_split(B, Hq, Hkv, max_len, d, num_cus, ctypes.byref(c), ctypes.byref(n)))
    return c.value, n.value


def prefill_plan(B: int, H: int, N: int, d: int, causal: bool, num_cus: int) -> dict:
    """The workgroup form attn_prefill takes for this shape on a device with num_cus CUs:
    {"waves": waves per workgroup, "rows_per_wave": query rows per wave, "stages": K/V
    LDS stages, "key_groups": waves splitting each row block's keys}.  Host only."""
    w, r, s, g = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().attn_prefill_plan(B, H, N, d, int(bool(causal)), num_cus, ctypes.byref(w), ctypes.byref(r),
                                   ctypes.byref(s), ctypes.byref(g)))
    return {"waves": w.value, "rows_per_wave": r.value, "stages": s.value, "key_groups": g.value}


def decode_workspace_bytes(B: int, H: int, n_split: int, d: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, H, n_split, d))


def build_id() -> str:
    """The source identifier compiled into the loaded libattn.so (see build.source_hash)."""
    return lib().attn_build_id().decode()


def status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def last_error() -> str:
    return lib().attn_last_error().decode()
