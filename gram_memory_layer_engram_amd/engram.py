"""Thin ctypes binding over libengram.so.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI (``include/engram.h``). torch supplies device memory and the current HIP
stream. There is no fallback: without the built library or a GPU every call
raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EUNSUPPORTED, ENGRAM_EHIP, ENGRAM_ENOSPACE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 32 << 20
W_BF16, W_MXFP8 = 0, 1
FORWARD_STORE_KV = 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class ForwardArgs(ctypes.Structure):
    """Mirror of ``engram_forward_args``."""

    _fields_ = [
        ("table", _vp), ("num_rows", _i64),
        ("hash_ids", _vp), ("ids_stride_t", _i64), ("ids_stride_c", _i64),
        ("w", _vp), ("w_scales", _vp), ("w_format", _i32),
        ("hidden", _vp), ("q_weight", _vp), ("k_weight", _vp), ("token_mask", _vp),
        ("T", _i64), ("hc", _i32), ("dim", _i32), ("n_cols", _i32), ("head_dim", _i32),
        ("eps", _f32), ("clamp", _f32),
        ("out", _vp), ("gate_out", _vp), ("err_flag", _vp),
        ("table_scales", _vp), ("options", _i32),
    ]


EXPORTS = {
    "engram_abi_version": (_i32, []),
    "engram_status_string": (ctypes.c_char_p, [_i32]),
    "engram_lookup": (_i32, [_vp, _i64, _i32, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "engram_lookup_background": (_i32, [_vp, _i64, _i32, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "engram_host_alloc": (_i32, [_sz, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "engram_host_free": (_i32, [_vp]),
    "engram_lookup_fp8": (_i32, [_vp, _vp, _i64, _i32, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "engram_mx_quantize": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "engram_wkv_workspace_size": (_sz, [_i64, _i32, _i32, _i32]),
    "engram_wkv": (_i32, [_vp, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "engram_wkv_gate_partials": (_i32, [_vp, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp]),
    "engram_gate": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _f32, _f32, _vp, _vp, _vp]),
    "engram_gate_finish": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _f32, _f32, _vp, _vp, _vp]),
    "engram_forward_workspace_size": (_sz, [ctypes.POINTER(ForwardArgs)]),
    "engram_forward": (_i32, [ctypes.POINTER(ForwardArgs), _vp, _sz, _vp]),
    "engram_forward_single_launch": (_i32, [ctypes.POINTER(ForwardArgs), _vp, _sz, _vp]),
    "engram_forward_noalloc": (_i32, [ctypes.POINTER(ForwardArgs), _vp]),
    "engram_probe_out_bytes": (_sz, []),
    "engram_probe_mfma": (_i32, [_i32, _i32, _vp, ctypes.POINTER(ctypes.c_double), _vp]),
    "engram_probe_read": (_i32, [_vp, _sz, _vp, _vp]),
    "engram_probe_stream": (_i32, [_vp, _vp, _sz, _i32, _vp]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libengram.so and declare its exports (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m gram_memory_layer_engram_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class EngramError(RuntimeError):
    pass


def _check(status: int) -> None:
    if status != ENGRAM_OK:
        msg = load_library().engram_status_string(status).decode()
        cls = ValueError if status in (ENGRAM_EINVAL, ENGRAM_EUNSUPPORTED, ENGRAM_ENOSPACE) else EngramError
        raise cls(f"libengram: {msg} (status {status})")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, HostTable):
        return t.device_ptr
    if not t.is_cuda:
        raise ValueError("libengram takes device tensors only")
    return t.data_ptr()


class HostTable:
    """A bf16 table ``[num_rows, head_dim]`` in page-locked host memory
    mapped into the device's address space (engram_host_alloc): lookups and
    forwards given it read the rows over the host link. ``host`` is a CPU
    tensor on that memory for filling it (``copy_from`` copies a device
    table in); ``device_ptr`` is what the kernels read through. Freed by
    ``close()`` or when collected."""

    def __init__(self, num_rows: int, head_dim: int, dtype=torch.bfloat16):
        L = load_library()
        self.shape = (int(num_rows), int(head_dim))
        self.dtype = dtype
        nbytes = self.shape[0] * self.shape[1] * torch.empty((), dtype=dtype).element_size()
        h, d = _vp(), _vp()
        _check(L.engram_host_alloc(nbytes, ctypes.byref(h), ctypes.byref(d)))
        self._host_ptr = h.value
        self.device_ptr = d.value
        buf = (ctypes.c_uint8 * nbytes).from_address(self._host_ptr)
        self.host = torch.frombuffer(buf, dtype=torch.uint8).view(dtype).view(self.shape)

    def copy_from(self, table: torch.Tensor) -> "HostTable":
        if tuple(table.shape) != self.shape or table.dtype != self.dtype:
            raise ValueError(f"table must be {self.dtype} {self.shape}")
        self.host.copy_(table)
        return self

    def dim(self) -> int:
        return 2

    def close(self) -> None:
        if getattr(self, "_host_ptr", None):
            self.host = None
            _check(load_library().engram_host_free(self._host_ptr))
            self._host_ptr = None
            self.device_ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dense(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def lookup(table, hash_ids: torch.Tensor, rows_out: torch.Tensor | None = None,
           err_flag: torch.Tensor | None = None, background: bool = False) -> torch.Tensor:
    """rows[t, c, :] = table[hash_ids[t, c], :] (hash_ids may be strided).
    ``table`` is a device tensor or a HostTable; ``background`` selects
    engram_lookup_background (half the grid, for a side stream)."""
    L = load_library()
    if not isinstance(table, HostTable):
        _dense(table, "table")
    T, C = hash_ids.shape
    hd = table.shape[1]
    if hash_ids.dtype != torch.int32:
        raise ValueError("hash_ids must be int32")
    if rows_out is None:
        rows_out = torch.empty((T, C, hd), dtype=table.dtype, device=hash_ids.device)
    _dense(rows_out, "rows_out")
    fn = L.engram_lookup_background if background else L.engram_lookup
    _check(fn(_ptr(table), table.shape[0], hd, _ptr(hash_ids),
              hash_ids.stride(0), hash_ids.stride(1), T, C,
              _ptr(rows_out), _ptr(err_flag), _stream()))
    return rows_out


def lookup_fp8(table_codes: torch.Tensor, table_scales: torch.Tensor, hash_ids: torch.Tensor,
               rows_out: torch.Tensor | None = None, err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """rows[t, c, :] = bf16(e4m3(codes[id]) * 2^(scales[id, j/32] - 127)), id = hash_ids[t, c]."""
    L = load_library()
    _dense(table_codes, "table_codes")
    _dense(table_scales, "table_scales")
    T, C = hash_ids.shape
    hd = table_codes.shape[1]
    if hash_ids.dtype != torch.int32:
        raise ValueError("hash_ids must be int32")
    if table_codes.dtype != torch.uint8 or table_scales.dtype != torch.uint8:
        raise ValueError("fp8 table: uint8 codes and uint8 scale bytes")
    if tuple(table_scales.shape) != (table_codes.shape[0], hd // 32):
        raise ValueError("table_scales must be [num_rows, head_dim / 32]")
    if rows_out is None:
        rows_out = torch.empty((T, C, hd), dtype=torch.bfloat16, device=table_codes.device)
    _dense(rows_out, "rows_out")
    _check(L.engram_lookup_fp8(_ptr(table_codes), _ptr(table_scales), table_codes.shape[0], hd,
                               _ptr(hash_ids), hash_ids.stride(0), hash_ids.stride(1), T, C,
                               _ptr(rows_out), _ptr(err_flag), _stream()))
    return rows_out


def mx_quantize(x: torch.Tensor, xq: torch.Tensor | None = None, xs: torch.Tensor | None = None):
    """bf16 [T, K] -> (e4m3fn codes uint8 [T, K], E8M0 bytes uint8 [T, K/32])."""
    L = load_library()
    _dense(x, "x")
    T, K = x.shape
    if xq is None:
        xq = torch.empty((T, K), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((T, K // 32), dtype=torch.uint8, device=x.device)
    _check(L.engram_mx_quantize(_ptr(x), T, K, _ptr(xq), _ptr(xs), _stream()))
    return xq, xs


def wkv(x: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor | None = None,
        kv: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """kv = bf16(x . W^T); MXFP8 when ``w_scales`` is given (w = uint8 codes)."""
    L = load_library()
    _dense(x, "x")
    _dense(w, "w")
    T, K = x.shape
    N = w.shape[0]
    fmt = W_BF16 if w_scales is None else W_MXFP8
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w must be [N, {K}], got {tuple(w.shape)}")
    if fmt == W_MXFP8:
        _dense(w_scales, "w_scales")
        if w.dtype != torch.uint8 or tuple(w_scales.shape) != (N // 32, K // 32):
            raise ValueError("MXFP8 wkv needs uint8 codes [N, K] and scales [N/32, K/32]")
    elif w.dtype != torch.bfloat16 or x.dtype != torch.bfloat16:
        raise ValueError("bf16 wkv needs bf16 x and w")
    if kv is None:
        kv = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    need = L.engram_wkv_workspace_size(T, K, N, fmt)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(L.engram_wkv(_ptr(x), T, K, _ptr(w), _ptr(w_scales), fmt, N, _ptr(kv),
                        _ptr(workspace), ws_bytes, _stream()))
    return kv


def wkv_gate_partials(x: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor | None,
                      hidden: torch.Tensor, q_weight: torch.Tensor, k_weight: torch.Tensor,
                      value: torch.Tensor | None = None, partials: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """The projection fused with the gate's kv-side sums: returns (value
    [T, dim] bf16, partials [hc, T, dim/256, 2] fp32 = (sum hidden*q*k*key,
    sum key^2) per 256-column key tile). MXFP8 when ``w_scales`` is given."""
    L = load_library()
    for t, n in ((x, "x"), (w, "w"), (hidden, "hidden"), (q_weight, "q_weight"), (k_weight, "k_weight")):
        _dense(t, n)
    T, K = x.shape
    _, hc, dim = hidden.shape
    N = (hc + 1) * dim
    fmt = W_BF16 if w_scales is None else W_MXFP8
    if tuple(w.shape) != (N, K):
        raise ValueError(f"w must be [{N}, {K}], got {tuple(w.shape)}")
    if fmt == W_MXFP8:
        _dense(w_scales, "w_scales")
    if value is None:
        value = torch.empty((T, dim), dtype=torch.bfloat16, device=x.device)
    if partials is None:
        partials = torch.empty((hc, T, max(1, dim // 256), 2), dtype=torch.float32, device=x.device)
    if tuple(value.shape) != (T, dim) or value.dtype != torch.bfloat16:
        raise ValueError(f"value must be bf16 [{T}, {dim}]")
    if tuple(partials.shape) != (hc, T, max(1, dim // 256), 2) or partials.dtype != torch.float32:
        raise ValueError(f"partials must be fp32 [{hc}, {T}, {dim // 256}, 2]")
    _dense(value, "value")
    _dense(partials, "partials")
    need = L.engram_wkv_workspace_size(T, K, N, fmt)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(L.engram_wkv_gate_partials(_ptr(x), T, K, _ptr(w), _ptr(w_scales), fmt, hc, dim, _ptr(hidden),
                                      _ptr(q_weight), _ptr(k_weight), _ptr(value), _ptr(partials),
                                      _ptr(workspace), ws_bytes, _stream()))
    return value, partials


def gate_finish(hidden: torch.Tensor, value: torch.Tensor, partials: torch.Tensor,
                token_mask: torch.Tensor | None = None, eps: float = 1e-6, clamp: float = 1e-6,
                out: torch.Tensor | None = None, gate_out: torch.Tensor | None = None) -> torch.Tensor:
    """The gate and update from wkv_gate_partials' value and partials."""
    L = load_library()
    for t, n in ((hidden, "hidden"), (value, "value"), (partials, "partials")):
        _dense(t, n)
    T, hc, dim = hidden.shape
    if tuple(partials.shape) != (hc, T, max(1, dim // 256), 2) or partials.dtype != torch.float32:
        raise ValueError(f"partials must be fp32 [{hc}, {T}, {dim // 256}, 2]")
    if out is None:
        out = torch.empty_like(hidden)
    _check(L.engram_gate_finish(_ptr(hidden), _ptr(value), _ptr(partials), _ptr(token_mask), T, hc, dim,
                                eps, clamp, _ptr(out), _ptr(gate_out), _stream()))
    return out


def gate(hidden: torch.Tensor, kv: torch.Tensor, q_weight: torch.Tensor, k_weight: torch.Tensor,
         token_mask: torch.Tensor | None = None, eps: float = 1e-6, clamp: float = 1e-6,
         out: torch.Tensor | None = None, gate_out: torch.Tensor | None = None) -> torch.Tensor:
    """out = hidden + sigmoid(signed-sqrt(normalized dot)) * value, masked rows copied."""
    L = load_library()
    for t, n in ((hidden, "hidden"), (kv, "kv"), (q_weight, "q_weight"), (k_weight, "k_weight")):
        _dense(t, n)
    T, hc, dim = hidden.shape
    if out is None:
        out = torch.empty_like(hidden)
    _check(L.engram_gate(_ptr(hidden), _ptr(kv), _ptr(q_weight), _ptr(k_weight),
                         _ptr(token_mask), T, hc, dim, eps, clamp, _ptr(out),
                         _ptr(gate_out), _stream()))
    return out


def forward_args(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask,
                 eps, clamp, out, gate_out=None, err_flag=None, table_scales=None,
                 store_kv=False) -> ForwardArgs:
    T, hc, dim = hidden.shape
    a = ForwardArgs()
    a.table = _ptr(table); a.num_rows = table.shape[0]
    a.hash_ids = _ptr(hash_ids)
    a.ids_stride_t = hash_ids.stride(0); a.ids_stride_c = hash_ids.stride(1)
    a.w = _ptr(w); a.w_scales = _ptr(w_scales)
    a.w_format = W_BF16 if w_scales is None else W_MXFP8
    a.hidden = _ptr(hidden); a.q_weight = _ptr(q_weight); a.k_weight = _ptr(k_weight)
    a.token_mask = _ptr(token_mask)
    a.T = T; a.hc = hc; a.dim = dim
    a.n_cols = hash_ids.shape[1]; a.head_dim = table.shape[1]
    a.eps = eps; a.clamp = clamp
    a.out = _ptr(out); a.gate_out = _ptr(gate_out); a.err_flag = _ptr(err_flag)
    if table_scales is not None:
        _dense(table_scales, "table_scales")
        if table.dtype != torch.uint8 or tuple(table_scales.shape) != (table.shape[0], table.shape[1] // 32):
            raise ValueError("fp8 table: uint8 codes [rows, hd] and scales [rows, hd / 32]")
    a.table_scales = _ptr(table_scales)
    a.options = FORWARD_STORE_KV if store_kv else 0
    return a


def forward_workspace_size(args: ForwardArgs) -> int:
    return load_library().engram_forward_workspace_size(ctypes.byref(args))


def forward(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask=None,
            eps=1e-6, clamp=1e-6, out=None, gate_out=None, err_flag=None, workspace=None,
            single_launch=False, table_scales=None, store_kv=False):
    """One Engram layer forward: lookup -> (MXFP8 quantize) -> wkv -> gate.
    ``single_launch`` selects engram_forward_single_launch (decode shapes);
    ``table_scales`` makes ``table`` an fp8 table (uint8 e4m3 codes);
    ``store_kv`` sets ENGRAM_FORWARD_STORE_KV: kv is stored whole and the
    plain gate reads it, instead of the default where the tiled GEMM reduces
    key tiles to the gate's partial sums and stores only the value."""
    L = load_library()
    for t, n in ((table, "table"), (w, "w"), (hidden, "hidden"),
                 (q_weight, "q_weight"), (k_weight, "k_weight")):
        if not isinstance(t, HostTable):
            _dense(t, n)
    if out is None:
        out = torch.empty_like(hidden)
    args = forward_args(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask,
                        eps, clamp, out, gate_out, err_flag, table_scales, store_kv)
    need = L.engram_forward_workspace_size(ctypes.byref(args))
    if workspace is None and need:
        workspace = new_forward_workspace(need, hidden.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    fn = L.engram_forward_single_launch if single_launch else L.engram_forward
    _check(fn(ctypes.byref(args), _ptr(workspace), ws_bytes, _stream()))
    return out


def forward_noalloc(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask=None,
                    eps=1e-6, clamp=1e-6, out=None, gate_out=None, err_flag=None, table_scales=None,
                    store_kv=False):
    """engram_forward_noalloc: the forward on the library's fixed device
    scratch (no workspace argument; ValueError when the input needs more than
    NOALLOC_SCRATCH_BYTES). ``out`` is allocated here when not given."""
    L = load_library()
    for t, n in ((table, "table"), (w, "w"), (hidden, "hidden"),
                 (q_weight, "q_weight"), (k_weight, "k_weight")):
        if not isinstance(t, HostTable):
            _dense(t, n)
    if out is None:
        out = torch.empty_like(hidden)
    args = forward_args(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask,
                        eps, clamp, out, gate_out, err_flag, table_scales, store_kv)
    _check(L.engram_forward_noalloc(ctypes.byref(args), _stream()))
    return out


def new_forward_workspace(nbytes: int, device) -> torch.Tensor:
    """A forward workspace: its leading 64 KiB of flags start at zero (every
    call leaves them zero again), so it is allocated zeroed once."""
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


class ForwardPlan:
    """A prepared forward: arguments are marshalled once and ``run()`` is a
    single C call (for decode loops, where per-call Python work would
    otherwise dominate). The plan keeps its tensors alive; change their
    contents in place between runs, not their storage."""

    def __init__(self, table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask=None,
                 eps=1e-6, clamp=1e-6, out=None, gate_out=None, err_flag=None, workspace=None,
                 stream=None, single_launch=False, table_scales=None, store_kv=False):
        L = load_library()
        for t, n in ((table, "table"), (w, "w"), (hidden, "hidden"),
                     (q_weight, "q_weight"), (k_weight, "k_weight")):
            if not isinstance(t, HostTable):
                _dense(t, n)
        if out is None:
            out = torch.empty_like(hidden)
        self.out = out
        self._keep = (table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask, gate_out,
                      err_flag, table_scales)
        self.args = forward_args(table, hash_ids, w, w_scales, hidden, q_weight, k_weight, token_mask,
                                 eps, clamp, out, gate_out, err_flag, table_scales, store_kv)
        need = L.engram_forward_workspace_size(ctypes.byref(self.args))
        if workspace is None and need:
            workspace = new_forward_workspace(need, hidden.device)
        self.workspace = workspace
        self._ws = _ptr(workspace)
        self._ws_bytes = 0 if workspace is None else workspace.numel()
        self._argp = ctypes.byref(self.args)
        self._fn = L.engram_forward_single_launch if single_launch else L.engram_forward
        self._stream = (torch.cuda.current_stream() if stream is None else stream).cuda_stream

    def run(self):
        status = self._fn(self._argp, self._ws, self._ws_bytes, self._stream)
        if status:
            _check(status)
        return self.out


# ------------------------------------------------------ measurement probes --


def probe_out(device="cuda") -> torch.Tensor:
    """Device words for the probes' per-thread results."""
    n = load_library().engram_probe_out_bytes() // 4
    return torch.empty(n, dtype=torch.int32, device=device)


def probe_mfma(w_format: int, iters: int, out: torch.Tensor) -> float:
    """Enqueue the register-only MFMA loop (bf16 or MXFP8); returns the flops
    it launches. ``out`` from ``probe_out``."""
    flops = ctypes.c_double(0.0)
    _check(load_library().engram_probe_mfma(w_format, iters, _ptr(out), ctypes.byref(flops), _stream()))
    return flops.value


def probe_read(buf: torch.Tensor, out: torch.Tensor) -> None:
    """Enqueue a streaming read of ``buf`` (dense, a multiple of 16 bytes)."""
    _dense(buf, "buf")
    _check(load_library().engram_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream()))


def probe_stream(src: torch.Tensor, dst: torch.Tensor, reads_per_write: int = 1) -> None:
    """Enqueue the R:1 streaming probe: dst (16-byte pieces) = XOR of
    ``reads_per_write`` consecutive dst-sized blocks of src (1 = a copy)."""
    _dense(src, "src")
    _dense(dst, "dst")
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != reads_per_write * nbytes:
        raise ValueError("probe_stream: src must hold reads_per_write times dst's bytes")
    _check(load_library().engram_probe_stream(_ptr(src), _ptr(dst), nbytes, reads_per_write, _stream()))
