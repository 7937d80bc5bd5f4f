"""MI355X-native MoE / gated-MLP FFN hot path: Python binding of libmoeffn.so.

Each function has the name of the C entry point it calls (see
``include/moeffn.h``) and does argument marshalling only: it checks the
tensors' device, dtype, shape and contiguity, allocates outputs that were not
passed in (torch supplies device memory), and passes raw pointers and the
current HIP stream to the library. Every step of the computation runs in the
library's HIP kernels; nothing here computes, and there is no fallback.

Weights are given [out_features, in_features]: w_gate / w_up are
[E, f, d] and w_down is [E, d, f] (the transpose of the pages' W in Y = X W),
and are packed once with ``pack_weights`` into the MFMA fragment order the
GEMMs read; the GEMM calls take the ``PackedWeights`` it returns.
"""

from __future__ import annotations

import ctypes
from typing import NamedTuple, Optional

import torch

from . import _lib

MF_F32, MF_BF16, MF_FP8_E4M3 = 0, 1, 2

_lib.load()  # fail loudly at import if the HIP library is missing

__all__ = [
    "MoEFFNError", "PackedWeights", "pack_weights", "pack_weights_kn", "rmsnorm", "rmsnorm_quantize_fp8",
    "moe_route_workspace_size",
    "moe_route",
    "moe_permute_workspace_size", "moe_permute", "moe_permute_noalloc", "moe_dispatch_masked", "MaskedDispatch",
    "grouped_gate_up_masked", "grouped_down_masked", "quantize_fp8_rows", "grouped_gate_up_a8",
    "grouped_down_a8",
    "grouped_swiglu", "grouped_gate_up", "grouped_down", "moe_combine", "tp_shard_mlp", "PermuteResult", "MoEFFNLayer",
    "version",
]


class MoEFFNError(RuntimeError):
    """A libmoeffn call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        msg = _lib.load().mf_status_string(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def version() -> str:
    return _lib.load().mf_version().decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MF_BF16
    if dt == torch.float32:
        return MF_F32
    if dt == torch.float8_e4m3fn:
        return MF_FP8_E4M3
    raise ValueError(f"unsupported dtype {dt}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(*ts: Optional[torch.Tensor]) -> None:
    cur = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libmoeffn takes device tensors only")
        if not t.is_contiguous():
            raise ValueError("libmoeffn takes contiguous tensors only")
        cur = torch.cuda.current_device() if cur is None else cur
        if t.device.index != cur:
            raise ValueError(f"libmoeffn: tensors must be on the current device (cuda:{cur}), "
                             f"got {t.device}")


def _need(name: str, what: str, t: Optional[torch.Tensor], shape, dtype) -> None:
    """t (if given) must have exactly `shape` and `dtype`: the kernels write and
    read whole buffers of those sizes, with no size passed for most of them."""
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: {what} must be {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _ok(name: str, status: int) -> None:
    if status != 0:
        raise MoEFFNError(name, status)


# --------------------------------------------------------------------------


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = gamma * x / sqrt(mean(x^2) + eps) over the last dim (bf16 or f32)."""
    if out is None:
        out = torch.empty_like(x)
    _dev(x, gamma, out)
    if x.dim() != 2:
        raise ValueError("rmsnorm: x [T, d], gamma [d], out [T, d] of one dtype")
    T, d = x.shape
    _need("rmsnorm", "gamma", gamma, (d,), x.dtype)
    _need("rmsnorm", "out", out, (T, d), x.dtype)
    _ok("rmsnorm", _lib.load().rmsnorm(_p(x), _p(gamma), _p(out), T, d, eps,
                                       _dtype_code(x.dtype), _s(stream)))
    return out


def rmsnorm_quantize_fp8(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5, *,
                         out: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                         scales: Optional[torch.Tensor] = None, stream=None):
    """rmsnorm (bf16) plus, in the same pass, quantize_fp8_rows of its output.
    Returns (y bf16 [T, d], q uint8 [T, d], scales f32 [T, d/128])."""
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("rmsnorm_quantize_fp8: x must be bf16 [T, d]")
    T, d = x.shape
    out = torch.empty_like(x) if out is None else out
    q = torch.empty((T, d), dtype=torch.uint8, device=x.device) if q is None else q
    if scales is None:
        scales = torch.empty((T, max(d // 128, 0)), dtype=torch.float32, device=x.device)
    n = "rmsnorm_quantize_fp8"
    _need(n, "gamma", gamma, (d,), torch.bfloat16)
    _need(n, "out", out, (T, d), torch.bfloat16)
    _need(n, "q", q, (T, d), torch.uint8)
    _need(n, "scales", scales, (T, max(d // 128, 0)), torch.float32)
    _dev(x, gamma, out, q, scales)
    _ok(n, _lib.load().rmsnorm_quantize_fp8(_p(x), _p(gamma), _p(out), _p(q), _p(scales), T, d,
                                            eps, _s(stream)))
    return out, q, scales


class PackedWeights(NamedTuple):
    """Weights [groups, N, K] rearranged by pack_weights (flat bytes on the device)."""
    data: torch.Tensor   # uint8, packed_weights_bytes(groups, N, K, dtype) bytes
    dtype: torch.dtype   # torch.bfloat16 or torch.float8_e4m3fn
    groups: int
    N: int
    K: int


def pack_weights(w: torch.Tensor, stream=None) -> PackedWeights:
    """Pack w ([groups, N, K] or [N, K], bf16 or float8_e4m3fn) for the GEMM calls."""
    w3 = w.unsqueeze(0) if w.dim() == 2 else w
    G, N, K = w3.shape
    code = _dtype_code(w3.dtype)
    nbytes = int(_lib.load().packed_weights_bytes(G, N, K, code))
    if nbytes == 0:
        raise ValueError(f"pack_weights: unsupported shape/dtype {tuple(w3.shape)} {w3.dtype}")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w3.device)
    _dev(w3, out)
    _ok("pack_weights", _lib.load().pack_weights(_p(w3), _p(out), G, N, K, code, _s(stream)))
    return PackedWeights(out, w3.dtype, G, N, K)


def pack_weights_kn(w: torch.Tensor, stream=None) -> PackedWeights:
    """Pack w stored [groups, K, N] or [K, N] ([in, out], Y = X W): the same bytes as
    pack_weights of its transpose."""
    w3 = w.unsqueeze(0) if w.dim() == 2 else w
    G, K, N = w3.shape
    code = _dtype_code(w3.dtype)
    nbytes = int(_lib.load().packed_weights_bytes(G, N, K, code))
    if nbytes == 0:
        raise ValueError(f"pack_weights_kn: unsupported shape/dtype {tuple(w3.shape)} {w3.dtype}")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w3.device)
    _dev(w3, out)
    _ok("pack_weights_kn", _lib.load().pack_weights_kn(_p(w3), _p(out), G, N, K, code, _s(stream)))
    return PackedWeights(out, w3.dtype, G, N, K)


def _pw(w, name: str) -> PackedWeights:
    if not isinstance(w, PackedWeights):
        raise TypeError(f"{name}: pass weights packed by pack_weights()")
    _dev(w.data)
    return w


def moe_route_workspace_size(T: int, d: int, E: int) -> int:
    return int(_lib.load().moe_route_workspace_size(T, d, E))


def moe_route(x: torch.Tensor, w_r: torch.Tensor, bias: torch.Tensor, k: int = 8,
              topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """Sigmoid-with-bias top-k router: returns (topk_idx [T,k] int32 ascending, topk_w [T,k] f32)."""
    T, d = x.shape
    w_r = _pw(w_r, "moe_route")
    E = w_r.N
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(1, moe_route_workspace_size(T, d, E)), dtype=torch.uint8,
                                device=x.device)
    _dev(x, bias, topk_idx, topk_w, workspace)
    if x.dtype != torch.bfloat16 or w_r.dtype != torch.bfloat16 or bias.dtype != torch.float32:
        raise ValueError("moe_route: x, w_r bf16 and bias f32")
    if w_r.groups != 1 or w_r.K != d or tuple(bias.shape) != (E,):
        raise ValueError("moe_route: w_r [E, d], bias [E]")
    _need("moe_route", "topk_idx", topk_idx, (T, k), torch.int32)
    _need("moe_route", "topk_w", topk_w, (T, k), torch.float32)
    _ok("moe_route", _lib.load().moe_route(
        _p(x), _p(w_r.data), _p(bias), T, d, E, k, _p(topk_idx), _p(topk_w), _p(workspace),
        workspace.numel() * workspace.element_size(), _s(stream)))
    return topk_idx, topk_w


def moe_permute_workspace_size(T: int, k: int, e_count: int) -> int:
    return int(_lib.load().moe_permute_workspace_size(T, k, e_count))


class PermuteResult(NamedTuple):
    counts: torch.Tensor     # [e_count] int32
    offsets: torch.Tensor    # [e_count+1] int32
    src_token: torch.Tensor  # [T*k] int32 (first offsets[-1] valid)
    inv_pos: torch.Tensor    # [T, k] int32, -1 = non-local
    x_perm: Optional[torch.Tensor]  # [T*k, d] (first offsets[-1] rows valid)


def moe_permute(topk_idx: torch.Tensor, e_begin: int, e_count: int,
                x: Optional[torch.Tensor] = None, *, x_perm: Optional[torch.Tensor] = None,
                counts=None, offsets=None, src_token=None, inv_pos=None, workspace=None,
                stream=None) -> PermuteResult:
    """Stable counting sort of routing slots by local expert (+ row gather when x is given)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    i32 = torch.int32
    counts = torch.empty(e_count, dtype=i32, device=dev) if counts is None else counts
    offsets = torch.empty(e_count + 1, dtype=i32, device=dev) if offsets is None else offsets
    src_token = torch.empty(T * k, dtype=i32, device=dev) if src_token is None else src_token
    inv_pos = torch.empty((T, k), dtype=i32, device=dev) if inv_pos is None else inv_pos
    need = moe_permute_workspace_size(T, k, e_count)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    d, xdt = 0, MF_BF16
    if x is not None:
        d = x.shape[1]
        xdt = _dtype_code(x.dtype)
        if x_perm is None:
            x_perm = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    _dev(topk_idx, x, x_perm, counts, offsets, src_token, inv_pos, workspace)
    if topk_idx.dtype != i32:
        raise ValueError("moe_permute: topk_idx must be int32")
    for what, t, shape in (("counts", counts, (e_count,)), ("offsets", offsets, (e_count + 1,)),
                           ("src_token", src_token, (T * k,)), ("inv_pos", inv_pos, (T, k))):
        _need("moe_permute", what, t, shape, i32)
    if x is not None:
        _need("moe_permute", "x", x, (T, d), x.dtype)
        _need("moe_permute", "x_perm", x_perm, (T * k, d), x.dtype)
    _ok("moe_permute", _lib.load().moe_permute(
        _p(topk_idx), T, k, e_begin, e_count, _p(x), d, xdt, _p(x_perm), _p(counts),
        _p(offsets), _p(src_token), _p(inv_pos), _p(workspace),
        workspace.numel() * workspace.element_size(), _s(stream)))
    return PermuteResult(counts, offsets, src_token, inv_pos, x_perm)


def moe_permute_noalloc(topk_idx: torch.Tensor, e_begin: int, e_count: int,
                        x: Optional[torch.Tensor] = None, *, x_perm: torch.Tensor,
                        counts: torch.Tensor, offsets: torch.Tensor, src_token: torch.Tensor,
                        inv_pos: torch.Tensor, stream=None) -> PermuteResult:
    """moe_permute through the allocation-free entry point: every output buffer
    is the caller's (nothing is allocated here or in the library; the count
    tables live in the library's static device array). ``x_perm`` may be None
    only when ``x`` is None (indices only)."""
    T, k = topk_idx.shape
    i32 = torch.int32
    if topk_idx.dtype != i32:
        raise ValueError("moe_permute_noalloc: topk_idx must be int32")
    for what, t, shape in (("counts", counts, (e_count,)), ("offsets", offsets, (e_count + 1,)),
                           ("src_token", src_token, (T * k,)), ("inv_pos", inv_pos, (T, k))):
        if t is None:
            raise ValueError(f"moe_permute_noalloc: {what} is required")
        _need("moe_permute_noalloc", what, t, shape, i32)
    d, xdt = 0, MF_BF16
    if x is not None:
        d = x.shape[1]
        xdt = _dtype_code(x.dtype)
        if x_perm is None:
            raise ValueError("moe_permute_noalloc: x_perm is required with x")
        _need("moe_permute_noalloc", "x", x, (T, d), x.dtype)
        _need("moe_permute_noalloc", "x_perm", x_perm, (T * k, d), x.dtype)
    _dev(topk_idx, x, x_perm, counts, offsets, src_token, inv_pos)
    _ok("moe_permute_noalloc", _lib.load().moe_permute_noalloc(
        _p(topk_idx), T, k, e_begin, e_count, _p(x), d, xdt, _p(x_perm), _p(counts),
        _p(offsets), _p(src_token), _p(inv_pos), _s(stream)))
    return PermuteResult(counts, offsets, src_token, inv_pos, x_perm)


class MaskedDispatch(NamedTuple):
    counts: torch.Tensor     # [e_count] int32: rows used per expert block
    row_index: torch.Tensor  # [e_count * cap] int32: token of each used row
    pos: torch.Tensor        # [T, k] int32: row of each slot or -1
    cap: int


def moe_dispatch_masked(topk_idx: torch.Tensor, e_begin: int, e_count: int, cap: int, *,
                        counts=None, row_index=None, pos=None, workspace=None,
                        stream=None) -> MaskedDispatch:
    """Masked (fixed-capacity) layout: slot (t, j) of local expert e -> row e*cap + rank."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    i32 = torch.int32
    counts = torch.empty(e_count, dtype=i32, device=dev) if counts is None else counts
    row_index = torch.empty(e_count * cap, dtype=i32, device=dev) if row_index is None else row_index
    pos = torch.empty((T, k), dtype=i32, device=dev) if pos is None else pos
    need = moe_permute_workspace_size(T, k, e_count)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(topk_idx, counts, row_index, pos, workspace)
    if topk_idx.dtype != i32:
        raise ValueError("moe_dispatch_masked: topk_idx must be int32")
    for what, t, shape in (("counts", counts, (e_count,)), ("row_index", row_index, (e_count * cap,)),
                           ("pos", pos, (T, k))):
        _need("moe_dispatch_masked", what, t, shape, i32)
    _ok("moe_dispatch_masked", _lib.load().moe_dispatch_masked(
        _p(topk_idx), T, k, e_begin, e_count, cap, _p(counts), _p(row_index), _p(pos),
        _p(workspace), workspace.numel() * workspace.element_size(), _s(stream)))
    return MaskedDispatch(counts, row_index, pos, cap)


def grouped_gate_up_masked(x: torch.Tensor, row_index: torch.Tensor, counts: torch.Tensor,
                           cap: int, w_gate, w_up, s_gate=None, s_up=None, *, h_out=None,
                           stream=None) -> torch.Tensor:
    """grouped_gate_up over the masked layout (rows V[row_index], blocks of cap). Returns h_out."""
    src_rows, d = x.shape
    w_gate, w_up = _pw(w_gate, "grouped_gate_up_masked"), _pw(w_up, "grouped_gate_up_masked")
    e_count, f = w_gate.groups, w_gate.N
    if w_gate.K != d or (w_up.groups, w_up.N, w_up.K) != (e_count, f, d):
        raise ValueError("grouped_gate_up_masked: w_gate/w_up [E, f, d]")
    n = "grouped_gate_up_masked"
    _need(n, "x", x, (src_rows, d), torch.bfloat16)
    _need(n, "row_index", row_index, (e_count * cap,), torch.int32)
    _need(n, "counts", counts, (e_count,), torch.int32)
    wdt = _grouped_dtype(w_gate, w_up)
    _block_scales(n, wdt, e_count, f, d, s_gate=s_gate, s_up=s_up)
    if h_out is None:
        h_out = torch.empty((e_count * cap, f), dtype=torch.bfloat16, device=x.device)
    _need(n, "h_out", h_out, (e_count * cap, f), torch.bfloat16)
    _dev(x, row_index, counts, s_gate, s_up, h_out)
    _ok("grouped_gate_up_masked", _lib.load().grouped_gate_up_masked(
        _p(x), _p(row_index), src_rows, _p(counts), cap, e_count, d, f, _p(w_gate.data),
        _p(w_up.data), wdt, _p(s_gate), _p(s_up), _p(h_out), _s(stream)))
    return h_out


def grouped_down_masked(h: torch.Tensor, counts: torch.Tensor, cap: int, w_down, s_down=None, *,
                        y_perm=None, stream=None) -> torch.Tensor:
    """grouped_down over the masked layout. Returns y_perm [E*cap, d]."""
    rows, f = h.shape
    w_down = _pw(w_down, "grouped_down_masked")
    e_count, d = w_down.groups, w_down.N
    if w_down.K != f or rows != e_count * cap:
        raise ValueError("grouped_down_masked: h [E*cap, f], w_down [E, d, f]")
    n = "grouped_down_masked"
    _need(n, "h", h, (rows, f), torch.bfloat16)
    _need(n, "counts", counts, (e_count,), torch.int32)
    wdt = _grouped_dtype(w_down)
    _block_scales(n, wdt, e_count, d, f, s_down=s_down)
    if y_perm is None:
        y_perm = torch.empty((rows, d), dtype=torch.bfloat16, device=h.device)
    _need(n, "y_perm", y_perm, (rows, d), torch.bfloat16)
    _dev(h, counts, s_down, y_perm)
    _ok("grouped_down_masked", _lib.load().grouped_down_masked(
        _p(h), _p(counts), cap, e_count, f, d, _p(w_down.data), wdt, _p(s_down), _p(y_perm),
        _s(stream)))
    return y_perm


def _block_scales(name: str, wdt: int, e_count: int, N: int, K: int, **scales) -> None:
    """fp8 weights need their [e_count, N/128, K/128] f32 block scales."""
    if wdt != MF_FP8_E4M3:
        return
    for what, t in scales.items():
        if t is None:
            raise ValueError(f"{name}: fp8 weights need {what}")
        _need(name, what, t, (e_count, N // 128, K // 128), torch.float32)


def _grouped_rows(x: torch.Tensor, row_index, name: str):
    """(max_rows, src_rows) of a grouped call: x is X_perm, or with row_index
    the un-permuted rows that row_index (moe_permute's src_token) gathers."""
    if row_index is None:
        return x.shape[0], 0
    if row_index.dtype != torch.int32 or row_index.dim() != 1:
        raise ValueError(f"{name}: row_index must be a 1-D int32 tensor")
    return row_index.numel(), x.shape[0]


def grouped_swiglu(x_perm: torch.Tensor, offsets: torch.Tensor, w_gate: torch.Tensor,
                   w_up: torch.Tensor, w_down: torch.Tensor, s_gate=None, s_up=None,
                   s_down=None, *, row_index=None, h_work=None, y_perm=None, stream=None):
    """Grouped expert gated MLPs over expert-contiguous rows. Returns (y_perm, h_work).

    With ``row_index`` (moe_permute's src_token), ``x_perm`` is the un-permuted
    input and row r of the grouped input is ``x_perm[row_index[r]]``."""
    max_rows, src_rows = _grouped_rows(x_perm, row_index, "grouped_swiglu")
    d = x_perm.shape[1]
    w_gate, w_up, w_down = (_pw(w, "grouped_swiglu") for w in (w_gate, w_up, w_down))
    e_count, f, d2 = w_gate.groups, w_gate.N, w_gate.K
    if (d2 != d or (w_up.groups, w_up.N, w_up.K) != (e_count, f, d)
            or (w_down.groups, w_down.N, w_down.K) != (e_count, d, f)):
        raise ValueError("grouped_swiglu: w_gate/w_up [E, f, d], w_down [E, d, f]")
    n = "grouped_swiglu"
    _need(n, "offsets", offsets, (e_count + 1,), torch.int32)
    _need(n, "x_perm", x_perm, (x_perm.shape[0], d), torch.bfloat16)
    wdt = _grouped_dtype(w_gate, w_up, w_down)
    _block_scales(n, wdt, e_count, f, d, s_gate=s_gate, s_up=s_up)
    _block_scales(n, wdt, e_count, d, f, s_down=s_down)
    if h_work is None:
        h_work = torch.empty((max_rows, f), dtype=torch.bfloat16, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((max_rows, d), dtype=torch.bfloat16, device=x_perm.device)
    _need(n, "h_work", h_work, (max_rows, f), torch.bfloat16)
    _need(n, "y_perm", y_perm, (max_rows, d), torch.bfloat16)
    _dev(x_perm, row_index, offsets, s_gate, s_up, s_down, h_work, y_perm)
    _ok("grouped_swiglu", _lib.load().grouped_swiglu(
        _p(x_perm), _p(row_index), src_rows, _p(offsets), e_count, max_rows, d, f,
        _p(w_gate.data), _p(w_up.data),
        _p(w_down.data), wdt,
        _p(s_gate), _p(s_up), _p(s_down), _p(h_work), _p(y_perm), _s(stream)))
    return y_perm, h_work


def _grouped_dtype(w_gate: PackedWeights, *rest: PackedWeights) -> int:
    wdt = _dtype_code(w_gate.dtype)
    if any(w.dtype != w_gate.dtype for w in rest):
        raise ValueError("grouped GEMM: one weight dtype")
    if wdt == MF_F32:
        raise ValueError("grouped GEMM: weights are bf16 or float8_e4m3fn")
    return wdt


def grouped_gate_up(x_perm: torch.Tensor, offsets: torch.Tensor, w_gate: torch.Tensor,
                    w_up: torch.Tensor, s_gate=None, s_up=None, *, row_index=None, h_out=None,
                    stream=None) -> torch.Tensor:
    """H = SiLU(X_perm W_gate_e) * (X_perm W_up_e) per expert segment. Returns h_out.

    ``row_index`` as in grouped_swiglu (the gather fused into the A load)."""
    max_rows, src_rows = _grouped_rows(x_perm, row_index, "grouped_gate_up")
    d = x_perm.shape[1]
    w_gate, w_up = _pw(w_gate, "grouped_gate_up"), _pw(w_up, "grouped_gate_up")
    e_count, f = w_gate.groups, w_gate.N
    if w_gate.K != d or (w_up.groups, w_up.N, w_up.K) != (e_count, f, d):
        raise ValueError("grouped_gate_up: w_gate/w_up [E, f, d]")
    n = "grouped_gate_up"
    _need(n, "offsets", offsets, (e_count + 1,), torch.int32)
    _need(n, "x_perm", x_perm, (x_perm.shape[0], d), torch.bfloat16)
    wdt = _grouped_dtype(w_gate, w_up)
    _block_scales(n, wdt, e_count, f, d, s_gate=s_gate, s_up=s_up)
    if h_out is None:
        h_out = torch.empty((max_rows, f), dtype=torch.bfloat16, device=x_perm.device)
    _need(n, "h_out", h_out, (max_rows, f), torch.bfloat16)
    _dev(x_perm, row_index, offsets, s_gate, s_up, h_out)
    _ok("grouped_gate_up", _lib.load().grouped_gate_up(
        _p(x_perm), _p(row_index), src_rows, _p(offsets), e_count, max_rows, d, f,
        _p(w_gate.data), _p(w_up.data), wdt, _p(s_gate), _p(s_up), _p(h_out), _s(stream)))
    return h_out


def grouped_down(h: torch.Tensor, offsets: torch.Tensor, w_down: torch.Tensor, s_down=None, *,
                 y_perm=None, stream=None) -> torch.Tensor:
    """Y_perm = H W_down_e per expert segment. Returns y_perm."""
    max_rows, f = h.shape
    w_down = _pw(w_down, "grouped_down")
    e_count, d = w_down.groups, w_down.N
    if w_down.K != f:
        raise ValueError("grouped_down: w_down [E, d, f]")
    n = "grouped_down"
    _need(n, "offsets", offsets, (e_count + 1,), torch.int32)
    _need(n, "h", h, (max_rows, f), torch.bfloat16)
    wdt = _grouped_dtype(w_down)
    _block_scales(n, wdt, e_count, d, f, s_down=s_down)
    if y_perm is None:
        y_perm = torch.empty((max_rows, d), dtype=torch.bfloat16, device=h.device)
    _need(n, "y_perm", y_perm, (max_rows, d), torch.bfloat16)
    _dev(h, offsets, s_down, y_perm)
    _ok("grouped_down", _lib.load().grouped_down(
        _p(h), _p(offsets), e_count, max_rows, f, d, _p(w_down.data), wdt, _p(s_down), _p(y_perm),
        _s(stream)))
    return y_perm


def quantize_fp8_rows(x: torch.Tensor, *, row_count=None, q=None, scales=None, stream=None):
    """Per-token 1x128-group E4M3FN codes of bf16 rows. Returns (q uint8 [rows, K],
    scales f32 [rows, K/128]). ``row_count`` (a one-element int32 device tensor,
    e.g. ``offsets[-1:]``) limits the rows quantised without a host sync."""
    rows, K = x.shape
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize_fp8_rows: x must be bf16")
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, max(K // 128, 0)), dtype=torch.float32, device=x.device)
    n = "quantize_fp8_rows"
    _need(n, "q", q, (rows, K), torch.uint8)
    _need(n, "scales", scales, (rows, max(K // 128, 0)), torch.float32)
    _need(n, "row_count", row_count, (1,), torch.int32)
    _dev(x, row_count, q, scales)
    _ok("quantize_fp8_rows", _lib.load().quantize_fp8_rows(_p(x), rows, _p(row_count), K, _p(q),
                                                           _p(scales), _s(stream)))
    return q, scales


def _a8_weights(name, *ws):
    ws = [_pw(w, name) for w in ws]
    if any(w.dtype != torch.float8_e4m3fn for w in ws):
        raise ValueError(f"{name}: weights must be packed float8_e4m3fn codes")
    return ws


def grouped_gate_up_a8(xq: torch.Tensor, x_scale: torch.Tensor, offsets: torch.Tensor,
                       w_gate, w_up, s_gate: torch.Tensor, s_up: torch.Tensor, *,
                       row_index=None, h_out=None, stream=None) -> torch.Tensor:
    """grouped_gate_up with fp8 activations (xq codes + x_scale per 1x128 group).
    Returns h_out bf16 [max_rows, f]."""
    max_rows, src_rows = _grouped_rows(xq, row_index, "grouped_gate_up_a8")
    d = xq.shape[1]
    w_gate, w_up = _a8_weights("grouped_gate_up_a8", w_gate, w_up)
    e_count, f = w_gate.groups, w_gate.N
    if w_gate.K != d or (w_up.groups, w_up.N, w_up.K) != (e_count, f, d):
        raise ValueError("grouped_gate_up_a8: w_gate/w_up [E, f, d]")
    n = "grouped_gate_up_a8"
    _need(n, "xq", xq, (xq.shape[0], d), torch.uint8)
    _need(n, "x_scale", x_scale, (xq.shape[0], d // 128), torch.float32)
    _need(n, "offsets", offsets, (e_count + 1,), torch.int32)
    _block_scales(n, MF_FP8_E4M3, e_count, f, d, s_gate=s_gate, s_up=s_up)
    if h_out is None:
        h_out = torch.empty((max_rows, f), dtype=torch.bfloat16, device=xq.device)
    _need(n, "h_out", h_out, (max_rows, f), torch.bfloat16)
    _dev(xq, x_scale, row_index, offsets, s_gate, s_up, h_out)
    _ok("grouped_gate_up_a8", _lib.load().grouped_gate_up_a8(
        _p(xq), _p(x_scale), _p(row_index), src_rows, _p(offsets), e_count, max_rows, d, f,
        _p(w_gate.data), _p(w_up.data), _p(s_gate), _p(s_up), _p(h_out), _s(stream)))
    return h_out


def grouped_down_a8(hq: torch.Tensor, h_scale: torch.Tensor, offsets: torch.Tensor, w_down,
                    s_down: torch.Tensor, *, y_perm=None, stream=None) -> torch.Tensor:
    """grouped_down with fp8 activations (hq codes + h_scale per 1x128 group).
    Returns y_perm bf16 [max_rows, d]."""
    max_rows, f = hq.shape
    (w_down,) = _a8_weights("grouped_down_a8", w_down)
    e_count, d = w_down.groups, w_down.N
    if w_down.K != f:
        raise ValueError("grouped_down_a8: w_down [E, d, f]")
    n = "grouped_down_a8"
    _need(n, "hq", hq, (max_rows, f), torch.uint8)
    _need(n, "h_scale", h_scale, (max_rows, f // 128), torch.float32)
    _need(n, "offsets", offsets, (e_count + 1,), torch.int32)
    _block_scales(n, MF_FP8_E4M3, e_count, d, f, s_down=s_down)
    if y_perm is None:
        y_perm = torch.empty((max_rows, d), dtype=torch.bfloat16, device=hq.device)
    _need(n, "y_perm", y_perm, (max_rows, d), torch.bfloat16)
    _dev(hq, h_scale, offsets, s_down, y_perm)
    _ok("grouped_down_a8", _lib.load().grouped_down_a8(
        _p(hq), _p(h_scale), _p(offsets), e_count, max_rows, f, d, _p(w_down.data), _p(s_down),
        _p(y_perm), _s(stream)))
    return y_perm


def moe_combine(y_perm: torch.Tensor, inv_pos: torch.Tensor, topk_w: torch.Tensor,
                out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                residual: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[t] = sum_j topk_w[t,j] * y_perm[inv_pos[t,j]] over local slots (+ residual[t])."""
    T, k = inv_pos.shape
    max_rows, d = y_perm.shape
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y_perm.device)
    if residual is not None and (residual.shape != out.shape or residual.dtype != out.dtype):
        raise ValueError("moe_combine: residual must match out in shape and dtype")
    n = "moe_combine"
    _need(n, "y_perm", y_perm, (max_rows, d), torch.bfloat16)
    _need(n, "inv_pos", inv_pos, (T, k), torch.int32)
    _need(n, "topk_w", topk_w, (T, k), torch.float32)
    _need(n, "out", out, (T, d), out.dtype)
    _dev(y_perm, inv_pos, topk_w, residual, out)
    _ok("moe_combine", _lib.load().moe_combine(_p(y_perm), _p(inv_pos), _p(topk_w), T, k, d,
                                               max_rows, _p(residual), _p(out),
                                               _dtype_code(out.dtype), _s(stream)))
    return out


def tp_shard_mlp(x: torch.Tensor, w_gate_s: torch.Tensor, w_up_s: torch.Tensor,
                 w_down_s: torch.Tensor, *, h_work=None, partial=None, stream=None):
    """One TP shard of the dense gated MLP. Returns (partial f32 [T,d], h_work [T,f_s])."""
    T, d = x.shape
    if x.dtype == torch.bfloat16:
        w_gate_s, w_up_s, w_down_s = (_pw(w, "tp_shard_mlp") for w in (w_gate_s, w_up_s, w_down_s))
        fs = w_gate_s.N
        shapes = [(w.groups, w.N, w.K) for w in (w_gate_s, w_up_s, w_down_s)]
        if shapes != [(1, fs, d), (1, fs, d), (1, d, fs)]:
            raise ValueError("tp_shard_mlp: w_gate_s/w_up_s [f_s, d], w_down_s [d, f_s]")
        ptrs = [w.data for w in (w_gate_s, w_up_s, w_down_s)]
    else:
        fs = w_gate_s.shape[0]
        if (tuple(w_gate_s.shape) != (fs, d) or tuple(w_up_s.shape) != (fs, d)
                or tuple(w_down_s.shape) != (d, fs)):
            raise ValueError("tp_shard_mlp: w_gate_s/w_up_s [f_s, d], w_down_s [d, f_s]")
        ptrs = [w_gate_s, w_up_s, w_down_s]
    if h_work is None:
        h_work = torch.empty((T, fs), dtype=x.dtype, device=x.device)
    if partial is None:
        partial = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _need("tp_shard_mlp", "h_work", h_work, (T, fs), x.dtype)
    _need("tp_shard_mlp", "partial", partial, (T, d), torch.float32)
    if x.dtype == torch.float32:
        for what, w in (("w_gate_s", w_gate_s), ("w_up_s", w_up_s), ("w_down_s", w_down_s)):
            _need("tp_shard_mlp", what, w, tuple(w.shape), torch.float32)
    _dev(x, *ptrs, h_work, partial)
    _ok("tp_shard_mlp", _lib.load().tp_shard_mlp(
        _p(x), _p(ptrs[0]), _p(ptrs[1]), _p(ptrs[2]), T, d, fs, _dtype_code(x.dtype),
        _p(h_work), _p(partial), _s(stream)))
    return partial, h_work


# --------------------------------------------------------------------------


class MoEFFNLayer:
    """One rank's MoE FFN sub-block, FFN(RMSNorm(x)), with buffers allocated once.

    ``forward`` enqueues rmsnorm -> moe_route -> moe_permute -> grouped_gate_up ->
    grouped_down (the two halves of grouped_swiglu) -> moe_combine on the
    current stream and returns the [T, d] output (the partial sum over this
    rank's experts [e_begin, e_begin + e_count), plus ``residual`` if given).
    The permutation runs indices-only: the gate/up GEMM gathers its rows
    V[src_token] inside its A load, so X_perm is never written. ``marks``, if
    given, is a list of 7 events recorded before each of the six stages and
    after the last (rmsnorm's slot is recorded even when the layer has no norm).
    """

    STAGES = ("rmsnorm", "moe_route", "moe_permute", "grouped_gate_up", "grouped_down",
              "moe_combine")

    def __init__(self, *, T: int, d: int, f: int, w_r, bias, w_gate, w_up, w_down,
                 e_begin: int = 0, gamma=None, s_gate=None, s_up=None, s_down=None,
                 k: int = 8, eps: float = 1e-5, out_dtype=torch.bfloat16,
                 act_fp8: bool = False, layout: str = "contiguous", cap: Optional[int] = None):
        """Weights are given [out, in] (w_r [E, d], w_gate/w_up [E_loc, f, d],
        w_down [E_loc, d, f]) and packed here, once.

        ``act_fp8`` (block-fp8 weights only): the expert GEMMs take fp8
        activations, as the block-fp8 prefill variant does: V is quantised per
        token and 1x128 group in the RMSNorm pass (rmsnorm_quantize_fp8; by
        quantize_fp8_rows when the layer has no RMSNorm) and H before the down
        GEMM (quantize_fp8_rows, timed with the down GEMM), and the GEMMs run
        on the fp8 MFMA (grouped_gate_up_a8 / grouped_down_a8).

        ``layout="masked"`` (the decode variant): moe_dispatch_masked replaces
        the permutation (fixed blocks of ``cap`` rows per local expert, default
        T, so no slot is dropped) and the GEMMs run over those blocks
        (grouped_gate_up_masked / grouped_down_masked); the combine reads the
        slots' block rows."""
        dev = w_r.device
        self.T, self.d, self.f, self.k, self.eps = T, d, f, k, eps
        self.e_begin, self.e_count = e_begin, w_gate.shape[0]
        self.gamma, self.bias = gamma, bias
        self.w_r = pack_weights(w_r)
        self.w = tuple(pack_weights(w) for w in (w_gate, w_up, w_down))
        self.s = (s_gate, s_up, s_down)
        bf = torch.bfloat16
        rows = T * k
        self.v = torch.empty((T, d), dtype=bf, device=dev) if gamma is not None else None
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(self.e_count, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.e_count + 1, dtype=torch.int32, device=dev)
        self.src_token = torch.empty(rows, dtype=torch.int32, device=dev)
        self.inv_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.workspace = torch.empty(max(1, moe_permute_workspace_size(T, k, self.e_count)),
                                     dtype=torch.uint8, device=dev)
        self.route_ws = torch.empty(max(1, moe_route_workspace_size(T, d, self.w_r.N)),
                                    dtype=torch.uint8, device=dev)
        self.h = torch.empty((rows, f), dtype=bf, device=dev)
        self.y_perm = torch.empty((rows, d), dtype=bf, device=dev)
        self.out = torch.empty((T, d), dtype=out_dtype, device=dev)
        self.act_fp8 = act_fp8
        if layout not in ("contiguous", "masked"):
            raise ValueError("MoEFFNLayer: layout is 'contiguous' or 'masked'")
        self.layout = layout
        if layout == "masked":
            if act_fp8:
                raise ValueError("MoEFFNLayer: the masked layout runs with bf16 activations")
            self.cap = T if cap is None else cap
            mrows = self.e_count * self.cap
            self.row_index = torch.empty(mrows, dtype=torch.int32, device=dev)
            self.h = torch.empty((mrows, f), dtype=bf, device=dev)
            self.y_perm = torch.empty((mrows, d), dtype=bf, device=dev)
        if act_fp8:
            if w_gate.dtype != torch.float8_e4m3fn or s_gate is None:
                raise ValueError("MoEFFNLayer: act_fp8 needs block-fp8 weights and scales")
            self.vq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.vs = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
            self.hq = torch.empty((rows, f), dtype=torch.uint8, device=dev)
            self.hs = torch.empty((rows, f // 128), dtype=torch.float32, device=dev)

    def forward(self, x: torch.Tensor, stream=None, marks=None,
                residual: Optional[torch.Tensor] = None) -> torch.Tensor:
        s = torch.cuda.current_stream() if stream is None else stream
        if tuple(x.shape) != (self.T, self.d) or x.dtype != torch.bfloat16:
            raise ValueError(f"MoEFFNLayer: x must be bf16 {(self.T, self.d)} (the shape the "
                             f"layer's buffers were sized for), got {x.dtype} {tuple(x.shape)}")

        def mark(i):
            if marks is not None:
                marks[i].record(s)

        mark(0)
        v = x
        if self.gamma is not None and self.act_fp8 and self.layout == "contiguous":
            # V and its per-token fp8 activations in one pass
            v, _, _ = rmsnorm_quantize_fp8(x, self.gamma, self.eps, out=self.v, q=self.vq,
                                           scales=self.vs, stream=s)
        elif self.gamma is not None:
            v = rmsnorm(x, self.gamma, self.eps, out=self.v, stream=s)
        mark(1)
        moe_route(v, self.w_r, self.bias, self.k, self.idx, self.topk_w, self.route_ws, stream=s)
        mark(2)
        if self.layout == "masked":
            moe_dispatch_masked(self.idx, self.e_begin, self.e_count, self.cap, counts=self.counts,
                                row_index=self.row_index, pos=self.inv_pos,
                                workspace=self.workspace, stream=s)
            mark(3)
            grouped_gate_up_masked(v, self.row_index, self.counts, self.cap, self.w[0], self.w[1],
                                   self.s[0], self.s[1], h_out=self.h, stream=s)
            mark(4)
            grouped_down_masked(self.h, self.counts, self.cap, self.w[2], self.s[2],
                                y_perm=self.y_perm, stream=s)
            mark(5)
            out = moe_combine(self.y_perm, self.inv_pos, self.topk_w, out=self.out,
                              residual=residual, stream=s)
            mark(6)
            return out
        moe_permute(self.idx, self.e_begin, self.e_count, None, counts=self.counts,
                    offsets=self.offsets, src_token=self.src_token, inv_pos=self.inv_pos,
                    workspace=self.workspace, stream=s)
        mark(3)
        if self.act_fp8:
            if self.gamma is None:  # no RMSNorm pass to fold the quantisation into
                quantize_fp8_rows(v, q=self.vq, scales=self.vs, stream=s)
            grouped_gate_up_a8(self.vq, self.vs, self.offsets, self.w[0], self.w[1], self.s[0],
                               self.s[1], row_index=self.src_token, h_out=self.h, stream=s)
            mark(4)
            # only the live rows of H (offsets[-1], known on the device)
            quantize_fp8_rows(self.h, row_count=self.offsets[-1:], q=self.hq, scales=self.hs,
                              stream=s)
            grouped_down_a8(self.hq, self.hs, self.offsets, self.w[2], self.s[2],
                            y_perm=self.y_perm, stream=s)
        else:
            grouped_gate_up(v, self.offsets, self.w[0], self.w[1], self.s[0], self.s[1],
                            row_index=self.src_token, h_out=self.h, stream=s)
            mark(4)
            grouped_down(self.h, self.offsets, self.w[2], self.s[2], y_perm=self.y_perm,
                         stream=s)
        mark(5)
        out = moe_combine(self.y_perm, self.inv_pos, self.topk_w, out=self.out,
                          residual=residual, stream=s)
        mark(6)
        return out

    __call__ = forward
