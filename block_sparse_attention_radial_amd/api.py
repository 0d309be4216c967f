"""Python binding of libradial.so (ctypes). Argument marshalling only.

Every step of the forward pass runs in the library. torch supplies device memory and
the current HIP stream. If the library has not been built, the calls raise: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

from .build import LIB_PATH

BLOCK = 128

RADIAL_OK = 0
_ERRORS = {
    -1: "INVALID_ARG", -2: "UNSUPPORTED_HEAD_DIM", -3: "CAPACITY", -4: "SHAPE_MISMATCH",
    -5: "MISALIGNED", -6: "TOO_LARGE", -7: "HIP",
}

# Every symbol that include/radial_attn.h declares, with its ctypes signature.
_SIGNATURES = {
    "radial_mask_dims": (ctypes.c_int32, [ctypes.c_int32] * 4 + [
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "radial_build_mask": (ctypes.c_int32, [ctypes.c_int32] * 4 + [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]),
    "radial_mask_dims_grid": (ctypes.c_int32, [ctypes.c_int32] * 5 + [
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "radial_build_mask_grid": (ctypes.c_int32, [ctypes.c_int32] * 5 + [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]),
    "radial_build_pairs": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_int32)]),
    "radial_attn_fwd": (ctypes.c_int32, [ctypes.c_void_p] * 7 + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float] + [ctypes.c_int32] * 7
        + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_element_table_bytes": (ctypes.c_int32, [ctypes.c_int64,
                                                    ctypes.POINTER(ctypes.c_int64)]),
    "radial_build_element_table": (ctypes.c_int32, [ctypes.c_void_p] * 2 + [
        ctypes.c_int32, ctypes.c_int64] + [ctypes.c_int32] * 3 + [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "radial_attn_fwd_element_table": (ctypes.c_int32, [ctypes.c_void_p] * 7 + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
        + [ctypes.c_int32] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_attn_fwd_rule": (ctypes.c_int32, [ctypes.c_void_p] * 5 + [ctypes.c_int32] * 5 + [
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float] + [ctypes.c_int32] * 3
        + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_attn_fwd_varlen_rule": (ctypes.c_int32, [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 5
        + [ctypes.c_void_p] * 2 + [ctypes.c_float] + [ctypes.c_int32] * 2
        + [ctypes.c_int64] * 2 + [ctypes.c_void_p]),
    "radial_attn_fwd_varlen": (ctypes.c_int32, [ctypes.c_void_p] * 6 + [ctypes.c_int32] + [
        ctypes.c_void_p] * 4 + [ctypes.c_float] + [ctypes.c_int32] * 5 + [ctypes.c_int64] * 2
        + [ctypes.c_void_p]),
    "radial_attn_fwd_varlen_element_table": (ctypes.c_int32, [ctypes.c_void_p] * 6 + [
        ctypes.c_int32] + [ctypes.c_void_p] * 4 + [ctypes.c_float, ctypes.c_void_p]
        + [ctypes.c_int32] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]),
    "radial_attn_bwd_varlen_element_table": (ctypes.c_int32, [ctypes.c_void_p] * 11 + [
        ctypes.c_int32] + [ctypes.c_void_p] * 4 + [ctypes.c_float, ctypes.c_void_p]
        + [ctypes.c_int32] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]),
    "radial_transpose_mask": (ctypes.c_int32, [ctypes.c_int32] + [ctypes.c_void_p] * 4),
    "radial_attn_bwd": (ctypes.c_int32, [ctypes.c_void_p] * 14 + [
        ctypes.c_int32, ctypes.c_float] + [ctypes.c_int32] * 7
        + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_attn_bwd_element_table": (ctypes.c_int32, [ctypes.c_void_p] * 14 + [
        ctypes.c_int32, ctypes.c_float, ctypes.c_void_p] + [ctypes.c_int32] * 4
        + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_attn_bwd_noalloc": (ctypes.c_int32, [ctypes.c_void_p] * 13 + [
        ctypes.c_int32, ctypes.c_float] + [ctypes.c_int32] * 7
        + [ctypes.c_int64] * 3 + [ctypes.c_void_p]),
    "radial_attn_bwd_varlen": (ctypes.c_int32, [ctypes.c_void_p] * 11 + [ctypes.c_int32] + [
        ctypes.c_void_p] * 4 + [ctypes.c_float] + [ctypes.c_int32] * 5 + [ctypes.c_int64] * 2
        + [ctypes.c_void_p]),
    "radial_error_string": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lib = None


class RadialError(RuntimeError):
    """A non-zero return code from libradial.so."""

    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {_ERRORS.get(code, code)} ({error_string(code)})")


def library_path() -> str:
    return os.environ.get("RADIAL_LIB", LIB_PATH)


def lib():
    """The loaded libradial.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m block_sparse_attention_radial_amd.build` (or __graft_entry__.build())")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def error_string(code: int) -> str:
    return lib().radial_error_string(code).decode()


def _check(fn: str, code: int):
    if code != RADIAL_OK:
        raise RadialError(fn, code)


@dataclass
class Mask:
    """Block mask in compressed-row form: int32 row_ptr[nb + 1], col_idx[nnz].

    `pairs` (optional, int32 [npairs, 2]) says which rows the kernel computes together
    (build_pairs); None means rows 2p and 2p + 1. It changes the time, not the result.
    `col_ptr` / `row_idx` (optional) are the transposed mask the backward pass walks;
    `transposed()` builds them when absent. `grid_w` is 0 for the 1-D spatial distance,
    or the width of the latent grid a frame is stored as (rows of grid_w tokens; the
    spatial distance is then the Manhattan distance on the grid). `element_table`
    (optional, int64 [nnz, 256], from `with_element_table()`) holds the element rule's
    decisions for every active block; element masking in the forward (and, for a
    symmetric mask, the backward) then reads them instead of evaluating the rule, with
    the same result bit for bit.
    """

    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    frames: int
    tokens_per_frame: int
    w0: int
    pairs: torch.Tensor | None = None
    col_ptr: torch.Tensor | None = None
    row_idx: torch.Tensor | None = None
    grid_w: int = 0
    element_table: torch.Tensor | None = None
    _symmetric: bool | None = field(default=None, repr=False, compare=False)

    @property
    def n(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def nb(self) -> int:
        return self.row_ptr.numel() - 1

    @property
    def nnz(self) -> int:
        return self.col_idx.numel()

    @property
    def device(self) -> torch.device:
        return self.row_ptr.device

    def to(self, device) -> "Mask":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return Mask(self.row_ptr.to(device), self.col_idx.to(device), self.frames,
                    self.tokens_per_frame, self.w0, mv(self.pairs), mv(self.col_ptr),
                    mv(self.row_idx), self.grid_w, mv(self.element_table))

    def symmetric(self) -> bool:
        """Whether the mask equals its transpose (every radial mask does; the backward reads
        an element table only then). Computed once, with the transposed mask."""
        if self._symmetric is None:
            t = self.transposed()
            self._symmetric = bool(torch.equal(t.row_ptr.cpu(), t.col_ptr.cpu())
                                   and torch.equal(t.col_idx.cpu(), t.row_idx.cpu()))
        return self._symmetric

    def with_element_table(self) -> "Mask":
        """This mask with element_table filled in (built on the mask's GPU when absent,
        radial_build_element_table, on torch's current stream)."""
        if self.element_table is None:
            self.element_table = build_element_table(self)
        return self

    def transposed(self) -> "Mask":
        """This mask with col_ptr / row_idx filled in (radial_transpose_mask, on the host,
        then moved to the mask's device)."""
        if self.col_ptr is None or self.row_idx is None:
            rp = self.row_ptr.to("cpu", torch.int32).contiguous()
            ci = self.col_idx.to("cpu", torch.int32).contiguous()
            cp = torch.empty(self.nb + 1, dtype=torch.int32)
            ri = torch.empty(max(ci.numel(), 1), dtype=torch.int32)
            _check("radial_transpose_mask", lib().radial_transpose_mask(
                self.nb, rp.data_ptr(), ci.data_ptr(), cp.data_ptr(), ri.data_ptr()))
            self.col_ptr = cp.to(self.device)
            self.row_idx = ri[:int(cp[-1])].to(self.device)
        return self


def build_element_table(mask: Mask) -> torch.Tensor:
    """The element table of a mask on the GPU (radial_build_element_table): int64
    [nnz, 256], 2048 bytes per active block, with the decisions of element masking by the
    mask's frame length, W0 and grid width. Asynchronous on torch's current stream."""
    if not mask.row_ptr.is_cuda or mask.col_idx.device != mask.row_ptr.device:
        raise ValueError("the mask must be on a GPU (Mask.to(device))")
    elem_s, elem_w0, elem_gw = _element_args(mask, True)
    nbytes = ctypes.c_int64(0)
    _check("radial_element_table_bytes",
           lib().radial_element_table_bytes(mask.nnz, ctypes.byref(nbytes)))
    table = torch.empty(max(nbytes.value // 8, 256), dtype=torch.int64, device=mask.device)
    stream = torch.cuda.current_stream(mask.device).cuda_stream
    _check("radial_build_element_table", lib().radial_build_element_table(
        mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.nb, mask.nnz, elem_s, elem_w0,
        elem_gw, table.data_ptr(), table.numel() * 8, stream))
    return table[:nbytes.value // 8].view(-1, 256)


def _check_table(table: torch.Tensor, nnz: int, device) -> None:
    if (table.device != device or table.dtype != torch.int64 or table.numel() != 256 * nnz
            or not table.is_contiguous()):
        raise ValueError("the mask's element_table must be its contiguous int64 [nnz, 256] "
                         "table on q's device (with_element_table)")


def _grid_rows(tokens_per_frame: int, grid_w: int | None) -> int:
    if grid_w is None:
        return 1
    if grid_w <= 0 or tokens_per_frame % grid_w:
        raise ValueError("the grid width must divide the tokens per frame")
    return tokens_per_frame // grid_w


def mask_dims(frames: int, tokens_per_frame: int, w0: int, block: int = BLOCK,
              grid_w: int | None = None):
    nb, nnz = ctypes.c_int32(), ctypes.c_int64()
    if grid_w is None:
        _check("radial_mask_dims", lib().radial_mask_dims(
            frames, tokens_per_frame, w0, block, ctypes.byref(nb), ctypes.byref(nnz)))
    else:
        _check("radial_mask_dims_grid", lib().radial_mask_dims_grid(
            frames, _grid_rows(tokens_per_frame, grid_w), grid_w, w0, block,
            ctypes.byref(nb), ctypes.byref(nnz)))
    return nb.value, nnz.value


def build_pairs(row_ptr: torch.Tensor, col_idx: torch.Tensor,
                tokens_per_frame: int = 0) -> torch.Tensor:
    """Pair table (int32 [npairs, 2], host) for a host CSR: rows with many key blocks in
    common share a workgroup; (a, -1) is a row that runs alone."""
    row_ptr = row_ptr.to("cpu", torch.int32).contiguous()
    col_idx = col_idx.to("cpu", torch.int32).contiguous()
    nb = row_ptr.numel() - 1
    pairs = torch.empty(max(nb, 1), 2, dtype=torch.int32)
    npairs = ctypes.c_int32()
    _check("radial_build_pairs", lib().radial_build_pairs(
        nb, row_ptr.data_ptr(), col_idx.data_ptr(), tokens_per_frame, pairs.data_ptr(),
        ctypes.byref(npairs)))
    return pairs[:npairs.value].clone()


def build_mask(frames: int, tokens_per_frame: int, w0: int, block: int = BLOCK,
               pairs: bool = True, grid_w: int | None = None) -> Mask:
    """The static radial block mask for a frames x tokens_per_frame video (host tensors),
    with its pair table unless `pairs` is False. `grid_w` switches to the 2-D grid
    distance on frames of tokens_per_frame / grid_w rows of grid_w tokens."""
    nb, nnz = mask_dims(frames, tokens_per_frame, w0, block, grid_w)
    row_ptr = torch.empty(nb + 1, dtype=torch.int32)
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32)
    if grid_w is None:
        _check("radial_build_mask", lib().radial_build_mask(
            frames, tokens_per_frame, w0, block, row_ptr.data_ptr(), col_idx.data_ptr(), nnz))
    else:
        _check("radial_build_mask_grid", lib().radial_build_mask_grid(
            frames, _grid_rows(tokens_per_frame, grid_w), grid_w, w0, block,
            row_ptr.data_ptr(), col_idx.data_ptr(), nnz))
    col_idx = col_idx[:nnz]
    table = build_pairs(row_ptr, col_idx, tokens_per_frame) if pairs else None
    # The radial mask is symmetric at block level: its transpose is itself.
    return Mask(row_ptr, col_idx, frames, tokens_per_frame, w0, table, row_ptr, col_idx,
                grid_w or 0)


def dense_mask(seqlen: int, device="cpu") -> Mask:
    """All-active CSR (every query block sees every key block): the dense baseline."""
    nb = (seqlen + BLOCK - 1) // BLOCK
    row_ptr = torch.arange(0, nb * nb + 1, nb, dtype=torch.int32, device=device)
    col_idx = torch.arange(nb, dtype=torch.int32, device=device).repeat(nb)
    return Mask(row_ptr, col_idx, 1, seqlen, 2**31 - 1, None, row_ptr, col_idx)


def _element_args(mask, element: bool):
    """(frame length, W0, grid width) for radial_attn_*: zeros for block semantics."""
    if not element:
        return 0, 0, 0
    if mask.tokens_per_frame < BLOCK:
        raise ValueError("element masking needs a frame length of at least 128 tokens")
    return mask.tokens_per_frame, mask.w0, mask.grid_w


@dataclass
class RuleMask:
    """The radial mask given by its rule alone: no CSR is stored, the kernel derives each
    row's key blocks on the fly (radial_attn_fwd_rule). `grid_w` is 0 for the 1-D
    distance or the grid width; `pairs` (optional int32 [npairs, 2]) is a pair table from
    build_pairs, as in Mask."""

    frames: int
    tokens_per_frame: int
    w0: int
    grid_w: int = 0
    pairs: torch.Tensor | None = None
    _built: Mask | None = field(default=None, repr=False, compare=False)

    @property
    def n(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def nb(self) -> int:
        return (self.n + BLOCK - 1) // BLOCK

    def to(self, device) -> "RuleMask":
        return RuleMask(self.frames, self.tokens_per_frame, self.w0, self.grid_w,
                        None if self.pairs is None else self.pairs.to(device), self._built)

    def built(self, device="cpu") -> Mask:
        """The CSR this rule gives (radial_build_mask / radial_build_mask_grid), cached,
        on `device`: what the backward pass walks."""
        if self._built is None:
            self._built = build_mask(self.frames, self.tokens_per_frame, self.w0,
                                     pairs=False, grid_w=self.grid_w or None)
        return self._built.to(device)


def rule_mask(frames: int, tokens_per_frame: int, w0: int, grid_w: int | None = None,
              pairs: bool = False) -> RuleMask:
    """A RuleMask; with `pairs`, its pair table is built on the host from the CSR (which
    is then kept for the backward pass)."""
    _grid_rows(tokens_per_frame, grid_w)
    m = RuleMask(frames, tokens_per_frame, w0, grid_w or 0)
    if pairs:
        m._built = build_mask(frames, tokens_per_frame, w0, pairs=True, grid_w=grid_w)
        m.pairs = m._built.pairs
    return m


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: "Mask | RuleMask",
             scale: float | None = None, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, element: bool = False) -> torch.Tensor:
    """Radial attention forward on q, k, v of shape [B, H, n, D] (bf16, on the GPU).

    Any layout with a contiguous last axis and strides shared by q, k, v and out works,
    e.g. a [B, n, H, D] buffer viewed as [B, H, n, D]. `lse` (optional, fp32 [B, H, n],
    contiguous) receives the natural-log log-sum-exp of every row. `element` applies the
    radial rule to single entries inside the active blocks, with the mask's frame length,
    W0 and distance (its grid width; block semantics otherwise); a Mask that carries an
    element table (Mask.with_element_table) gives the same decisions from the table. With
    a RuleMask the kernel derives the key blocks from the rule instead of reading a CSR.
    The call is asynchronous on torch's current stream.
    """
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share the shape [B, H, n, D]")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    rule = isinstance(mask, RuleMask)
    if (not rule and (mask.row_ptr.device != q.device or mask.col_idx.device != q.device)) or (
            mask.pairs is not None and mask.pairs.device != q.device):
        raise ValueError("the mask must be on the same device as q (Mask.to(device))")
    if mask.pairs is not None and (mask.pairs.dtype != torch.int32 or mask.pairs.dim() != 2
                                   or mask.pairs.shape[1] != 2
                                   or not mask.pairs.is_contiguous()):
        raise ValueError("mask.pairs must be a contiguous int32 [npairs, 2] tensor")
    if q.stride() != k.stride() or q.stride() != v.stride() or q.stride(-1) != 1:
        raise ValueError("q, k, v must share strides with a contiguous last axis")
    B, H, n, D = q.shape
    if rule and n != mask.n:
        raise ValueError("q's sequence length must be frames * tokens_per_frame")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.stride() != q.stride() or out.dtype != q.dtype:
        raise ValueError("out must match q in shape, strides and dtype")
    if lse is not None and (lse.shape != (B, H, n) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor on q's device")
    if scale is None:
        scale = D ** -0.5
    elem_s, elem_w0, elem_gw = _element_args(mask, element)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if rule:
        _check("radial_attn_fwd_rule", lib().radial_attn_fwd_rule(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(), mask.frames, mask.tokens_per_frame,
            mask.grid_w, mask.w0, int(bool(element)),
            None if mask.pairs is None else mask.pairs.data_ptr(),
            0 if mask.pairs is None else mask.pairs.shape[0], float(scale), B, H, D,
            q.stride(0), q.stride(1), q.stride(2), stream))
        return out
    table = mask.element_table if element else None
    if table is not None:
        _check_table(table, mask.nnz, q.device)
        _check("radial_attn_fwd_element_table", lib().radial_attn_fwd_element_table(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(),
            mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.nb,
            None if mask.pairs is None else mask.pairs.data_ptr(),
            0 if mask.pairs is None else mask.pairs.shape[0], float(scale), table.data_ptr(),
            B, H, n, D, q.stride(0), q.stride(1), q.stride(2), stream))
        return out
    _check("radial_attn_fwd", lib().radial_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(),
        mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.nb,
        None if mask.pairs is None else mask.pairs.data_ptr(),
        0 if mask.pairs is None else mask.pairs.shape[0], float(scale), elem_s, elem_w0,
        elem_gw, B, H, n, D, q.stride(0), q.stride(1), q.stride(2), stream))
    return out


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             do: torch.Tensor, lse: torch.Tensor, mask: "Mask | RuleMask",
             scale: float | None = None,
             element: bool = False):
    """Gradients (dq, dk, dv) of attn_fwd for the output gradient `do`, from the forward's
    output `o` and log-sum-exp `lse` (all on the GPU; layouts as for attn_fwd). The call
    is asynchronous on torch's current stream. A RuleMask is walked as the CSR its rule
    gives (built on the host once). With element masking, a symmetric Mask that carries an
    element table gives the decisions from the table (the same ones, bit for bit)."""
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, do)):
        raise ValueError("q, k, v, o, do must share the shape [B, H, n, D]")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v, o, do)):
        raise TypeError("q, k, v, o, do must be bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in (k, v, o, do, lse)):
        raise ValueError("every tensor must be on the same GPU")
    if any(t.stride() != q.stride() for t in (k, v, o, do)) or q.stride(-1) != 1:
        raise ValueError("q, k, v, o, do must share strides with a contiguous last axis")
    B, H, n, D = q.shape
    if lse.shape != (B, H, n) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [B, H, n] output")
    if isinstance(mask, RuleMask):
        mask = mask.built(q.device)
    mask = mask.transposed()
    if any(t.device != q.device for t in (mask.row_ptr, mask.col_idx, mask.col_ptr,
                                          mask.row_idx)):
        raise ValueError("the mask must be on the same device as q (Mask.to(device))")
    if scale is None:
        scale = D ** -0.5
    elem_s, elem_w0, elem_gw = _element_args(mask, element)
    dq, dk, dv = (torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
                  for _ in range(3))
    delta = torch.empty(2, B, H, n, dtype=torch.float32, device=q.device)  # D_i, base-2 lse
    stream = torch.cuda.current_stream(q.device).cuda_stream
    table = mask.element_table if element else None
    if table is not None and mask.symmetric():
        _check_table(table, mask.nnz, q.device)
        _check("radial_attn_bwd_element_table", lib().radial_attn_bwd_element_table(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
            mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.col_ptr.data_ptr(),
            mask.row_idx.data_ptr(), mask.nb, float(scale), table.data_ptr(), B, H, n, D,
            q.stride(0), q.stride(1), q.stride(2), stream))
        return dq, dk, dv
    _check("radial_attn_bwd", lib().radial_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
        mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.col_ptr.data_ptr(),
        mask.row_idx.data_ptr(), mask.nb, float(scale), elem_s, elem_w0,
        elem_gw, B, H, n, D, q.stride(0), q.stride(1), q.stride(2), stream))
    return dq, dk, dv


def _like_q(do: torch.Tensor, q: torch.Tensor) -> torch.Tensor:
    """The output gradient in q's strides (the backward kernels take one set of strides
    for every tensor). A gradient in other strides (a contiguous one for a [B, n, H, D]
    view, or the zero strides of an expanded sum's gradient) is copied into a new tensor."""
    if do.stride() == q.stride() and do.dtype == q.dtype:
        return do
    return torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device).copy_(do)


def attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     do: torch.Tensor, lse: torch.Tensor, mask: Mask,
                     scale: float | None = None, element: bool = False, out=None):
    """attn_bwd through radial_attn_bwd_noalloc: the library allocates nothing (its D_i
    workspace is static device memory, shared by every call on the device). `out`
    (optional) is a tuple (dq, dk, dv) of tensors in q's shape and strides; without it
    they are allocated here. `mask` must already hold its transpose on q's device
    (Mask.transposed().to(device)), so that this call makes no host work either."""
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, do)):
        raise ValueError("q, k, v, o, do must share the shape [B, H, n, D]")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v, o, do)):
        raise TypeError("q, k, v, o, do must be bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in (k, v, o, do, lse)):
        raise ValueError("every tensor must be on the same GPU")
    if any(t.stride() != q.stride() for t in (k, v, o, do)) or q.stride(-1) != 1:
        raise ValueError("q, k, v, o, do must share strides with a contiguous last axis")
    B, H, n, D = q.shape
    if lse.shape != (B, H, n) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [B, H, n] output")
    if mask.col_ptr is None or mask.row_idx is None or any(
            t.device != q.device for t in (mask.row_ptr, mask.col_idx, mask.col_ptr,
                                           mask.row_idx)):
        raise ValueError("the mask and its transpose must be on q's device")
    if scale is None:
        scale = D ** -0.5
    elem_s, elem_w0, elem_gw = _element_args(mask, element)
    if out is None:
        out = tuple(torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
                    for _ in range(3))
    elif any(t.shape != q.shape or t.stride() != q.stride() or t.dtype != q.dtype
             or t.device != q.device for t in out):
        raise ValueError("out must be three tensors in q's shape, strides, dtype and device")
    dq, dk, dv = out
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check("radial_attn_bwd_noalloc", lib().radial_attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), mask.row_ptr.data_ptr(),
        mask.col_idx.data_ptr(), mask.col_ptr.data_ptr(), mask.row_idx.data_ptr(), mask.nb,
        float(scale), elem_s, elem_w0, elem_gw, B, H, n, D, q.stride(0), q.stride(1),
        q.stride(2), stream))
    return dq, dk, dv


class RadialAttentionFunction(torch.autograd.Function):
    """attn_fwd with its backward (attn_bwd) for autograd."""

    @staticmethod
    def forward(ctx, q, k, v, mask, scale, element):
        B, H, n, _ = q.shape
        lse = torch.empty(B, H, n, dtype=torch.float32, device=q.device)
        o = attn_fwd(q, k, v, mask, scale=scale, lse=lse, element=element)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.mask, ctx.scale, ctx.element = mask, scale, element
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, _like_q(do, q), lse, ctx.mask, scale=ctx.scale,
                              element=ctx.element)
        return dq, dk, dv, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: "Mask | RuleMask",
              scale: float | None = None, element: bool = False) -> torch.Tensor:
    """Radial attention with autograd support (forward attn_fwd, backward attn_bwd)."""
    return RadialAttentionFunction.apply(q, k, v, mask, scale, element)


@dataclass
class VarlenMask:
    """The block masks of a varlen batch, concatenated as radial_attn_fwd_varlen takes
    them: sample b's row_ptr (rebased to index the concatenated col_idx) follows those of
    the samples before it, and likewise its pair table and (for the backward pass) its
    transposed mask col_ptr / row_idx. `element_table` (optional, from
    `with_element_table()`) is the samples' element tables concatenated likewise."""

    seq_tokens: list
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    tokens_per_frame: int
    w0: int
    pairs: torch.Tensor | None = None
    npairs: list | None = None
    grid_w: int = 0
    col_ptr: torch.Tensor | None = None
    row_idx: torch.Tensor | None = None
    element_table: torch.Tensor | None = None
    _symmetric: bool | None = field(default=None, repr=False, compare=False)

    @property
    def batch(self) -> int:
        return len(self.seq_tokens)

    def to(self, device) -> "VarlenMask":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return VarlenMask(list(self.seq_tokens), self.row_ptr.to(device), self.col_idx.to(device),
                          self.tokens_per_frame, self.w0, mv(self.pairs),
                          None if self.npairs is None else list(self.npairs), self.grid_w,
                          mv(self.col_ptr), mv(self.row_idx), mv(self.element_table))

    def symmetric(self) -> bool:
        """Whether every sample's mask equals its transpose (computed once)."""
        if self._symmetric is None:
            self._symmetric = (self.col_ptr is not None and self.row_idx is not None
                               and bool(torch.equal(self.row_ptr.cpu(), self.col_ptr.cpu()))
                               and bool(torch.equal(self.col_idx.cpu(), self.row_idx.cpu())))
        return self._symmetric

    def with_element_table(self) -> "VarlenMask":
        """This batch with element_table filled in: each sample's table built on the mask's
        GPU from its slice of the concatenated CSR, then concatenated (torch's current
        stream)."""
        if self.element_table is None:
            rp = self.row_ptr.cpu()
            tables, r0 = [], 0
            for n in self.seq_tokens:
                nb = (n + BLOCK - 1) // BLOCK
                if n % self.tokens_per_frame:
                    raise ValueError("element masking needs whole frames in every sample")
                lo, hi = int(rp[r0]), int(rp[r0 + nb])
                m = Mask((self.row_ptr[r0:r0 + nb + 1] - lo).contiguous(),
                         self.col_idx[lo:hi].contiguous(), n // self.tokens_per_frame,
                         self.tokens_per_frame, self.w0, grid_w=self.grid_w)
                tables.append(build_element_table(m))
                r0 += nb + 1
            self.element_table = torch.cat(tables)
        return self


def concat_masks(masks: list) -> VarlenMask:
    """One VarlenMask from per-sample masks of one frame length, W0 and distance (host
    tensors)."""
    if not masks:
        raise ValueError("a varlen batch needs at least one sample")
    S, w0, gw = masks[0].tokens_per_frame, masks[0].w0, masks[0].grid_w
    if any(m.tokens_per_frame != S or m.w0 != w0 or m.grid_w != gw for m in masks):
        raise ValueError("the samples must share the frame length, W0 and grid width")
    rps, cps, off, off_t = [], [], 0, 0
    for m in masks:
        m.transposed()
        rps.append(m.row_ptr.to("cpu", torch.int32) + off)
        cps.append(m.col_ptr.to("cpu", torch.int32) + off_t)
        off += m.nnz
        off_t += m.row_idx.numel()
    with_pairs = all(m.pairs is not None for m in masks)
    return VarlenMask([m.n for m in masks], torch.cat(rps),
                      torch.cat([m.col_idx.to("cpu", torch.int32) for m in masks]), S, w0,
                      torch.cat([m.pairs.to("cpu") for m in masks]) if with_pairs else None,
                      [m.pairs.shape[0] for m in masks] if with_pairs else None, gw,
                      torch.cat(cps),
                      torch.cat([m.row_idx.to("cpu", torch.int32) for m in masks]))


def build_varlen_mask(frames: list, tokens_per_frame: int, w0: int, pairs: bool = True,
                      grid_w: int | None = None):
    """The radial masks of videos with the given frame counts (one frame length, one W0,
    one distance)."""
    return concat_masks([build_mask(f, tokens_per_frame, w0, pairs=pairs, grid_w=grid_w)
                         for f in frames])


@dataclass
class VarlenRuleMask:
    """The masks of a varlen batch given by their rule alone (no CSR): sample b is a
    video of frames[b] frames; the kernel derives each row's key blocks on the fly
    (radial_attn_fwd_varlen_rule). `pairs` / `npairs` (optional) as in VarlenMask."""

    frames: list
    tokens_per_frame: int
    w0: int
    grid_w: int = 0
    pairs: torch.Tensor | None = None
    npairs: list | None = None
    _built: "VarlenMask | None" = field(default=None, repr=False, compare=False)

    @property
    def seq_tokens(self) -> list:
        return [f * self.tokens_per_frame for f in self.frames]

    def built(self, device="cpu") -> "VarlenMask":
        """The concatenated CSRs this rule gives (built on the host once, cached), on
        `device`: what the backward pass walks."""
        if self._built is None:
            self._built = build_varlen_mask(self.frames, self.tokens_per_frame, self.w0,
                                            pairs=False, grid_w=self.grid_w or None)
        return self._built.to(device)

    @property
    def batch(self) -> int:
        return len(self.frames)

    def to(self, device) -> "VarlenRuleMask":
        return VarlenRuleMask(list(self.frames), self.tokens_per_frame, self.w0, self.grid_w,
                              None if self.pairs is None else self.pairs.to(device),
                              None if self.npairs is None else list(self.npairs), self._built)


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    mask: "VarlenMask | VarlenRuleMask",
                    scale: float | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, element: bool = False) -> torch.Tensor:
    """Radial attention forward on a packed batch: q, k, v of shape [total_tokens, H, D]
    (bf16, on the GPU), sample b holding the next mask.seq_tokens[b] tokens. `lse`
    (optional) is fp32 [H, total_tokens]. Asynchronous on torch's current stream."""
    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share the shape [total_tokens, H, D]")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.stride() != k.stride() or q.stride() != v.stride() or q.stride(-1) != 1:
        raise ValueError("q, k, v must share strides with a contiguous last axis")
    total, H, D = q.shape
    if sum(mask.seq_tokens) != total:
        raise ValueError("the samples' lengths must add up to q's token count")
    rule = isinstance(mask, VarlenRuleMask)
    if (not rule and (mask.row_ptr.device != q.device or mask.col_idx.device != q.device)) or (
            mask.pairs is not None and mask.pairs.device != q.device):
        raise ValueError("the mask must be on the same device as q (VarlenMask.to(device))")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.stride() != q.stride() or out.dtype != q.dtype:
        raise ValueError("out must match q in shape, strides and dtype")
    if lse is not None and (lse.shape != (H, total) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [H, total_tokens] tensor on q's device")
    if scale is None:
        scale = D ** -0.5
    elem_s, elem_w0, elem_gw = _element_args(mask, element)
    npr = None if mask.npairs is None else (ctypes.c_int32 * mask.batch)(*mask.npairs)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if rule:
        frames = (ctypes.c_int32 * mask.batch)(*mask.frames)
        _check("radial_attn_fwd_varlen_rule", lib().radial_attn_fwd_varlen_rule(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(), frames, mask.batch,
            mask.tokens_per_frame, mask.grid_w, mask.w0, int(bool(element)),
            None if mask.pairs is None else mask.pairs.data_ptr(), npr, float(scale), H, D,
            q.stride(1), q.stride(0), stream))
        return out
    seq = (ctypes.c_int32 * mask.batch)(*mask.seq_tokens)
    table = mask.element_table if element else None
    if table is not None:
        _check_table(table, mask.col_idx.numel(), q.device)
        _check("radial_attn_fwd_varlen_element_table", lib().radial_attn_fwd_varlen_element_table(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(), seq, mask.batch, mask.row_ptr.data_ptr(),
            mask.col_idx.data_ptr(), None if mask.pairs is None else mask.pairs.data_ptr(),
            npr, float(scale), table.data_ptr(), H, D, q.stride(1), q.stride(0), stream))
        return out
    _check("radial_attn_fwd_varlen", lib().radial_attn_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), seq, mask.batch, mask.row_ptr.data_ptr(),
        mask.col_idx.data_ptr(), None if mask.pairs is None else mask.pairs.data_ptr(), npr,
        float(scale), elem_s, elem_w0, elem_gw, H, D, q.stride(1), q.stride(0), stream))
    return out


def attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    do: torch.Tensor, lse: torch.Tensor, mask: VarlenMask,
                    scale: float | None = None, element: bool = False):
    """Gradients (dq, dk, dv) of attn_fwd_varlen on a packed batch [total_tokens, H, D],
    from its output `o` and lse [H, total_tokens]. Asynchronous on torch's current
    stream."""
    if q.dim() != 3 or any(t.shape != q.shape for t in (k, v, o, do)):
        raise ValueError("q, k, v, o, do must share the shape [total_tokens, H, D]")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v, o, do)):
        raise TypeError("q, k, v, o, do must be bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in (k, v, o, do, lse)):
        raise ValueError("every tensor must be on the same GPU")
    if any(t.stride() != q.stride() for t in (k, v, o, do)) or q.stride(-1) != 1:
        raise ValueError("q, k, v, o, do must share strides with a contiguous last axis")
    total, H, D = q.shape
    if isinstance(mask, VarlenRuleMask):
        mask = mask.built(q.device)
    if sum(mask.seq_tokens) != total:
        raise ValueError("the samples' lengths must add up to q's token count")
    if lse.shape != (H, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [H, total_tokens] output")
    if mask.col_ptr is None or mask.row_idx is None:
        raise ValueError("the mask has no transposed rows (build it with concat_masks)")
    if any(t.device != q.device for t in (mask.row_ptr, mask.col_idx, mask.col_ptr,
                                          mask.row_idx)):
        raise ValueError("the mask must be on the same device as q (VarlenMask.to(device))")
    if scale is None:
        scale = D ** -0.5
    elem_s, elem_w0, elem_gw = _element_args(mask, element)
    dq, dk, dv = (torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
                  for _ in range(3))
    delta = torch.empty(2, H, total, dtype=torch.float32, device=q.device)  # D_i, base-2 lse
    seq = (ctypes.c_int32 * mask.batch)(*mask.seq_tokens)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    table = mask.element_table if element else None
    if table is not None and mask.symmetric():
        _check_table(table, mask.col_idx.numel(), q.device)
        _check("radial_attn_bwd_varlen_element_table", lib().radial_attn_bwd_varlen_element_table(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), seq,
            mask.batch, mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(),
            mask.col_ptr.data_ptr(), mask.row_idx.data_ptr(), float(scale), table.data_ptr(),
            H, D, q.stride(1), q.stride(0), stream))
        return dq, dk, dv
    _check("radial_attn_bwd_varlen", lib().radial_attn_bwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), seq, mask.batch,
        mask.row_ptr.data_ptr(), mask.col_idx.data_ptr(), mask.col_ptr.data_ptr(),
        mask.row_idx.data_ptr(), float(scale), elem_s, elem_w0, elem_gw, H, D, q.stride(1),
        q.stride(0), stream))
    return dq, dk, dv


class RadialAttentionVarlenFunction(torch.autograd.Function):
    """attn_fwd_varlen with its backward (attn_bwd_varlen) for autograd."""

    @staticmethod
    def forward(ctx, q, k, v, mask, scale, element):
        total, H, _ = q.shape
        lse = torch.empty(H, total, dtype=torch.float32, device=q.device)
        o = attn_fwd_varlen(q, k, v, mask, scale=scale, lse=lse, element=element)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.mask, ctx.scale, ctx.element = mask, scale, element
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd_varlen(q, k, v, o, _like_q(do, q), lse, ctx.mask,
                                     scale=ctx.scale, element=ctx.element)
        return dq, dk, dv, None, None, None


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: VarlenMask,
                     scale: float | None = None, element: bool = False) -> torch.Tensor:
    """Radial attention on a packed varlen batch with autograd support."""
    return RadialAttentionVarlenFunction.apply(q, k, v, mask, scale, element)
