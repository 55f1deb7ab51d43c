"""Python binding of liblpfa: argument marshalling only, every step runs in the HIP kernels.

PyTorch provides device memory and the current stream; the library launches on that
stream and never allocates. The names follow the LP-FA4 README (section "MXFP8 forward
and backward"): ``VarlenMeta.from_lengths`` builds the packed-sequence metadata once on the
host, ``quantize_mxfp8_varlen`` makes the E4M3 payload plus per-32 E8M0 scales with
128-token-padded per-sequence scale storage, and ``lp_attn_varlen_fwd`` returns
``(out, lse)``.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple, Union

import torch

from . import _lib

HEAD_DIM = 128
PAD = 128

Descale = Union[None, float, torch.Tensor]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class VarlenMeta:
    """Packed variable-length metadata, built once from host lengths (dense = one uniform length).

    ``cu_seqlens`` are packed token offsets, ``cu_scale`` the offsets of each sequence's
    scale rows (each sequence padded to a multiple of 128 tokens).
    """

    lengths: Tuple[int, ...]
    cu_seqlens_host: Tuple[int, ...]
    cu_scale_host: Tuple[int, ...]
    cu_seqlens: torch.Tensor
    cu_scale: torch.Tensor
    device: torch.device = field(repr=False, default=None)

    @classmethod
    def from_lengths(cls, lengths: Sequence[int], device="cuda") -> "VarlenMeta":
        lengths = tuple(int(v) for v in lengths)
        if any(v < 0 for v in lengths):
            raise ValueError("sequence lengths must be non-negative")
        cu, cs = [0], [0]
        for v in lengths:
            cu.append(cu[-1] + v)
            cs.append(cs[-1] + -(-v // PAD) * PAD)
        if cu[-1] >= 2 ** 31 or cs[-1] >= 2 ** 31:
            raise ValueError("packed length exceeds int32 offsets")
        dev = torch.device(device)
        return cls(lengths, tuple(cu), tuple(cs),
                   torch.tensor(cu, dtype=torch.int32, device=dev),
                   torch.tensor(cs, dtype=torch.int32, device=dev), dev)

    @classmethod
    def dense(cls, batch: int, seqlen: int, device="cuda") -> "VarlenMeta":
        """Dense (batch, seqlen) attention as uniform packed offsets."""
        return cls.from_lengths([seqlen] * batch, device)

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    @property
    def total_tokens(self) -> int:
        return self.cu_seqlens_host[-1]

    @property
    def total_scale_rows(self) -> int:
        return self.cu_scale_host[-1]

    @property
    def max_seqlen(self) -> int:
        return max(self.lengths) if self.lengths else 0


@dataclass
class Mxfp8Tensor:
    """MXFP8 operand: E4M3 payload (T, H, 128) uint8 and E8M0 scales (sum P(L_i), H, 4) uint8.

    ``group_max`` (optional, (sum P(L_i) / 16, H) uint8): the largest scale byte of each 16-row
    group of the scale storage over its real rows (0 for a group of pad rows only), written by the
    quantizer. Used for K by the attention's precision guard (results are the same without it).
    ``deq`` (optional, (T, H, 128) BF16): the quantized values themselves (payload times the block
    scale), written by the quantizer on request (``with_deq``). Used for K by the BF16-V forward's
    tiles that fail the precision guard (results are the same without it)."""

    payload: torch.Tensor
    scales: torch.Tensor
    meta: VarlenMeta
    group_max: Optional[torch.Tensor] = None
    deq: Optional[torch.Tensor] = None


@dataclass
class Mxfp8TokensTensor:
    """MXFP8 along tokens (V for the ``pv_mode="mx"`` P V product): E4M3 payload (T, H, 128) uint8
    and E8M0 scales (sum P(L_i) / 32, H, 128) uint8, one per 32 consecutive tokens of a sequence
    per (head, column); rows past a sequence's last 32-token block hold 0x7F."""

    payload: torch.Tensor
    scales: torch.Tensor
    meta: VarlenMeta


def _check_rows(x: torch.Tensor, name: str) -> None:
    if x.dim() != 3 or x.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be (tokens, heads, {HEAD_DIM}), got {tuple(x.shape)}")
    if x.stride(2) != 1:
        raise ValueError(f"{name} must be contiguous along head_dim")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _fp_input(x: torch.Tensor) -> int:
    _check_rows(x, "x")
    if x.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    if x.dtype == torch.float32:
        return _lib.DTYPE_FP32
    raise ValueError("x must be bfloat16 or float32")


def _check_out(t: torch.Tensor, shape, dtype, device, name: str) -> None:
    if t.shape != shape or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device}")


def quantize_mxfp8_varlen(x: torch.Tensor, meta: VarlenMeta, scaling_mode: str = "rceil",
                          out: Optional[Mxfp8Tensor] = None, with_deq: bool = False) -> Mxfp8Tensor:
    """MXFP8-quantize packed (tokens, heads, 128) BF16/FP32 ``x`` (RCEIL default, FLOOR optional).

    ``out``: an Mxfp8Tensor of the right shapes to write into (reused buffers); a new one otherwise
    (its ``deq``, if set, is written too). ``with_deq``: a new tensor also carries ``deq``, the
    quantized values as BF16 (for K of the BF16-V forward on data that fails the precision guard).
    """
    mode = _lib.SCALING.get(scaling_mode)
    if mode is None:
        raise ValueError(f"scaling_mode must be one of {sorted(_lib.SCALING)}, got {scaling_mode!r}")
    dt = _fp_input(x)
    t, h, _ = x.shape
    if t != meta.total_tokens:
        raise ValueError(f"x has {t} tokens, metadata says {meta.total_tokens}")
    gshape = (meta.total_scale_rows // 16, h)
    if out is None:
        payload = torch.empty((t, h, HEAD_DIM), dtype=torch.uint8, device=x.device)
        scales = torch.empty((meta.total_scale_rows, h, 4), dtype=torch.uint8, device=x.device)
        group_max = torch.empty(gshape, dtype=torch.uint8, device=x.device)
        deq = torch.empty((t, h, HEAD_DIM), dtype=torch.bfloat16, device=x.device) if with_deq else None
        out = Mxfp8Tensor(payload, scales, meta, group_max, deq)
    else:
        _check_out(out.payload, (t, h, HEAD_DIM), torch.uint8, x.device, "out.payload")
        _check_out(out.scales, (meta.total_scale_rows, h, 4), torch.uint8, x.device, "out.scales")
        if out.group_max is not None:
            _check_out(out.group_max, gshape, torch.uint8, x.device, "out.group_max")
        if out.deq is not None:
            _check_out(out.deq, (t, h, HEAD_DIM), torch.bfloat16, x.device, "out.deq")
        if out.meta is not meta:
            out = Mxfp8Tensor(out.payload, out.scales, meta, out.group_max, out.deq)
    rc = _lib.load().mxfp8_quantize_varlen(
        x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, HEAD_DIM, meta.cu_seqlens.data_ptr(),
        meta.cu_scale.data_ptr(), meta.num_seqs, meta.total_scale_rows, mode, out.payload.data_ptr(),
        out.scales.data_ptr(), _ptr(out.group_max), _ptr(out.deq), _stream())
    if rc:
        _lib.check("mxfp8_quantize_varlen", rc)
    return out


def quantize_mxfp8_varlen_tokens(x: torch.Tensor, meta: VarlenMeta, scaling_mode: str = "rceil",
                                 out: Optional[Mxfp8TokensTensor] = None) -> Mxfp8TokensTensor:
    """MXFP8-quantize packed (tokens, heads, 128) BF16/FP32 ``x`` along tokens (blocks of 32
    consecutive tokens of a sequence, per head and column): the V operand of ``pv_mode="mx"``.

    ``out``: an Mxfp8TokensTensor of the right shapes to write into; a new one otherwise."""
    mode = _lib.SCALING.get(scaling_mode)
    if mode is None:
        raise ValueError(f"scaling_mode must be one of {sorted(_lib.SCALING)}, got {scaling_mode!r}")
    dt = _fp_input(x)
    t, h, _ = x.shape
    if t != meta.total_tokens:
        raise ValueError(f"x has {t} tokens, metadata says {meta.total_tokens}")
    sshape = (meta.total_scale_rows // 32, h, HEAD_DIM)
    if out is None:
        out = Mxfp8TokensTensor(torch.empty((t, h, HEAD_DIM), dtype=torch.uint8, device=x.device),
                                torch.empty(sshape, dtype=torch.uint8, device=x.device), meta)
    else:
        _check_out(out.payload, (t, h, HEAD_DIM), torch.uint8, x.device, "out.payload")
        _check_out(out.scales, sshape, torch.uint8, x.device, "out.scales")
        if out.meta is not meta:
            out = Mxfp8TokensTensor(out.payload, out.scales, meta)
    rc = _lib.load().mxfp8_quantize_varlen_tokens(
        x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, HEAD_DIM, meta.cu_seqlens.data_ptr(),
        meta.cu_scale.data_ptr(), meta.num_seqs, meta.total_scale_rows, mode, out.payload.data_ptr(),
        out.scales.data_ptr(), _stream())
    if rc:
        _lib.check("mxfp8_quantize_varlen_tokens", rc)
    return out


def prepare_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, meta_q: VarlenMeta, meta_k: VarlenMeta,
                scaling_mode: str = "rceil",
                out: Optional[Tuple[Mxfp8Tensor, Mxfp8Tensor, torch.Tensor]] = None
                ) -> Tuple[Mxfp8Tensor, Mxfp8Tensor, torch.Tensor]:
    """The fp8-PV forward's preparation in one launch: (quantize_mxfp8_varlen(q), quantize_mxfp8_varlen(k)
    with group maxima, cast_e4m3(v)), byte-identical to the three calls. q, k, v share dtype and
    strides. ``out``: (q_mx, k_mx, v_codes) buffers to write into."""
    mode = _lib.SCALING.get(scaling_mode)
    if mode is None:
        raise ValueError(f"scaling_mode must be one of {sorted(_lib.SCALING)}, got {scaling_mode!r}")
    dt = _fp_input(q)
    for t, name in ((k, "k"), (v, "v")):
        _check_rows(t, name)
        if t.dtype != q.dtype or t.stride()[:2] != q.stride()[:2]:
            raise ValueError(f"{name} must have q's dtype and strides")
    tq, h, _ = q.shape
    tk = k.shape[0]
    if tq != meta_q.total_tokens or tk != meta_k.total_tokens or v.shape[0] != tk or k.shape[1] != h or v.shape[1] != h:
        raise ValueError("q, k, v shapes disagree with the metadata")
    if meta_q.num_seqs != meta_k.num_seqs:
        raise ValueError("query and key metadata must have the same number of sequences")
    dev = q.device
    if out is None:
        qo = Mxfp8Tensor(torch.empty((tq, h, HEAD_DIM), dtype=torch.uint8, device=dev),
                         torch.empty((meta_q.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), meta_q)
        ko = Mxfp8Tensor(torch.empty((tk, h, HEAD_DIM), dtype=torch.uint8, device=dev),
                         torch.empty((meta_k.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), meta_k,
                         torch.empty((meta_k.total_scale_rows // 16, h), dtype=torch.uint8, device=dev))
        vo = torch.empty((tk, h, HEAD_DIM), dtype=torch.uint8, device=dev)
    else:
        qo, ko, vo = out
        _check_out(qo.payload, (tq, h, HEAD_DIM), torch.uint8, dev, "q payload")
        _check_out(qo.scales, (meta_q.total_scale_rows, h, 4), torch.uint8, dev, "q scales")
        _check_out(ko.payload, (tk, h, HEAD_DIM), torch.uint8, dev, "k payload")
        _check_out(ko.scales, (meta_k.total_scale_rows, h, 4), torch.uint8, dev, "k scales")
        if ko.group_max is not None:
            _check_out(ko.group_max, (meta_k.total_scale_rows // 16, h), torch.uint8, dev, "k group_max")
        _check_out(vo, (tk, h, HEAD_DIM), torch.uint8, dev, "v codes")
    rc = _lib.load().mxfp8_prepare_qkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, q.stride(0), q.stride(1), tq, tk, h, HEAD_DIM,
        meta_q.cu_seqlens.data_ptr(), meta_q.cu_scale.data_ptr(), meta_k.cu_seqlens.data_ptr(),
        meta_k.cu_scale.data_ptr(), meta_q.num_seqs, meta_q.total_scale_rows, meta_k.total_scale_rows, mode,
        qo.payload.data_ptr(), qo.scales.data_ptr(), ko.payload.data_ptr(), ko.scales.data_ptr(),
        None if ko.group_max is None else ko.group_max.data_ptr(), vo.data_ptr(), _stream())
    if rc:
        _lib.check("mxfp8_prepare_qkv", rc)
    return qo, ko, vo


def e4m3_group_max_shape(tokens: int, heads: int) -> Tuple[int, int]:
    """Shape of :func:`cast_e4m3`'s group maxima: one byte per 16 tokens and head."""
    return (-(-int(tokens) // 16), int(heads))


def cast_e4m3(x: torch.Tensor, out: Optional[torch.Tensor] = None,
              group_max_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unscaled E4M3 cast (fp8 PV mode's V; per-tensor FP8 Q, K, V): uint8 codes, same
    (tokens, heads, 128) shape, contiguous.

    ``out``: a contiguous uint8 tensor of that shape to write into; a new one otherwise.
    ``group_max_out``: optional contiguous uint8 tensor of :func:`e4m3_group_max_shape` that
    receives the largest code magnitude of every 16 tokens of each head; for a per-tensor K, pass
    it to :func:`lp_attn_varlen_fwd` as ``k_group_max`` (the precision guard's bound on |k|)."""
    dt = _fp_input(x)
    t, h, _ = x.shape
    if out is None:
        out = torch.empty((t, h, HEAD_DIM), dtype=torch.uint8, device=x.device)
    else:
        _check_out(out, (t, h, HEAD_DIM), torch.uint8, x.device, "out")
    if group_max_out is not None:
        _check_out(group_max_out, e4m3_group_max_shape(t, h), torch.uint8, x.device, "group_max_out")
    rc = _lib.load().lp_fp8_cast_e4m3(x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, HEAD_DIM,
                                      out.data_ptr(), _ptr(group_max_out), _stream())
    if rc:
        _lib.check("lp_fp8_cast_e4m3", rc)
    return out


def cast_e4m3_current(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-tensor current scaling to E4M3: (codes, descale) with descale = amax(|x|) / 448 (float32,
    1 for an all-zero tensor) as a (1, 1) float32 GPU tensor and codes = E4M3(x / descale). The
    descale plugs into :func:`lp_attn_varlen_fwd` as a per-tensor q/k/v descale, or dequantizes an
    FP8 output."""
    dt = _fp_input(x)
    t, h, _ = x.shape
    if out is None:
        out = torch.empty((t, h, HEAD_DIM), dtype=torch.uint8, device=x.device)
    else:
        _check_out(out, (t, h, HEAD_DIM), torch.uint8, x.device, "out")
    work = torch.empty((257,), dtype=torch.float32, device=x.device)   # LPFA_CURRENT_WORK_FLOATS
    descale = torch.empty((1, 1), dtype=torch.float32, device=x.device)
    rc = _lib.load().lp_fp8_cast_current(x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, HEAD_DIM,
                                         work.data_ptr(), out.data_ptr(), descale.data_ptr(), _stream())
    if rc:
        _lib.check("lp_fp8_cast_current", rc)
    return out, descale


def cast_e4m3_current_noalloc(x: torch.Tensor, out: torch.Tensor, descale: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """:func:`cast_e4m3_current` for callers that cannot allocate (HIP graph capture, serving loops):
    ``out`` (uint8, x's shape, contiguous) and ``descale`` (one float32 element) are given, and the
    library keeps its scratch in a static device array, so nothing is allocated. Calls that
    overlap on one GPU share that array and must be serialised."""
    dt = _fp_input(x)
    t, h, _ = x.shape
    _check_out(out, (t, h, HEAD_DIM), torch.uint8, x.device, "out")
    if descale.dtype != torch.float32 or descale.numel() != 1 or descale.device != x.device:
        raise ValueError("descale must be a one-element float32 tensor on x's device")
    rc = _lib.load().lp_fp8_cast_current_noalloc(x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, HEAD_DIM,
                                                 out.data_ptr(), descale.data_ptr(), _stream())
    if rc:
        _lib.check("lp_fp8_cast_current_noalloc", rc)
    return out, descale


def _as_codes(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError("FP8 operands must be uint8 codes or torch.float8_e4m3fn")
    return t


def _descale(d: Descale, num_seqs: int, heads: int, device) -> Tuple[Optional[torch.Tensor], int, int]:
    """A descale as (device fp32 tensor or None, stride over sequences, stride over heads).

    A host float equal to 1.0 becomes None (no descale): the kernel reads a missing descale
    as 1.0 through the same arithmetic, so this changes no bit of the output.
    """
    if d is None:
        return None, 0, 0
    if isinstance(d, (int, float)):
        if float(d) == 1.0:
            return None, 0, 0
        return torch.full((1, 1), float(d), dtype=torch.float32, device=device), 0, 0
    if not d.is_cuda or d.dtype != torch.float32:
        raise ValueError("descale tensors must be float32 GPU tensors")
    if d.dim() == 0:
        d = d.reshape(1, 1)
    if d.dim() != 2 or d.shape[0] not in (1, num_seqs) or d.shape[1] not in (1, heads):
        raise ValueError(f"descale must broadcast to (num_seqs={num_seqs}, heads={heads}), got {tuple(d.shape)}")
    s_seq = 0 if d.shape[0] == 1 else d.stride(0)
    s_head = 0 if d.shape[1] == 1 else d.stride(1)
    return d, s_seq, s_head


def longest_first_tile_order(meta_q: VarlenMeta, meta_k: VarlenMeta, heads: int) -> torch.Tensor:
    """Work order of 128-query tiles, most keys first, built once on the host from the lengths."""
    tiles = []
    for r, (lq, lk) in enumerate(zip(meta_q.lengths, meta_k.lengths)):
        for qt in range(-(-lq // 128)):
            for h in range(heads):
                tiles.append((lk, r, h, qt))
    tiles.sort(key=lambda t: (-t[0], t[1], t[3], t[2]))
    flat: List[int] = [v for _, r, h, qt in tiles for v in (r, h, qt)]
    return torch.tensor(flat, dtype=torch.int32, device=meta_q.device)


class AttnPlan:
    """A prepared attention call: sizes, metadata, scale, descales, work order and outputs are
    checked and marshalled once; each call then sets the operand pointers and launches.

    Same arguments and semantics as :func:`lp_attn_varlen_fwd`. ``mx`` selects block-scaled
    QK^T (operands are Mxfp8Tensor) or per-tensor FP8 (operands are raw E4M3 codes);
    ``qk_bf16`` the BF16 FlashAttention forward (BF16 q and k, ``mx=False``, ``pv_mode="bf16"``).
    Descale tensors are read at each launch, so they may be updated in place between calls.
    """

    def __init__(self, meta_q: VarlenMeta, meta_k: VarlenMeta, num_heads: int, pv_mode: str = "bf16",
                 mx: bool = True, softmax_scale: Optional[float] = None, q_descale: Descale = None,
                 k_descale: Descale = None, v_descale: Descale = None,
                 tile_order: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, qk_bf16: bool = False,
                 fp8_score_guard: Optional[float] = None):
        if qk_bf16 and (mx or pv_mode != "bf16"):
            raise ValueError("BF16 q/k (qk_bf16) need mx=False and pv_mode='bf16'")
        if pv_mode not in _lib.PV_MODES:
            raise ValueError(f"pv_mode must be one of {sorted(_lib.PV_MODES)}, got {pv_mode!r}")
        if meta_q.num_seqs != meta_k.num_seqs:
            raise ValueError("query and key metadata have different sequence counts")
        for lq, lk in zip(meta_q.lengths, meta_k.lengths):
            if lq > 0 and lk == 0:
                raise ValueError("a sequence with queries must have at least one key")
        if meta_q.device != meta_k.device or meta_q.device.type != "cuda":
            raise ValueError("metadata must live on one GPU")
        if pv_mode == "mx" and not mx:
            raise ValueError("pv_mode='mx' needs MX (block-scaled) Q and K")
        h = int(num_heads)
        if h < 1:
            raise ValueError("num_heads must be positive")
        dev = meta_q.device
        tq, tk = meta_q.total_tokens, meta_k.total_tokens
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
        if out is None:
            out = torch.empty((tq, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((h, tq), dtype=torch.float32, device=dev)
        if out.shape != (tq, h, HEAD_DIM) or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous bfloat16 (Tq, H, 128) tensor")
        if lse.shape != (h, tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 (H, Tq) tensor")
        qd, qss, qsh = _descale(q_descale, meta_q.num_seqs, h, dev)
        kd, kss, ksh = _descale(k_descale, meta_q.num_seqs, h, dev)
        vd, vss, vsh = _descale(v_descale, meta_q.num_seqs, h, dev)

        a = _lib.AttnArgs()
        a.struct_size = ctypes.sizeof(_lib.AttnArgs)
        a.pv_mode = _lib.PV_MODES[pv_mode]
        a.qk_bf16 = 1 if qk_bf16 else 0
        if mx:
            a.cu_scale_q, a.cu_scale_k = _ptr(meta_q.cu_scale), _ptr(meta_k.cu_scale)
        a.cu_seqlens_q, a.cu_seqlens_k = _ptr(meta_q.cu_seqlens), _ptr(meta_k.cu_seqlens)
        a.num_seqs = meta_q.num_seqs
        a.max_seqlen_q, a.max_seqlen_k = meta_q.max_seqlen, meta_k.max_seqlen
        a.total_q, a.total_k = tq, tk
        a.num_heads, a.head_dim = h, HEAD_DIM
        a.softmax_scale = float(softmax_scale)
        a.causal = 0
        if fp8_score_guard is not None:
            if not float(fp8_score_guard) != 0.0 or math.isnan(float(fp8_score_guard)):
                raise ValueError("fp8_score_guard must be a non-zero number (negative: never FP8 scores)")
            a.fp8_score_guard = float(fp8_score_guard)
        a.q_descale, a.k_descale, a.v_descale = _ptr(qd), _ptr(kd), _ptr(vd)
        a.q_descale_stride_seq, a.q_descale_stride_head = qss, qsh
        a.k_descale_stride_seq, a.k_descale_stride_head = kss, ksh
        a.v_descale_stride_seq, a.v_descale_stride_head = vss, vsh
        a.out, a.lse = _ptr(out), _ptr(lse)
        if tile_order is not None:
            if tile_order.dtype != torch.int32 or not tile_order.is_cuda or tile_order.numel() % 3:
                raise ValueError("tile_order must be a GPU int32 tensor of (seq, head, tile) triples")
            a.tile_order, a.num_tiles = _ptr(tile_order), tile_order.numel() // 3
        self._args = a
        self._ref = ctypes.byref(a)
        self._keep = (meta_q, meta_k, qd, kd, vd, tile_order)   # everything the struct points at
        self._fn = _lib.load().lp_attn_varlen_fwd
        self.meta_q, self.meta_k, self.num_heads, self.mx, self.pv_mode = meta_q, meta_k, h, bool(mx), pv_mode
        self.out, self.lse = out, lse
        self._qshape, self._kshape = (tq, h, HEAD_DIM), (tk, h, HEAD_DIM)
        self._vdtype = torch.bfloat16 if pv_mode == "bf16" else torch.uint8
        self.qk_bf16 = bool(qk_bf16)
        self._qkdtype = torch.bfloat16 if qk_bf16 else torch.uint8
        self._dev = out.device                    # indexed ("cuda:0"), as operand tensors report it

    def _operand(self, t: torch.Tensor, shape, dtype, name: str) -> None:
        if t.dtype == torch.float8_e4m3fn and dtype == torch.uint8:
            t = t.view(torch.uint8)
        if t.shape != shape or t.dtype != dtype or t.stride(2) != 1 or t.device != self._dev:
            raise ValueError(f"{name} must be a {dtype} tensor of shape {shape} on {self._dev}, contiguous "
                             f"along head_dim (got {t.dtype} {tuple(t.shape)} on {t.device})")

    def __call__(self, q: Union[Mxfp8Tensor, torch.Tensor], k: Union[Mxfp8Tensor, torch.Tensor],
                 v: torch.Tensor, timing: Optional[Tuple] = None,
                 k_group_max: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        a = self._args
        if self.mx:
            if not (isinstance(q, Mxfp8Tensor) and isinstance(k, Mxfp8Tensor)):
                raise ValueError("this plan is block-scaled: q and k must be Mxfp8Tensor")
            if k_group_max is not None:
                raise ValueError("k_group_max is for per-tensor K; an Mxfp8Tensor K carries its own group_max")
            if (q.meta is not self.meta_q and q.meta.lengths != self.meta_q.lengths) or \
                    (k.meta is not self.meta_k and k.meta.lengths != self.meta_k.lengths):
                raise ValueError("q/k were quantized with different sequence metadata")
            qp, kp = q.payload, k.payload
            a.q_scale, a.k_scale = q.scales.data_ptr(), k.scales.data_ptr()
            if k.group_max is not None:
                gm, gshape = k.group_max, (self.meta_k.total_scale_rows // 16, self.num_heads)
                if gm.shape != gshape or gm.dtype != torch.uint8 or not gm.is_contiguous() or gm.device != self._dev:
                    raise ValueError(f"k.group_max must be a contiguous uint8 tensor of shape {gshape} on {self._dev}")
                a.k_scale_group_max = gm.data_ptr()
            else:
                a.k_scale_group_max = None
            # K's BF16 values (from the quantizer) serve the BF16-V kernel's guard-failing tiles
            if k.deq is not None and self.pv_mode == "bf16":
                _check_out(k.deq, (self.meta_k.total_tokens, self.num_heads, HEAD_DIM), torch.bfloat16, self._dev, "k.deq")
                a.k_deq = k.deq.data_ptr()
            else:
                a.k_deq = None
            _check_out(q.scales, (self.meta_q.total_scale_rows, self.num_heads, 4), torch.uint8, self._dev, "q.scales")
            _check_out(k.scales, (self.meta_k.total_scale_rows, self.num_heads, 4), torch.uint8, self._dev, "k.scales")
        else:
            if isinstance(q, Mxfp8Tensor) or isinstance(k, Mxfp8Tensor):
                raise ValueError("this plan takes raw q and k (E4M3 codes, or BF16 with qk_bf16)")
            qp, kp = q, k
            if k_group_max is not None:
                if self.qk_bf16:
                    raise ValueError("k_group_max is for E4M3 K")
                _check_out(k_group_max, e4m3_group_max_shape(self.meta_k.total_tokens, self.num_heads), torch.uint8,
                           self._dev, "k_group_max")
                a.k_scale_group_max = k_group_max.data_ptr()
            else:
                a.k_scale_group_max = None
        self._operand(qp, self._qshape, self._qkdtype, "q")
        self._operand(kp, self._kshape, self._qkdtype, "k")
        if self.pv_mode == "mx":
            if not isinstance(v, Mxfp8TokensTensor):
                raise ValueError("pv_mode='mx' needs v as an Mxfp8TokensTensor (quantize_mxfp8_varlen_tokens)")
            if v.meta is not self.meta_k and v.meta.lengths != self.meta_k.lengths:
                raise ValueError("v was quantized with different sequence metadata")
            vs, sshape = v.scales, (self.meta_k.total_scale_rows // 32, self.num_heads, HEAD_DIM)
            if vs.shape != sshape or vs.dtype != torch.uint8 or not vs.is_contiguous() or vs.device != self._dev:
                raise ValueError(f"v.scales must be a contiguous uint8 tensor of shape {sshape} on {self._dev}")
            a.v_scale = vs.data_ptr()
            v = v.payload
        else:
            if isinstance(v, Mxfp8TokensTensor):
                raise ValueError("an Mxfp8TokensTensor V needs pv_mode='mx'")
            a.v_scale = None
        self._operand(v, self._kshape, self._vdtype, "v")
        a.q, a.k, a.v = qp.data_ptr(), kp.data_ptr(), v.data_ptr()
        a.q_stride_tok, a.q_stride_head = qp.stride(0), qp.stride(1)
        a.k_stride_tok, a.k_stride_head = kp.stride(0), kp.stride(1)
        a.v_stride_tok, a.v_stride_head = v.stride(0), v.stride(1)
        if timing is not None:
            st, sp = (int(getattr(e, "cuda_event", e) or 0) for e in timing)
            if not st or not sp:
                raise ValueError("timing events must exist: record each once before passing them")
            a.start_event, a.stop_event = st, sp
        else:
            a.start_event = a.stop_event = None
        rc = self._fn(self._ref, _stream())
        if rc:
            _lib.check("lp_attn_varlen_fwd", rc)
        return self.out, self.lse


def lp_attn_varlen_fwd(q: Union[Mxfp8Tensor, torch.Tensor], k: Union[Mxfp8Tensor, torch.Tensor],
                       v: torch.Tensor, meta_q: VarlenMeta, meta_k: VarlenMeta, pv_mode: str = "bf16",
                       softmax_scale: Optional[float] = None, q_descale: Descale = None,
                       k_descale: Descale = None, v_descale: Descale = None,
                       tile_order: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None,
                       timing: Optional[Tuple] = None,
                       k_group_max: Optional[torch.Tensor] = None,
                       fp8_score_guard: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Noncausal head_dim-128 attention forward over packed sequences -> (out BF16 (Tq,H,128), lse FP32 (H,Tq)).

    ``q``/``k`` are Mxfp8Tensor (block-scaled QK^T), raw E4M3 codes (per-tensor FP8 mode), or
    BF16 tensors (the BF16 FlashAttention forward: BF16 scores, needs ``pv_mode="bf16"``).
    ``v`` is BF16 for ``pv_mode="bf16"``, E4M3 codes for ``pv_mode="fp8"`` (unscaled, see
    :func:`cast_e4m3`) or an :class:`Mxfp8TokensTensor` for ``pv_mode="mx"`` (MX Q and K only). Descales are floats or fp32 tensors broadcastable to (num_seqs, heads).
    ``timing``: optional (start, stop) ``torch.cuda.Event`` pair with timing enabled, each
    recorded once before (so the handles exist); the kernel's dispatch stamps them, and
    ``start.elapsed_time(stop)`` is then the kernel's own duration.
    ``k_group_max``: per-tensor mode, the group maxima of K's cast (:func:`cast_e4m3`), which give
    the precision guard its bound on |k|. ``fp8_score_guard``: the guard's threshold (default 16;
    negative: never FP8 scores).
    """
    if pv_mode not in _lib.PV_MODES:
        raise ValueError(f"pv_mode must be one of {sorted(_lib.PV_MODES)}, got {pv_mode!r}")
    mx_q, mx_k = isinstance(q, Mxfp8Tensor), isinstance(k, Mxfp8Tensor)
    if mx_q != mx_k:
        raise ValueError("q and k must both be Mxfp8Tensor (MX mode) or both raw E4M3 (per-tensor mode)")
    qk_bf16 = not mx_q and q.dtype == torch.bfloat16
    if qk_bf16 and k.dtype != torch.bfloat16:
        raise ValueError("BF16 q needs BF16 k")
    if qk_bf16:
        qp, kp = q, k
    else:
        qp = q.payload if mx_q else _as_codes(q)
        kp = k.payload if mx_k else _as_codes(k)
    vt = v
    if pv_mode == "mx":
        if not isinstance(v, Mxfp8TokensTensor):
            raise ValueError("pv_mode='mx' needs v as an Mxfp8TokensTensor (quantize_mxfp8_varlen_tokens)")
        v = v.payload
    for t, name in ((qp, "q"), (kp, "k"), (v, "v")):
        _check_rows(t, name)
    if pv_mode == "bf16" and v.dtype != torch.bfloat16:
        raise ValueError("pv_mode='bf16' needs a bfloat16 V")
    if pv_mode == "fp8":
        v = _as_codes(v)
    if qp.shape[0] != meta_q.total_tokens or kp.shape[0] != meta_k.total_tokens or v.shape[0] != kp.shape[0]:
        raise ValueError("tensor token counts do not match the metadata")
    h = qp.shape[1]
    if kp.shape[1] != h or v.shape[1] != h:
        raise ValueError("q, k and v must have the same number of heads")
    plan = AttnPlan(meta_q, meta_k, h, pv_mode=pv_mode, mx=mx_q, softmax_scale=softmax_scale,
                    q_descale=q_descale, k_descale=k_descale, v_descale=v_descale, tile_order=tile_order,
                    out=out, lse=lse, qk_bf16=qk_bf16, fp8_score_guard=fp8_score_guard)
    return plan(q if mx_q else qp, k if mx_k else kp, vt if pv_mode == "mx" else v, timing=timing,
                k_group_max=k_group_max)


class BwdPlan:
    """A prepared :func:`lp_attn_varlen_bwd`: operands checked, outputs allocated and the C
    arguments marshalled once; each call launches the backward on the current stream and returns
    the same output objects (overwritten)."""

    def __init__(self, q: Mxfp8Tensor, k: Mxfp8Tensor, v: Mxfp8Tensor,
                 q_t: Mxfp8TokensTensor, k_t: Mxfp8TokensTensor,
                 out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                 softmax_scale: Optional[float] = None, output_mxfp8_dkv: bool = False,
                 scaling_mode: str = "rceil"):
        if scaling_mode not in _lib.SCALING:
            raise ValueError(f"scaling_mode must be one of {sorted(_lib.SCALING)}, got {scaling_mode!r}")
        if not all(isinstance(t, Mxfp8Tensor) for t in (q, k, v)):
            raise ValueError("q, k and v must be Mxfp8Tensor (quantize_mxfp8_varlen)")
        if not all(isinstance(t, Mxfp8TokensTensor) for t in (q_t, k_t)):
            raise ValueError("q_t and k_t must be Mxfp8TokensTensor (quantize_mxfp8_varlen_tokens)")
        meta_q, meta_k = q.meta, k.meta
        if v.meta.lengths != meta_k.lengths or q_t.meta.lengths != meta_q.lengths or k_t.meta.lengths != meta_k.lengths:
            raise ValueError("operands disagree on sequence lengths")
        if meta_q.num_seqs != meta_k.num_seqs:
            raise ValueError("query and key metadata must have the same number of sequences")
        for a_, b_ in zip(meta_q.lengths, meta_k.lengths):
            if a_ > 0 and b_ == 0:
                raise ValueError("a sequence with queries needs keys")
        for t, name in ((q.payload, "q"), (k.payload, "k"), (v.payload, "v"), (q_t.payload, "q_t"),
                        (k_t.payload, "k_t"), (out, "out"), (dout, "dout")):
            _check_rows(t, name)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        tq, h = q.payload.shape[0], q.payload.shape[1]
        tk = k.payload.shape[0]
        dev = q.payload.device
        if tq != meta_q.total_tokens or tk != meta_k.total_tokens:
            raise ValueError("token counts do not match the metadata")
        rq, rk = meta_q.total_scale_rows, meta_k.total_scale_rows
        u8 = torch.uint8
        for t, name, shape, dtype in ((out, "out", (tq, h, HEAD_DIM), torch.bfloat16),
                                      (dout, "dout", (tq, h, HEAD_DIM), torch.bfloat16),
                                      (lse, "lse", (h, tq), torch.float32),
                                      (k.payload, "k", (tk, h, HEAD_DIM), u8), (v.payload, "v", (tk, h, HEAD_DIM), u8),
                                      (q_t.payload, "q_t", (tq, h, HEAD_DIM), u8),
                                      (k_t.payload, "k_t", (tk, h, HEAD_DIM), u8),
                                      (q.scales, "q scales", (rq, h, 4), u8), (k.scales, "k scales", (rk, h, 4), u8),
                                      (v.scales, "v scales", (rk, h, 4), u8),
                                      (q_t.scales, "q_t scales", (rq // 32, h, HEAD_DIM), u8),
                                      (k_t.scales, "k_t scales", (rk // 32, h, HEAD_DIM), u8)):
            _check_out(t, shape, dtype, dev, name)
        if q.payload.dtype != u8:
            raise ValueError("q must hold E4M3 codes (uint8)")
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._keep = (q, k, v, q_t, k_t, out, dout, lse)
        self.work = torch.empty((_lib.bwd_work_bytes(tq, tk, h),), dtype=torch.uint8, device=dev)
        self.dq = torch.empty((tq, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.mx = bool(output_mxfp8_dkv)
        if self.mx:
            dk = torch.empty((tk, h, HEAD_DIM), dtype=torch.uint8, device=dev)
            dv = torch.empty((tk, h, HEAD_DIM), dtype=torch.uint8, device=dev)
            dks = torch.empty((meta_k.total_scale_rows, h, HEAD_DIM // 32), dtype=torch.uint8, device=dev)
            dvs = torch.empty((meta_k.total_scale_rows, h, HEAD_DIM // 32), dtype=torch.uint8, device=dev)
            self.dk, self.dv = Mxfp8Tensor(dk, dks, meta_k), Mxfp8Tensor(dv, dvs, meta_k)
        else:
            dk = torch.empty((tk, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
            dv = torch.empty((tk, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
            dks = dvs = None
            self.dk, self.dv = dk, dv
        a = _lib.BwdArgs()
        a.struct_size = ctypes.sizeof(_lib.BwdArgs)
        a.q, a.q_scale = _ptr(q.payload), _ptr(q.scales)
        a.k, a.k_scale = _ptr(k.payload), _ptr(k.scales)
        a.v, a.v_scale = _ptr(v.payload), _ptr(v.scales)
        a.q_t, a.q_t_scale = _ptr(q_t.payload), _ptr(q_t.scales)
        a.k_t, a.k_t_scale = _ptr(k_t.payload), _ptr(k_t.scales)
        a.out, a.dout, a.lse = _ptr(out), _ptr(dout), _ptr(lse)
        a.cu_seqlens_q, a.cu_seqlens_k = _ptr(meta_q.cu_seqlens), _ptr(meta_k.cu_seqlens)
        a.cu_scale_q, a.cu_scale_k = _ptr(meta_q.cu_scale), _ptr(meta_k.cu_scale)
        a.num_seqs, a.num_heads, a.head_dim, a.causal = meta_q.num_seqs, h, HEAD_DIM, 0
        a.total_q, a.total_k = tq, tk
        a.total_scale_rows_q, a.total_scale_rows_k = meta_q.total_scale_rows, meta_k.total_scale_rows
        a.softmax_scale = float(softmax_scale)
        a.output_mxfp8_dkv = 1 if self.mx else 0
        a.scaling_mode = _lib.SCALING[scaling_mode]
        a.work, a.dq, a.dk, a.dv = _ptr(self.work), _ptr(self.dq), _ptr(dk), _ptr(dv)
        a.dk_scale, a.dv_scale = _ptr(dks), _ptr(dvs)
        self._args = a
        self._ref = ctypes.byref(a)
        self._lib = _lib.load()

    def __call__(self):
        _lib.check("lp_attn_varlen_bwd", self._lib.lp_attn_varlen_bwd(self._ref, _stream()))
        return self.dq, self.dk, self.dv


def lp_attn_varlen_bwd(q: Mxfp8Tensor, k: Mxfp8Tensor, v: Mxfp8Tensor,
                       q_t: Mxfp8TokensTensor, k_t: Mxfp8TokensTensor,
                       out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                       softmax_scale: Optional[float] = None, output_mxfp8_dkv: bool = False,
                       scaling_mode: str = "rceil"):
    """Attention backward on MXFP8 operands -> (dq, dk, dv).

    ``q``, ``k``, ``v``: head_dim-orientation operands (:func:`quantize_mxfp8_varlen`);
    ``q_t``, ``k_t``: Q and K along tokens (:func:`quantize_mxfp8_varlen_tokens`); ``out`` and
    ``lse``: the forward's results; ``dout``: the output gradient (BF16 (Tq, H, 128)).
    The metadata comes from the operands (Q's for queries, K's for keys).
    Returns BF16 (Tq|Tk, H, 128) tensors, or with ``output_mxfp8_dkv`` dk and dv as
    :class:`Mxfp8Tensor` (E4M3 payload and E8M0 scales per 32-element block, K's metadata,
    ``scaling_mode`` RCEIL or FLOOR). dq is BF16 either way.
    """
    return BwdPlan(q, k, v, q_t, k_t, out, dout, lse, softmax_scale, output_mxfp8_dkv, scaling_mode)()
