"""GPU parity of the MXFP8 quantizer and the unscaled E4M3 cast: bit-exact against the oracle.

Inputs: an exhaustive sweep of every finite BF16 pattern, laid out in 32-element blocks
both at their own scale and next to anchors that force other block exponents (so every
pattern meets RNE ties, subnormal codes and saturation); random FP32 over a wide exponent
range with subnormals and signed zeros; strided inputs; the workloads' own Q/K, including
the packed varlen one whose scale storage has pad rows; empty sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_workload, make_custom, bf16_bits_to_f32, f32_to_bf16_bits
from helpers import bf16_to_device, f64

pytestmark = pytest.mark.gpu

ANCHORS = [None, 448.0, 1.0, 1.7578125, 2.0 ** 20 * 448, 2.0 ** 100, 3.0e38, 2.0 ** -100, 2.0 ** -126,
           0.5, 1e-3, 7.0]


def _finite_bf16_bits():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return bits[np.isfinite(f)].astype(np.uint16)


def _sweep_tensor(anchor, rng):
    """(T, 1, 128) BF16 bits: every finite BF16 pattern once; element 0 of each block is the anchor."""
    bits = _finite_bf16_bits()
    rng.shuffle(bits)
    per = 31 if anchor is not None else 32
    nblk = -(-len(bits) // per)
    out = np.zeros((nblk, 32), dtype=np.uint16)
    flat = np.zeros(nblk * per, dtype=np.uint16)
    flat[:len(bits)] = bits
    if anchor is None:
        out[:] = flat.reshape(nblk, 32)
    else:
        a = np.float32(anchor).view(np.uint32) >> 16
        out[:, 0] = np.where(rng.random(nblk) < 0.5, a, a | 0x8000)
        out[:, 1:] = flat.reshape(nblk, 31)
    nblk4 = -(-nblk // 4) * 4
    full = np.zeros((nblk4, 32), dtype=np.uint16)
    full[:nblk] = out
    return full.reshape(-1, 1, 128)


def _gpu_quant(x: torch.Tensor, lengths, mode):
    meta = lp.VarlenMeta.from_lengths(lengths, x.device)
    mx = lp.quantize_mxfp8_varlen(x, meta, scaling_mode=mode)
    torch.cuda.synchronize()
    return mx.payload.cpu().numpy(), mx.scales.cpu().numpy()


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("anchor", ANCHORS)
def test_exhaustive_bf16_sweep(mode, anchor):
    rng = np.random.default_rng(100 + ANCHORS.index(anchor))
    bits = _sweep_tensor(anchor, rng)
    t = bits.shape[0]
    lengths = [t]
    x = bf16_to_device(bits)
    payload, scales = _gpu_quant(x, lengths, mode)
    rp, rs, _ = oracle.mx_quantize_varlen(f64(bits), np.array([0, t]), mode)
    assert np.array_equal(scales, rs)
    bad = np.nonzero(payload != rp)
    assert bad[0].size == 0, (bad[0][:5], payload[bad][:5], rp[bad][:5], f64(bits)[bad][:5])


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_random_fp32(mode):
    rng = np.random.default_rng(7)
    t, h = 300, 3
    x = rng.standard_normal((t, h, 128)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(t, h, 4)).repeat(32, axis=2)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] = 0.0
    x[rng.random(x.shape) < 0.01] = -0.0
    x[5, 1, :32] = 0.0                                           # an all-zero block
    x[6, 2, 32:64] = np.float32(1e-42) * np.arange(32)           # subnormal-only block
    assert np.all(np.isfinite(x))
    lengths = [100, 0, 77, 123]
    xg = torch.from_numpy(x).cuda()
    payload, scales = _gpu_quant(xg, lengths, mode)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rp, rs, _ = oracle.mx_quantize_varlen(x.astype(np.float64), cu, mode)
    assert np.array_equal(scales, rs)
    assert np.array_equal(payload, rp)


def test_strided_input():
    """A (T, H, 128) view with token/head strides of a wider buffer (e.g. a fused QKV tensor)."""
    wl = make_custom([200, 57], [200, 57], heads=4, seed=3)
    qkv = torch.zeros((257, 3, 4, 128), dtype=torch.bfloat16, device="cuda")
    qkv[:, 1] = bf16_to_device(wl.q_bits)
    view = qkv[:, 1]
    assert view.stride() == (3 * 4 * 128, 128, 1)
    payload, scales = _gpu_quant(view, [200, 57], "rceil")
    rp, rs, _ = oracle.mx_quantize_varlen(f64(wl.q_bits), wl.cu_q, "rceil")
    assert np.array_equal(payload, rp) and np.array_equal(scales, rs)


@pytest.mark.parametrize("name", ["tiny", "dense", "varlen"])
def test_workload_qk(name):
    wl = make_workload(name, seed=0)
    for bits, lengths in ((wl.q_bits, wl.lengths_q), (wl.k_bits, wl.lengths_k)):
        payload, scales = _gpu_quant(bf16_to_device(bits), lengths, "rceil")
        cu = np.concatenate([[0], np.cumsum(lengths)])
        rp, rs, _ = oracle.mx_quantize_varlen(f64(bits), cu, "rceil")
        assert np.array_equal(payload, rp)
        assert np.array_equal(scales, rs)   # includes the 0x7F pad rows


@pytest.mark.parametrize("name", ["tiny", "varlen"])
def test_deq_output(name):
    """The quantizer's optional BF16 output (`with_deq`): the quantized values themselves, payload
    times 2^e, which have at most 4 significant bits and so are exact in BF16 here. Compared bit
    for bit with the oracle's dequantization of its own quantization; payload and scales are
    unchanged by the extra output. Pad rows have no tokens and write nothing."""
    wl = make_workload(name, seed=0)
    dev = torch.device("cuda")
    for bits, lengths in ((wl.q_bits, wl.lengths_q), (wl.k_bits, wl.lengths_k)):
        meta = lp.VarlenMeta.from_lengths(lengths, dev)
        mx = lp.quantize_mxfp8_varlen(bf16_to_device(bits), meta, with_deq=True)
        torch.cuda.synchronize()
        cu = np.concatenate([[0], np.cumsum(lengths)])
        rp, rs, _ = oracle.mx_quantize_varlen(f64(bits), cu, "rceil")
        assert np.array_equal(mx.payload.cpu().numpy(), rp) and np.array_equal(mx.scales.cpu().numpy(), rs)
        want = oracle.bf16_round(oracle.mx_dequantize_varlen(rp, rs, cu))
        got = mx.deq.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, want)


def test_cross_keys_full_size():
    """The cross-attention workload's 32768-token key tensor, every byte."""
    wl = make_workload("cross", seed=0)
    payload, scales = _gpu_quant(bf16_to_device(wl.k_bits), wl.lengths_k, "rceil")
    rp, rs, _ = oracle.mx_quantize_varlen(f64(wl.k_bits), wl.cu_k, "rceil")
    assert np.array_equal(payload, rp) and np.array_equal(scales, rs)


def test_empty_and_padding_only():
    x = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    meta = lp.VarlenMeta.from_lengths([0, 0], "cuda")
    mx = lp.quantize_mxfp8_varlen(x, meta)
    assert mx.payload.shape == (0, 2, 128) and mx.scales.shape == (0, 2, 4)
    x = torch.ones((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    mx = lp.quantize_mxfp8_varlen(x, lp.VarlenMeta.from_lengths([1], "cuda"))
    torch.cuda.synchronize()
    s = mx.scales.cpu().numpy()
    assert s.shape == (128, 2, 4) and np.all(s[0] == 119) and np.all(s[1:] == 0x7F)
    assert np.all(mx.payload.cpu().numpy() == 0x78)


def test_cast_exhaustive_bf16():
    bits = _finite_bf16_bits()
    n = -(-len(bits) // 128) * 128
    full = np.zeros(n, dtype=np.uint16)
    full[:len(bits)] = bits
    full = full.reshape(-1, 1, 128)
    y = lp.cast_e4m3(bf16_to_device(full))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), oracle.e4m3_cast(f64(full)))


def test_cast_fp32_and_strided():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((100, 2, 3, 128)) * np.exp2(rng.integers(-20, 12, (100, 2, 3, 1)))).astype(np.float32)
    xg = torch.from_numpy(x).cuda()[:, 1]                       # strided view (T, 3, 128)
    y = lp.cast_e4m3(xg)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), oracle.e4m3_cast(x[:, 1].astype(np.float64)))


def test_deterministic_repeat():
    wl = make_workload("dense", seed=1)
    x = bf16_to_device(wl.q_bits)
    a = _gpu_quant(x, wl.lengths_q, "rceil")
    b = _gpu_quant(x, wl.lengths_q, "rceil")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _group_max_from_scales(scales: np.ndarray, lengths) -> np.ndarray:
    """Largest scale byte of each (16-row group of the scale storage, head) over the group's real
    rows, 0 for a group of pad rows only."""
    rows, h, _ = scales.shape
    valid = np.zeros(rows, dtype=bool)
    start = 0
    for n in lengths:
        valid[start:start + n] = True
        start += -(-n // 128) * 128
    masked = np.where(valid[:, None, None], scales, 0).astype(np.uint8)
    return masked.reshape(rows // 16, 16, h, 4).max(axis=(1, 3))


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_group_max(mode, dtype):
    """The quantizer's per-(16-row group, head) maximum scale byte equals the maximum of the
    oracle's scale bytes over the group's real rows (pad rows, which hold 0x7F, excluded; 0 for a
    group of pad rows only), with ragged lengths, empty sequences and block exponents that differ
    from block to block."""
    rng = np.random.default_rng(12)
    lengths = [0, 300, 1, 128, 129, 0, 517]
    h = 3
    t = sum(lengths)
    x = rng.standard_normal((t, h, 128)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, size=(t, h, 4)).repeat(32, axis=2)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, size=(t, 1, 1))).astype(np.float32)   # rows differ too
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        xd, xo = bf16_to_device(bits), f64(bits)
    else:
        xd, xo = torch.from_numpy(x).cuda(), x.astype(np.float64)
    meta = lp.VarlenMeta.from_lengths(lengths, xd.device)
    mx = lp.quantize_mxfp8_varlen(xd, meta, scaling_mode=mode)
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    _, rs, _ = oracle.mx_quantize_varlen(xo, cu, mode)
    assert np.array_equal(mx.scales.cpu().numpy(), rs)
    got = mx.group_max.cpu().numpy()
    want = _group_max_from_scales(rs, lengths)
    assert got.shape == want.shape == (meta.total_scale_rows // 16, h)
    assert (want == 0).any()   # some groups hold pad rows only
    assert np.array_equal(got, want)
    # the maxima really differ across blocks and heads in this input
    assert len(np.unique(want)) > 3


def test_group_max_optional():
    """Without a group_max buffer the quantizer writes payload and scales only, bit-identically."""
    wl = make_custom([300, 77], [300, 77], heads=2, seed=13)
    x = bf16_to_device(wl.q_bits)
    meta = lp.VarlenMeta.from_lengths(wl.lengths_q, x.device)
    a = lp.quantize_mxfp8_varlen(x, meta)
    b = lp.quantize_mxfp8_varlen(x, meta, out=lp.Mxfp8Tensor(torch.empty_like(a.payload), torch.empty_like(a.scales), meta))
    torch.cuda.synchronize()
    assert b.group_max is None
    assert torch.equal(a.payload, b.payload) and torch.equal(a.scales, b.scales)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cast_group_max(dtype):
    """The cast's optional group maxima: per 16 tokens and head, the largest code magnitude, equal to
    the NumPy maximum over the oracle's codes (a ragged last group included); the codes are the
    plain cast's, bit for bit."""
    from helpers import e4m3_group_max
    rng = np.random.default_rng(1400)
    t, h = 1000 + 13, 3
    x = rng.standard_normal((t, h, 128)).astype(np.float32) * np.exp2(rng.integers(-12, 9, size=(t, h, 1))).astype(np.float32)
    x[rng.random(x.shape) < 1e-4] = 500.0                                 # saturating values
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()
    gm = torch.empty(lp.e4m3_group_max_shape(t, h), dtype=torch.uint8, device="cuda")
    codes = lp.cast_e4m3(xt, group_max_out=gm)
    plain = lp.cast_e4m3(xt)
    torch.cuda.synchronize()
    ref_codes = oracle.e4m3_cast(x.astype(np.float64))
    assert np.array_equal(codes.cpu().numpy(), ref_codes) and torch.equal(codes, plain)
    assert np.array_equal(gm.cpu().numpy(), e4m3_group_max(ref_codes))
