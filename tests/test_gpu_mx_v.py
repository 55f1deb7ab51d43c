"""GPU parity of the MX-scaled V path: the token-orientation quantizer (bit-exact against the
oracle) and the attention forward with V in MXFP8 along tokens (pv_mode "mx", within the
attention tolerances), plus the exact identity that ties it to the fp8 mode.

LP-FA4 README, section "MXFP8 forward and backward": V is quantized like Q and K and keeps
both hardware orientations; the forward's P V product contracts over tokens, so its V operand
has one E8M0 scale per 32 tokens of each head_dim column.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_custom, make_workload, bf16_bits_to_f32
from helpers import (bf16_to_device, oracle_operands, compare, assert_within, f64, record, pv_rounding_bound,
                     assert_within_bound)
from test_gpu_quant import _sweep_tensor

pytestmark = pytest.mark.gpu


def _gpu_tokens(x: torch.Tensor, lengths, mode):
    meta = lp.VarlenMeta.from_lengths(lengths, x.device)
    mx = lp.quantize_mxfp8_varlen_tokens(x, meta, scaling_mode=mode)
    torch.cuda.synchronize()
    return mx.payload.cpu().numpy(), mx.scales.cpu().numpy()


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("anchor", [None, 448.0, 2.0 ** 100, 2.0 ** -126])
def test_tokens_bf16_sweep(mode, anchor):
    """Every finite BF16 pattern, grouped into 32-token column blocks next to anchors."""
    rng = np.random.default_rng(300 + (0 if anchor is None else int(np.log2(anchor)) + 200))
    bits = _sweep_tensor(anchor, rng)
    t = bits.shape[0]
    payload, scales = _gpu_tokens(bf16_to_device(bits), [t], mode)
    rp, rs, _ = oracle.mx_quantize_varlen_tokens(f64(bits), np.array([0, t]), mode)
    assert np.array_equal(scales, rs)
    assert np.array_equal(payload, rp)


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_tokens_varlen_fp32_and_padding(mode):
    """FP32 over a wide exponent range; ragged sequences (last blocks with fewer than 32 tokens,
    rows past each sequence's last block, an empty sequence)."""
    rng = np.random.default_rng(310)
    lengths = [45, 0, 128, 7, 300]
    t, h = sum(lengths), 3
    x = rng.standard_normal((t, h, 128)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=(t, h, 1))).astype(np.float32)
    x[rng.random(x.shape) < 0.01] = 0.0
    payload, scales = _gpu_tokens(torch.from_numpy(x).cuda(), lengths, mode)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rp, rs, _ = oracle.mx_quantize_varlen_tokens(x.astype(np.float64), cu, mode)
    assert np.array_equal(scales, rs)
    assert np.array_equal(payload, rp)


def test_tokens_strided_input():
    wl = make_custom([200], [200], heads=4, seed=311)
    full = bf16_to_device(wl.q_bits)
    x = full[:, 1:3, :]                                   # head stride 128, token stride 512
    payload, scales = _gpu_tokens(x, [200], "rceil")
    rp, rs, _ = oracle.mx_quantize_varlen_tokens(f64(wl.q_bits)[:, 1:3, :], np.array([0, 200]))
    assert np.array_equal(scales, rs) and np.array_equal(payload, rp)


def _run(wl, **kw):
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk)
    v = lp.quantize_mxfp8_varlen_tokens(bf16_to_device(wl.v_bits), mk)
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="mx", **kw)
    torch.cuda.synchronize()
    return out, lse, v


SMALL = [
    ([300], [300], 2),
    ([1], [1], 1),
    ([129, 5, 260], [70, 333, 1], 3),          # Lq != Lk, ragged tails in both
    ([0, 200, 0, 17], [3, 150, 0, 400], 2),     # empty sequences
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_parity(case):
    lq, lk, h = SMALL[case]
    wl = make_custom(lq, lk, heads=h, seed=320 + case)
    out, lse, v = _run(wl)
    ops = oracle_operands(wl, "mx")
    assert np.array_equal(v.payload.cpu().numpy(), ops["pv"]) and np.array_equal(v.scales.cpu().numpy(), ops["sv"])
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="mx")
    assert_within(compare(out, lse, ref))


def test_dense_sampled():
    wl = make_workload("dense", seed=0)
    out, lse, _ = _run(wl)
    ops = oracle_operands(wl, "mx")
    rows = {0: np.arange(0, 2048, 7)}
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="mx", rows=rows)
    assert_within(compare(out, lse, ref))


def test_varlen_no_outliers_sampled():
    """The varlen workload's sequence lengths with N(0, 1) data: element-wise tolerances."""
    lengths = make_workload("varlen", seed=0).lengths_q
    wl = make_custom(lengths, lengths, heads=16, seed=350)
    out, lse, _ = _run(wl)
    ops = oracle_operands(wl, "mx")
    rows = {r: np.arange(0, lq, 29) for r, lq in enumerate(wl.lengths_q) if lq > 0}
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="mx", rows=rows)
    assert_within(compare(out, lse, ref))


def test_varlen_outliers_sampled():
    """Packed varlen with x20 outliers. P is unscaled E4M3 here, as in the fp8 mode: below 2^-6 it
    falls into E4M3's subnormal range, whose steps are 2^-9 absolute. The oracle rounds P against
    the final row maximum and the kernel against its running one (up to 2^8 lower, so its small
    probabilities stay normal), and on rows whose softmax spreads over thousands of keys with x20
    V outliers the two differ by more than the plain absolute bound. Every sampled element is
    held instead to the bound derived from the oracle's unrounded probabilities
    (helpers.pv_rounding_bound: the oracle's own rounding error, exactly, plus the largest the
    kernel's rounding at any reference maximum it may use can add); LSE, which the rounding does
    not touch, keeps the plain bound."""
    wl = make_workload("varlen", seed=0)
    out, lse, _ = _run(wl)
    ops = oracle_operands(wl, "mx")
    rows = {r: np.arange(0, lq, 13) for r, lq in enumerate(wl.lengths_q) if lq > 0}
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="mx", rows=rows)
    st = compare(out, lse, ref)
    record(st)
    assert st["lse_max"] <= 1e-3, st
    bound = pv_rounding_bound(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, rows, "mx", ref)
    assert_within_bound(out, ref, bound)


def test_unit_scales_equal_fp8_mode_bit_for_bit():
    """V whose 32-token column blocks all have maxima of exactly 448 and E4M3 values: every V
    scale is 1 (byte 0x7F) and the payload is the plain E4M3 cast, so the mx mode must give the
    fp8 mode's output bits exactly."""
    rng = np.random.default_rng(330)
    lq, lk, h = [200, 64], [300, 97], 2
    wl = make_custom(lq, lk, heads=h, seed=331)
    tk = sum(lk)
    codes = rng.integers(0, 0x7E, size=(tk, h, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(tk, h, 128)) << 7).astype(np.uint8)
    v = oracle.e4m3_decode(codes)
    c0 = 0
    for L in lk:
        for b in range(0, L, 32):
            v[c0 + b] = 448.0
        c0 += L
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(lq, dev)
    mk = lp.VarlenMeta.from_lengths(lk, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk)
    vt = torch.from_numpy(v.astype(np.float32)).to(dev)
    vmx = lp.quantize_mxfp8_varlen_tokens(vt, mk)
    v8 = lp.cast_e4m3(vt)
    torch.cuda.synchronize()
    assert np.array_equal(vmx.payload.cpu().numpy(), v8.cpu().numpy())
    assert np.all(vmx.scales.cpu().numpy() == 0x7F)   # real blocks (e = 0) and the rows past them
    o1, l1 = lp.lp_attn_varlen_fwd(q, k, vmx, mq, mk, pv_mode="mx")
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = lp.lp_attn_varlen_fwd(q, k, v8, mq, mk, pv_mode="fp8")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_packed_equals_each_sequence_alone():
    wl = make_custom([150, 40, 260], [200, 33, 129], heads=2, seed=340)
    out, lse, _ = _run(wl)
    for r in range(3):
        one = make_custom([wl.lengths_q[r]], [wl.lengths_k[r]], heads=2, seed=0)
        one.q_bits = wl.q_bits[wl.cu_q[r]:wl.cu_q[r + 1]]
        one.k_bits = wl.k_bits[wl.cu_k[r]:wl.cu_k[r + 1]]
        one.v_bits = wl.v_bits[wl.cu_k[r]:wl.cu_k[r + 1]]
        o1, l1, _ = _run(one)
        assert torch.equal(o1, out[wl.cu_q[r]:wl.cu_q[r + 1]])
        assert torch.equal(l1, lse[:, wl.cu_q[r]:wl.cu_q[r + 1]])
