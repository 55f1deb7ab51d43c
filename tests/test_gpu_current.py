"""GPU parity of per-tensor current scaling (amax -> s = amax / 448 -> E4M3(x / s)): bit-exact
codes and scale against the oracle; attention on current-scaled Q/K/V within the attention
tolerances; and an FP8 output with its own current scale, which keeps a small attention output
accurate where a unit scale does not (the negative control of the TensorRT-LLM TE-backend PR:
stale scales lose accuracy on the same inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_custom, make_workload, bf16_bits_to_f32
from helpers import bf16_to_device, compare, assert_within, f64

pytestmark = pytest.mark.gpu


def _check_cast(x: torch.Tensor, xs: np.ndarray):
    codes, s = lp.cast_e4m3_current(x)
    torch.cuda.synchronize()
    rc, rs = oracle.current_quantize(xs)
    assert float(s.item()) == float(rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_bf16_random():
    wl = make_custom([700], [700], heads=3, seed=600)
    _check_cast(bf16_to_device(wl.q_bits), bf16_bits_to_f32(wl.q_bits))


def test_fp32_wide_range_and_strided():
    rng = np.random.default_rng(601)
    x = (rng.standard_normal((257, 4, 128)) * np.exp2(rng.integers(-30, 10, size=(257, 4, 1)))).astype(np.float32)
    full = torch.from_numpy(x).cuda()
    _check_cast(full, x)
    _check_cast(full[:, 1:3, :], x[:, 1:3, :])           # head stride 128, token stride 512


@pytest.mark.parametrize("where", ["last", "first", "middle"])
def test_many_workgroups_ragged_tail(where):
    """4099 tokens x 5 heads: 327920 eight-element chunks, more than one pass of the 256
    amax workgroups' 4-deep stride loop (262144 chunks) with a ragged tail; the largest
    magnitude is planted where the partial maxima must carry it."""
    rng = np.random.default_rng(602)
    x = rng.standard_normal((4099, 5, 128)).astype(np.float32)
    pos = {"last": (4098, 4, 127), "first": (0, 0, 0), "middle": (2049, 2, 77)}[where]
    x[pos] = -37.5
    _check_cast(torch.from_numpy(x).cuda(), x)


def test_all_zero_and_empty():
    z = torch.zeros((40, 2, 128), dtype=torch.bfloat16, device="cuda")
    codes, s = lp.cast_e4m3_current(z)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and int(codes.sum().item()) == 0
    e = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    codes, s = lp.cast_e4m3_current(e)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and codes.shape == (0, 2, 128)


def _current_attention(wl):
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    (q, dq), (k, dk), (v, dv) = (lp.cast_e4m3_current(bf16_to_device(b)) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="fp8", q_descale=dq, k_descale=dk, v_descale=dv)
    torch.cuda.synchronize()
    n, h = len(wl.lengths_q), wl.num_heads
    ops = {}
    for name, bits in (("q", wl.q_bits), ("k", wl.k_bits), ("v", wl.v_bits)):
        codes, s = oracle.current_quantize(bf16_bits_to_f32(bits))
        ops[name] = (oracle.e4m3_decode(codes), np.full((n, h), np.float64(s)))
    ref = oracle.attention_varlen(ops["q"][0], ops["k"][0], ops["v"][0], wl.cu_q, wl.cu_k, pv_mode="fp8",
                                  q_descale=ops["q"][1], k_descale=ops["k"][1], v_descale=ops["v"][1])
    return out, lse, ref


def test_attention_on_current_scaled_operands():
    wl = make_custom([300, 200], [260, 330], heads=3, seed=610)
    out, lse, ref = _current_attention(wl)
    assert_within(compare(out, lse, ref))


def test_fp8_output_with_current_scale():
    """An attention output spread over many keys is small (|O| ~ std(V) / sqrt(keys)); here V has
    std 2^-4 and O stays below 2^-6, E4M3's smallest normal. Its current-scaled E4M3 copy keeps
    E4M3's relative precision; a cast at unit scale falls into the subnormal range (steps of
    2^-9) and loses it on the same values."""
    wl = make_custom([256], [8192], heads=2, seed=620)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk)
    v = bf16_to_device(wl.v_bits) * 0.0625        # exact: a power of two on BF16 values
    out, _ = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="bf16")
    codes, s = lp.cast_e4m3_current(out)
    unit = lp.cast_e4m3(out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    rc, rs = oracle.current_quantize(o)
    assert float(s.item()) == float(rs) and np.array_equal(codes.cpu().numpy(), rc)
    assert np.abs(o).max() < 2.0 ** -6           # a small output, as the page describes
    rel = lambda d: float(np.linalg.norm(d - o) / np.linalg.norm(o))
    cur = rel(oracle.e4m3_decode(codes.cpu().numpy()) * float(s.item()))
    stale = rel(oracle.e4m3_decode(unit.cpu().numpy()))
    assert cur < 0.03, cur                       # E4M3's relative rounding, std 2^-4/sqrt(3)
    assert stale > 4 * cur, (stale, cur)
