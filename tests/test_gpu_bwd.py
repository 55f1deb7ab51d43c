"""GPU parity of the attention backward on MXFP8 operands (lp_attn_varlen_bwd) against the oracle.

Inputs: the GPU quantizers produce both orientations of Q and K and the head_dim orientation of
V; the oracle quantizes the same BF16 values with its own code. The forward's output and LSE
that the backward consumes come from the oracle's forward (rounded to BF16 and FP32), so no
oracle input comes from the GPU. For the large workloads the oracle computes a subset of heads;
the GPU's other heads get O = 0 and LSE = 1e4 (P = 0, D = 0), so their gradients must be zero.

Tolerances (per head and tensor, against the oracle's float64 gradients, which round P and dS
to BF16 as the kernel does): max |err| <= 1e-2 * max |ref| and ||err|| <= 5e-3 * ||ref||. The
kernel differs from the oracle by FP32 sums and exp2, which flip an occasional BF16 rounding of
P or dS by one unit (2^-7 of that term), and by the BF16 rounding of the outputs (relative
2^-8 at most, ~2^-8/sqrt(3) in norm). MXFP8 dK/dV: each element within an E4M3 half step of the
reference at the GPU's block scale (|x|/16, or 2^(e-10) below E4M3's normal range; with FLOOR
scales plus the saturation of magnitudes above 448 * 2^e) plus the BF16 bound; at least 99% of
the scale bytes equal the oracle's quantization of its own gradients, and the rest differ by one.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import f32_to_bf16_bits, make_custom, make_output_grad, make_workload
from helpers import bf16_to_device, f64

pytestmark = pytest.mark.gpu

G_MAX_REL = 1e-2
G_NORM_REL = 5e-3


def _deq_d(x, cu):
    pay, sc, cs = oracle.mx_quantize_varlen(x, cu)
    return oracle.mx_dequantize_varlen(pay, sc, cu, cs)


def _deq_t(x, cu):
    pay, sc, cs = oracle.mx_quantize_varlen_tokens(x, cu)
    return oracle.mx_dequantize_varlen_tokens(pay, sc, cu, cs)


class Case:
    """One backward problem: GPU results for every head, oracle gradients for heads `sel`."""

    def __init__(self, wl, seed, sel=None, softmax_scale=None, mx=False, mode="rceil"):
        h = wl.num_heads
        self.sel = list(range(h)) if sel is None else list(sel)
        self.wl, self.mx, self.mode = wl, mx, mode
        tau = 128 ** -0.5 if softmax_scale is None else softmax_scale
        cu_q, cu_k = wl.cu_q, wl.cu_k
        xq, xk, xv = (f64(b)[:, self.sel] for b in (wl.q_bits, wl.k_bits, wl.v_bits))
        qd, kd, vd = _deq_d(xq, cu_q), _deq_d(xk, cu_k), _deq_d(xv, cu_k)
        qt, kt = _deq_t(xq, cu_q), _deq_t(xk, cu_k)
        fwd = oracle.attention_varlen(qd, kd, vd, cu_q, cu_k, pv_mode="bf16", softmax_scale=tau)
        tq = int(cu_q[-1])
        o_bits = np.zeros((tq, h, 128), dtype=np.uint16)
        o_bits[:, self.sel] = f32_to_bf16_bits(fwd.out.astype(np.float32))
        lse = np.full((h, tq), 1e4, dtype=np.float32)
        lse[self.sel] = fwd.lse.astype(np.float32)
        do_bits = make_output_grad(tq, h, seed)
        self.ref = oracle.attention_varlen_bwd(qd, kd, vd, qt, kt, f64(o_bits)[:, self.sel],
                                               f64(do_bits)[:, self.sel], lse[self.sel].astype(np.float64),
                                               cu_q, cu_k, softmax_scale=tau)
        self.meta_q = lp.VarlenMeta.from_lengths(wl.lengths_q)
        self.meta_k = lp.VarlenMeta.from_lengths(wl.lengths_k)
        q, k, v = (bf16_to_device(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
        self.ops = (lp.quantize_mxfp8_varlen(q, self.meta_q), lp.quantize_mxfp8_varlen(k, self.meta_k),
                    lp.quantize_mxfp8_varlen(v, self.meta_k), lp.quantize_mxfp8_varlen_tokens(q, self.meta_q),
                    lp.quantize_mxfp8_varlen_tokens(k, self.meta_k))
        self.out, self.dout = bf16_to_device(o_bits), bf16_to_device(do_bits)
        self.lse = torch.from_numpy(lse).cuda()
        self.tau = tau

    def run(self):
        res = lp.lp_attn_varlen_bwd(*self.ops, self.out, self.dout, self.lse, softmax_scale=self.tau,
                                    output_mxfp8_dkv=self.mx, scaling_mode=self.mode)
        torch.cuda.synchronize()
        return res


def _check(name, got, ref, sel):
    """got: (T, H, 128) float64 over all heads; ref: (T, len(sel), 128)."""
    others = [hh for hh in range(got.shape[1]) if hh not in sel]
    if others:
        assert np.all(got[:, others] == 0), f"{name}: heads outside the oracle's subset are not zero"
    g = got[:, sel]
    for j, hh in enumerate(sel):
        err = np.abs(g[:, j] - ref[:, j])
        m = np.abs(ref[:, j]).max()
        if m == 0:
            assert err.max() == 0, name
            continue
        print(f"{name} head {hh}: max err {err.max():.3e} ({err.max() / m:.2e} of max), "
              f"norm rel {np.linalg.norm(err) / np.linalg.norm(ref[:, j]):.2e}")
        assert err.max() <= G_MAX_REL * m, f"{name} head {hh}: max err {err.max()} vs max |ref| {m}"
        assert np.linalg.norm(err) <= G_NORM_REL * np.linalg.norm(ref[:, j]), f"{name} head {hh}: norm"


def _bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_all(case, res):
    dq, dk, dv = res
    _check("dq", _bf16(dq), case.ref.dq, case.sel)
    if case.mx:
        for name, t, ref in (("dk", dk, case.ref.dk), ("dv", dv, case.ref.dv)):
            _check_mx(name, t, ref, case)
    else:
        _check("dk", _bf16(dk), case.ref.dk, case.sel)
        _check("dv", _bf16(dv), case.ref.dv, case.sel)


def _check_mx(name, t, ref, case):
    pay = t.payload.cpu()
    sc = t.scales.cpu().numpy()
    cu_k = case.wl.cu_k
    cs = np.asarray(case.meta_k.cu_scale_host)
    codes = pay.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)  # library decoding
    rows = np.concatenate([np.arange(cs[i], cs[i] + cu_k[i + 1] - cu_k[i]) for i in range(len(cu_k) - 1)]).astype(int)
    pad = np.setdiff1d(np.arange(sc.shape[0]), rows)
    assert np.all(sc[pad] == 0x7F), f"{name}: pad scale rows"
    e = sc[rows].astype(np.int64) - 127                                     # (Tk, H, 4)
    deq = codes * np.repeat(np.ldexp(1.0, e), 32, axis=2)
    others = [hh for hh in range(deq.shape[1]) if hh not in case.sel]
    if others:
        assert np.all(deq[:, others] == 0), f"{name}: heads outside the oracle's subset are not zero"
    _, rs, _ = oracle.mx_quantize_varlen(ref, cu_k, case.mode)
    rs_real = rs[rows].astype(np.int64)
    gs = sc[rows][:, case.sel].astype(np.int64)
    agree = np.mean(gs == rs_real)
    print(f"{name}: scale bytes equal to the oracle's on {agree:.4%} of blocks")
    assert agree >= 0.99 and np.all(np.abs(gs - rs_real) <= 1), f"{name}: scales"
    for j, hh in enumerate(case.sel):
        r = ref[:, j]
        m = np.abs(r).max()
        sc2 = np.ldexp(1.0, np.repeat(e[:, hh], 32, axis=1))
        # E4M3 half step, plus FLOOR's saturation of magnitudes above 448 * 2^e (RCEIL never saturates)
        step = np.maximum(np.abs(r) / 16, sc2 * 2.0 ** -10) + np.maximum(np.abs(r) - 448 * sc2, 0)
        err = np.abs(deq[:, hh] - r)
        bound = step * 1.07 + 1.07 * G_MAX_REL * m
        assert np.all(err <= bound), f"{name} head {hh}: max excess {(err - bound).max()}"


def test_small_ragged():
    wl = make_custom([1, 100, 257, 64], [130, 1, 300, 64], heads=3, seed=800)
    case = Case(wl, seed=801)
    _check_all(case, case.run())


def test_keys_without_queries():
    wl = make_custom([0, 70, 5], [50, 90, 128], heads=2, seed=802)
    case = Case(wl, seed=803)
    dq, dk, dv = case.run()
    assert torch.all(dk[:50] == 0) and torch.all(dv[:50] == 0)
    _check_all(case, (dq, dk, dv))


def test_softmax_scale_and_determinism():
    wl = make_custom([190], [333], heads=2, seed=804)
    case = Case(wl, seed=805, softmax_scale=0.05)
    a = case.run()
    _check_all(case, a)
    b = case.run()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_mxfp8_dkdv_small(mode):
    wl = make_custom([1, 100, 257], [130, 200, 300], heads=2, seed=806)
    case = Case(wl, seed=807, mx=True, mode=mode)
    _check_all(case, case.run())


def test_dense_full_size():
    """The benchmark's dense shape: 1 x 2048 tokens, 16 heads (oracle on heads 0 and 9)."""
    wl = make_workload("dense", seed=0)
    case = Case(wl, seed=808, sel=[0, 9])
    _check_all(case, case.run())


def test_dense_full_size_mxfp8_dkdv():
    wl = make_workload("dense", seed=0)
    case = Case(wl, seed=809, sel=[5], mx=True)
    _check_all(case, case.run())


def test_varlen_outliers():
    """Eight sequences of 128..4096 tokens with x20 outliers (oracle on head 3)."""
    wl = make_workload("varlen", seed=0)
    case = Case(wl, seed=810, sel=[3])
    _check_all(case, case.run())


def test_cross_scaled():
    """Queries and keys of different lengths (the cross workload with lengths divided by 8)."""
    wl = make_workload("cross", seed=0, scale_tokens=8)
    case = Case(wl, seed=811, sel=[0, 15])
    _check_all(case, case.run())


def test_mismatched_operands_are_rejected_before_launch():
    wl = make_custom([40, 70], [50, 90], heads=2, seed=812)
    case = Case(wl, seed=813)
    qd, kd, vd, qt, kt = case.ops
    other = make_custom([40, 70], [50, 90], heads=3, seed=814)
    k3 = lp.quantize_mxfp8_varlen(bf16_to_device(other.k_bits), lp.VarlenMeta.from_lengths(other.lengths_k))
    with pytest.raises(ValueError):   # K with 3 heads against Q with 2
        lp.lp_attn_varlen_bwd(qd, k3, vd, qt, kt, case.out, case.dout, case.lse)
    with pytest.raises(ValueError):   # Q's token orientation in place of K's
        lp.lp_attn_varlen_bwd(qd, kd, vd, qt, qt, case.out, case.dout, case.lse)
    with pytest.raises(ValueError):   # LSE of the wrong shape
        lp.lp_attn_varlen_bwd(qd, kd, vd, qt, kt, case.out, case.dout, case.lse[:, :10])
