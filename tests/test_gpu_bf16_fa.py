"""GPU parity of the BF16 FlashAttention forward (BF16 Q, K and V; BF16 scores summed in FP32,
online softmax, BF16 P V): the LP-FA4 README's BF16 flash_attn_func path, the baseline that the
MXFP8 forward is compared with. The oracle is the same plain two-pass attention on the BF16
values (no quantization), with P rounded to BF16.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_custom, make_workload
from helpers import bf16_to_device, compare, assert_within, f64

pytestmark = pytest.mark.gpu


def _run(wl, **kw):
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q, k, v = bf16_to_device(wl.q_bits), bf16_to_device(wl.k_bits), bf16_to_device(wl.v_bits)
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="bf16", **kw)
    torch.cuda.synchronize()
    return out, lse


def _ref(wl, rows=None, **kw):
    return oracle.attention_varlen(f64(wl.q_bits), f64(wl.k_bits), f64(wl.v_bits), wl.cu_q, wl.cu_k,
                                   pv_mode="bf16", rows=rows, **kw)


SMALL = [
    ([300], [300], 2),
    ([1], [1], 1),
    ([128], [128], 1),
    ([129, 5, 260], [70, 333, 1], 3),          # Lq != Lk, ragged tails in both
    ([0, 200, 0, 17], [3, 150, 0, 400], 2),     # empty sequences
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_parity(case):
    lq, lk, h = SMALL[case]
    wl = make_custom(lq, lk, heads=h, seed=400 + case)
    out, lse = _run(wl)
    assert_within(compare(out, lse, _ref(wl)))


def test_dense_sampled():
    wl = make_workload("dense", seed=0)
    out, lse = _run(wl)
    assert_within(compare(out, lse, _ref(wl, rows={0: np.arange(0, 2048, 7)})))


def test_varlen_sampled():
    """Packed varlen with x20 outliers: |O| reaches ~60, where O may exceed 2e-2 by one BF16 ulp of
    the reference (the output's own rounding and that of the BF16 probabilities)."""
    wl = make_workload("varlen", seed=0)
    out, lse = _run(wl)
    rows = {r: np.arange(0, lq, 13) for r, lq in enumerate(wl.lengths_q) if lq > 0}
    assert_within(compare(out, lse, _ref(wl, rows=rows)), bf16_allowance=True)


def test_cross_sampled():
    wl = make_workload("cross", seed=0)
    out, lse = _run(wl)
    st = compare(out, lse, _ref(wl, rows={0: np.arange(0, 4096, 61)}))
    assert_within(st)
    assert st["o_rel"] < 0.004, st


def test_descales():
    wl = make_custom([260, 70], [190, 300], heads=3, seed=410)
    rng = np.random.default_rng(411)
    qd, kd = np.exp2(rng.uniform(-4, 2, (2, 3))), np.exp2(rng.uniform(-4, 2, (2, 3)))
    t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")
    out, lse = _run(wl, q_descale=t(qd), k_descale=t(kd))
    assert_within(compare(out, lse, _ref(wl, q_descale=qd, k_descale=kd)))


def test_packed_equals_each_sequence_alone():
    wl = make_custom([150, 40, 260], [200, 33, 129], heads=2, seed=420)
    out, lse = _run(wl)
    for r in range(3):
        one = make_custom([wl.lengths_q[r]], [wl.lengths_k[r]], heads=2, seed=0)
        one.q_bits = wl.q_bits[wl.cu_q[r]:wl.cu_q[r + 1]]
        one.k_bits = wl.k_bits[wl.cu_k[r]:wl.cu_k[r + 1]]
        one.v_bits = wl.v_bits[wl.cu_k[r]:wl.cu_k[r + 1]]
        o1, l1 = _run(one)
        assert torch.equal(o1, out[wl.cu_q[r]:wl.cu_q[r + 1]])
        assert torch.equal(l1, lse[:, wl.cu_q[r]:wl.cu_q[r + 1]])
