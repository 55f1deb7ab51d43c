"""GPU parity of the one-launch preparation (prepare_qkv): byte-identical to the three separate
calls (Q and K quantizers, V cast) and to the oracle's quantizer and cast, including K's group
maxima (the largest scale byte over each 16-row group's real rows, 0 for pad rows only)."""
import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_custom, make_workload
from helpers import bf16_to_device, f64

pytestmark = pytest.mark.gpu


def _group_max(scales, cu, cs):
    rows, h, _ = scales.shape
    real = np.zeros(rows, dtype=bool)
    for i in range(len(cu) - 1):
        real[cs[i]:cs[i] + cu[i + 1] - cu[i]] = True
    m = np.where(real[:, None, None], scales, 0).max(axis=2)          # (rows, H)
    return m.reshape(rows // 16, 16, h).max(axis=1).astype(np.uint8)


def _check(wl, x_of=bf16_to_device, mode="rceil"):
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k)
    q, k, v = (x_of(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
    qo, ko, vo = lp.prepare_qkv(q, k, v, mq, mk, scaling_mode=mode)
    qs = lp.quantize_mxfp8_varlen(q, mq, scaling_mode=mode)
    ks = lp.quantize_mxfp8_varlen(k, mk, scaling_mode=mode)
    vs = lp.cast_e4m3(v)
    torch.cuda.synchronize()
    for a, b in ((qo.payload, qs.payload), (qo.scales, qs.scales), (ko.payload, ks.payload),
                 (ko.scales, ks.scales), (ko.group_max, ks.group_max), (vo, vs)):
        assert torch.equal(a, b)
    pq, sq, _ = oracle.mx_quantize_varlen(f64(wl.q_bits), wl.cu_q, mode)
    pk, sk, csk = oracle.mx_quantize_varlen(f64(wl.k_bits), wl.cu_k, mode)
    assert np.array_equal(qo.payload.cpu().numpy(), pq) and np.array_equal(qo.scales.cpu().numpy(), sq)
    assert np.array_equal(ko.payload.cpu().numpy(), pk) and np.array_equal(ko.scales.cpu().numpy(), sk)
    assert np.array_equal(ko.group_max.cpu().numpy(), _group_max(sk, wl.cu_k, csk))
    assert np.array_equal(vo.cpu().numpy(), oracle.e4m3_cast(f64(wl.v_bits)))


def test_ragged_with_empty_sequences():
    _check(make_custom([0, 100, 257, 1], [130, 0, 300, 64], heads=3, seed=900))


def test_floor_mode():
    _check(make_custom([77, 300], [129, 5], heads=2, seed=901), mode="floor")


def test_fp32_inputs():
    wl = make_custom([50, 140], [33, 260], heads=2, seed=902)
    _check(wl, x_of=lambda b: bf16_to_device(b).float())


@pytest.mark.parametrize("name", ["dense", "varlen"])
def test_workloads_full_size(name):
    _check(make_workload(name, seed=0))
