"""GPU parity of the fused attention forward against the oracle, plus the path's exact invariants.

Element-by-element comparisons at sizes the oracle finishes in seconds (several 128-query
and 128-key tiles with ragged tails), all five workloads at their real sizes on sampled
query rows (every row of the sampled ones: all heads, all 128 dims, all keys), and the bit
identities the pages fix: a unit descale equals no descale, a descale of 2 changes the
output, packed varlen equals each sequence alone, and the run is deterministic.
Tolerances (absolute, against the float64 oracle): O max 2e-2, O mean 2e-3, LSE max 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import precision_attention_mxfp8_amd as lp
from synth import make_workload, make_custom
from helpers import (bf16_to_device, oracle_operands, compare, assert_within, record, pv_rounding_bound,
                     assert_within_bound, e4m3_group_max)

pytestmark = pytest.mark.gpu


def _run_mx(wl, pv_mode, scaling="rceil", tile_order=False, **kw):
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq, scaling)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk, scaling)
    v = bf16_to_device(wl.v_bits)
    if pv_mode == "fp8":
        v = lp.cast_e4m3(v)
    order = lp.longest_first_tile_order(mq, mk, wl.num_heads) if tile_order else None
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode=pv_mode, tile_order=order, **kw)
    torch.cuda.synchronize()
    return out, lse, q, k


def _rows(wl, every):
    return {r: np.arange(0, lq, every) for r, lq in enumerate(wl.lengths_q) if lq > 0}


# ---------------------------------------------------------------- small, every element
SMALL = [
    ([300], [300], 2),
    ([128], [128], 1),
    ([1], [1], 1),
    ([129, 5, 260], [70, 333, 1], 3),          # Lq != Lk, ragged tails in both
    ([0, 200, 0, 17], [3, 150, 0, 400], 2),     # empty sequences (no queries) are skipped
]


@pytest.mark.parametrize("scores", ["guarded", "bf16"])
@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_parity_mx(pv_mode, case, scores):
    """Every element against the oracle. scores="bf16" forces the BF16 score path (fp8_score_guard
    < 0): the dequantized-K pipeline with BF16 V, the two-group kernel's BF16 score loop with E4M3 V."""
    lq, lk, h = SMALL[case]
    wl = make_custom(lq, lk, heads=h, seed=40 + case)
    out, lse, q, k = _run_mx(wl, pv_mode, fp8_score_guard=None if scores == "guarded" else -1.0)
    ops = oracle_operands(wl, pv_mode)
    assert np.array_equal(q.payload.cpu().numpy(), ops["pq"]) and np.array_equal(q.scales.cpu().numpy(), ops["sq"])
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode=pv_mode)
    st = compare(out, lse, ref)
    assert_within(st)


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_small_parity_pertensor_descales(pv_mode):
    wl = make_custom([260, 70], [190, 300], heads=3, seed=50)
    rng = np.random.default_rng(51)
    d = {t: np.exp2(rng.uniform(-4, 2, (2, 3))) for t in "qkv"}
    if pv_mode == "bf16":
        d["v"] = None
    ops = oracle_operands(wl, pv_mode, mode="pertensor", descales=d)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = torch.from_numpy(ops["pq"]).to(dev)
    k = torch.from_numpy(ops["pk"]).to(dev)
    v = torch.from_numpy(ops["pv"]).to(dev) if pv_mode == "fp8" else bf16_to_device(wl.v_bits)
    t = lambda a: None if a is None else torch.tensor(a, dtype=torch.float32, device=dev)
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode=pv_mode, q_descale=t(d["q"]),
                                     k_descale=t(d["k"]), v_descale=t(d["v"]))
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode=pv_mode,
                                  q_descale=d["q"], k_descale=d["k"], v_descale=d["v"])
    assert_within(compare(out, lse, ref))


def _pertensor_tiles_on_fp8_path(q_codes, lengths, heads, c_of, k_codes=None, lengths_k=None):
    """The precision guard's decision for every (sequence, head, 128-query tile) in per-tensor mode,
    recomputed on the host: FP8 scores when c * max|q| * max|k| <= 16, with max|q| the largest code
    magnitude of the tile's queries and max|k| the largest code of the 16-token groups that hold the
    sequence's keys (k_codes given: the kernel reads the cast's group maxima), or 448 (c_of(seq,
    head): the float32 softmax_scale * log2(e) * q_descale * k_descale the kernel forms)."""
    vals = np.abs(oracle.e4m3_decode(q_codes))
    gm = None if k_codes is None else oracle.e4m3_decode(e4m3_group_max(k_codes))
    ok, t0, k0 = [], 0, 0
    lengths_k = lengths if lengths_k is None else lengths_k
    for r, L in enumerate(lengths):
        for hh in range(heads):
            kb = np.float32(448.0) if gm is None else np.float32(gm[k0 // 16:(k0 + lengths_k[r] - 1) // 16 + 1, hh].max())
            for q0 in range(0, L, 128):
                qb = vals[t0 + q0:t0 + min(q0 + 128, L), hh].max()
                ok.append(np.float32(np.float32(c_of(r, hh)) * np.float32(qb)) * kb <= 16.0)
        t0 += L
        k0 += lengths_k[r]
    return np.array(ok)


def _pertensor_run(wl, d, rows=None, k_group_max=False):
    ops = oracle_operands(wl, "fp8", mode="pertensor", descales=d)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q, k, v = (torch.from_numpy(ops[n]).to(dev) for n in ("pq", "pk", "pv"))
    t = lambda a: None if a is None else torch.tensor(a, dtype=torch.float32, device=dev)
    gm = torch.from_numpy(e4m3_group_max(ops["pk"])).to(dev) if k_group_max else None
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="fp8", q_descale=t(d["q"]), k_descale=t(d["k"]),
                                     v_descale=t(d["v"]), k_group_max=gm)
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="fp8",
                                  q_descale=d["q"], k_descale=d["k"], v_descale=d["v"], rows=rows)
    return ops, out, lse, ref


def _c_of(d, tau=1.0 / math.sqrt(128)):
    s = np.float32(np.float32(tau) * np.float32(1.0 / math.log(2.0)))
    g = lambda a, r, hh: np.float32(1.0) if a is None else np.float32(a[r, hh])
    return lambda r, hh: np.float32(np.float32(s * g(d["q"], r, hh)) * g(d["k"], r, hh))


def test_small_parity_pertensor_fp8_scores():
    """Per-tensor mode with descales that put every query tile on the FP8-score path (k_descale
    2^-6: K's codes carry the range, so c * max|q| * 448 stays under the guard), element by element
    against the oracle."""
    wl = make_custom([260, 70], [190, 300], heads=3, seed=53)
    rng = np.random.default_rng(54)
    d = {"q": np.exp2(rng.uniform(-1, 1, (2, 3))), "k": np.full((2, 3), 2.0 ** -6), "v": np.exp2(rng.uniform(-2, 2, (2, 3)))}
    ops, out, lse, ref = _pertensor_run(wl, d)
    assert np.all(_pertensor_tiles_on_fp8_path(ops["pq"], wl.lengths_q, 3, _c_of(d)))
    assert_within(compare(out, lse, ref))


def test_pertensor_fp8_scores_full_size(pertensor_wl):
    """The per-tensor workload (2 x 16384, 24 heads) with k_descale 2^-6: every one of its 6144
    query tiles takes FP8 scores; sampled rows (every 61st, all heads and keys) against the oracle."""
    wl = pertensor_wl
    d = {"q": None, "k": np.full((2, 24), 2.0 ** -6), "v": None}
    ops, out, lse, ref = _pertensor_run(wl, d, rows=_rows(wl, 61))
    on_fp8 = _pertensor_tiles_on_fp8_path(ops["pq"], wl.lengths_q, 24, _c_of(d))
    assert on_fp8.size == 6144 and np.all(on_fp8)
    assert_within(compare(out, lse, ref))


def test_floor_scaled_inputs():
    wl = make_custom([300], [260], heads=2, seed=52)
    out, lse, q, k = _run_mx(wl, "bf16", scaling="floor")
    from helpers import f64
    pq, sq, cq = oracle.mx_quantize_varlen(f64(wl.q_bits), wl.cu_q, "floor")
    pk, sk, ck = oracle.mx_quantize_varlen(f64(wl.k_bits), wl.cu_k, "floor")
    ref = oracle.attention_varlen(oracle.mx_dequantize_varlen(pq, sq, wl.cu_q, cq),
                                  oracle.mx_dequantize_varlen(pk, sk, wl.cu_k, ck), f64(wl.v_bits),
                                  wl.cu_q, wl.cu_k, pv_mode="bf16")
    assert_within(compare(out, lse, ref))


# ---------------------------------------------------------------- the five workloads
def test_tiny_full():
    wl = make_workload("tiny", seed=0)
    out, lse, _, _ = _run_mx(wl, "bf16")
    ops = oracle_operands(wl, "bf16")
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="bf16")
    assert_within(compare(out, lse, ref))


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_dense_sampled(pv_mode):
    wl = make_workload("dense", seed=0)
    out, lse, _, _ = _run_mx(wl, pv_mode)
    ops = oracle_operands(wl, pv_mode)
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode=pv_mode,
                                  rows=_rows(wl, 7))
    assert_within(compare(out, lse, ref))


@pytest.mark.parametrize("tile_order", [False, True])
def test_varlen_sampled(tile_order):
    """Packed varlen with x20 outliers. Outlier rows reach |O| ~ 60, where a BF16 ulp is 2^-2:
    O is held to 2e-2 plus one BF16 ulp of the oracle value there, and the count of elements past
    the plain bound is recorded. LSE and the mean error keep the plain bounds."""
    wl = make_workload("varlen", seed=0)
    out, lse, _, _ = _run_mx(wl, "bf16", tile_order=tile_order)
    ops = oracle_operands(wl, "bf16")
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="bf16",
                                  rows=_rows(wl, 13))
    st = compare(out, lse, ref)
    assert_within(st, bf16_allowance=True)
    # the allowance is only ever needed where the output itself is large: at |O| >= 2 one BF16
    # ulp (2^-6 or more) is already most of the absolute bound
    o = out.float().cpu().numpy().astype(np.float64)
    mask = ~np.isnan(ref.lse[0])
    big_err = np.abs(o[mask] - ref.out[mask]) > 2e-2
    assert np.all(np.abs(ref.out[mask][big_err]) >= 2.0)
    # and every element within the bound derived from the probabilities' BF16 rounding
    bound = pv_rounding_bound(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, _rows(wl, 13), "bf16", ref)
    assert_within_bound(out, ref, bound)


@pytest.mark.parametrize("case", ["ragged_outliers", "varlen", "ragged_no_outliers"])
def test_k_deq_same_results(case):
    """K's BF16 values from the quantizer (`with_deq`) spare the BF16-V kernel's guard-failing tiles
    their own conversion of K; they hold the same values the tiles would compute (same conversion
    instruction), so O and LSE are bit-identical with and without them. With them the kernel starts
    every tile on that path and takes the guard's decision there: the outlier data puts every tile
    over the guard's bound; without outliers the tiles pass and hand over to the FP8-score path,
    again with results identical to the run without K's BF16 values."""
    if case == "varlen":
        wl = make_workload("varlen", seed=0)
    elif case == "ragged_outliers":
        wl = make_custom([300, 1, 130, 64], [129, 257, 5, 400], heads=3, seed=61, outlier_rate=0.01)
    else:
        wl = make_custom([300, 1, 130, 64], [129, 257, 5, 400], heads=3, seed=62)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk, with_deq=True)
    v = bf16_to_device(wl.v_bits)
    out1, lse1 = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="bf16")
    k_plain = lp.Mxfp8Tensor(k.payload, k.scales, k.meta, k.group_max)
    out0, lse0 = lp.lp_attn_varlen_fwd(q, k_plain, v, mq, mk, pv_mode="bf16")
    torch.cuda.synchronize()
    assert torch.equal(out1, out0)
    assert torch.equal(lse1.nan_to_num(), lse0.nan_to_num())
    if case != "varlen":  # small enough for the oracle everywhere
        ops = oracle_operands(wl, "bf16")
        ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="bf16")
        assert_within(compare(out1, lse1, ref), bf16_allowance=True)


def test_varlen_fp8_pv_sampled():
    """The outlier varlen workload in the fp8 PV mode (E4M3 V, unscaled E4M3 P). As in the mx
    mode, E4M3 P rounded against the kernel's running maximum and against the oracle's final one
    differ by more than the plain absolute bound on rows spread over thousands of keys with x20
    V outliers: every sampled element is held to the bound derived from the oracle's unrounded
    probabilities (helpers.pv_rounding_bound), LSE to the plain bound."""
    wl = make_workload("varlen", seed=0)
    out, lse, _, _ = _run_mx(wl, "fp8")
    ops = oracle_operands(wl, "fp8")
    rows = _rows(wl, 13)
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="fp8", rows=rows)
    st = compare(out, lse, ref)
    record(st)
    assert st["lse_max"] <= 1e-3, st
    bound = pv_rounding_bound(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, rows, "fp8", ref)
    assert_within_bound(out, ref, bound)


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_cross_sampled(pv_mode):
    wl = make_workload("cross", seed=0)
    out, lse, _, _ = _run_mx(wl, pv_mode)
    ops = oracle_operands(wl, pv_mode)
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode=pv_mode,
                                  rows=_rows(wl, 61))
    st = compare(out, lse, ref)
    assert_within(st)
    # |O| is small here (softmax spread over many keys), so bound the relative error too. E4M3
    # rounding of each probability has a relative std of 2^-4/sqrt(3) = 3.6%, and the kernel and
    # the oracle round against different maxima; BF16 rounding is 2^5 times finer.
    assert st["o_rel"] < (0.06 if pv_mode == "fp8" else 0.004), st


@pytest.fixture(scope="module")
def pertensor_wl():
    return make_workload("pertensor", seed=0)


_PT_CACHE = {}


def _pertensor_ops(wl, case):
    """Oracle-prepared per-tensor payloads (E4M3(x / s)) for one descale case, computed once."""
    if case not in _PT_CACHE:
        _PT_CACHE[case] = oracle_operands(wl, "fp8", mode="pertensor", descales=wl.descales[case])
    return _PT_CACHE[case]


@pytest.mark.parametrize("case", ["none", "calibrated", "perhead"])
@pytest.mark.parametrize("gmax", [False, True])
def test_pertensor_sampled(pertensor_wl, case, gmax):
    """The per-tensor workload's descale cases. With K's group maxima (as the cast writes them) the
    precision guard bounds |k| by the data, and at least 95% of the 6144 query tiles take FP8
    scores (recomputed on the host); without them it must assume 448 and most tiles take BF16
    scores. Sampled rows (every 61st, all heads and keys) against the oracle either way."""
    wl = pertensor_wl
    d = wl.descales[case]
    ops = _pertensor_ops(wl, case)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    q = torch.from_numpy(ops["pq"]).to(dev)
    k = torch.from_numpy(ops["pk"]).to(dev)
    v = torch.from_numpy(ops["pv"]).to(dev)
    gm = torch.from_numpy(e4m3_group_max(ops["pk"])).to(dev) if gmax else None
    t = lambda a: None if a is None else torch.tensor(a, dtype=torch.float32, device=dev)
    out, lse = lp.lp_attn_varlen_fwd(q, k, v, mq, mq, pv_mode="fp8", q_descale=t(d["q"]),
                                     k_descale=t(d["k"]), v_descale=t(d["v"]), k_group_max=gm)
    torch.cuda.synchronize()
    on_fp8 = _pertensor_tiles_on_fp8_path(ops["pq"], wl.lengths_q, 24, _c_of(d), ops["pk"] if gmax else None)
    record({"case": case, "gmax": gmax, "fp8_tiles": int(on_fp8.sum()), "tiles": int(on_fp8.size)})
    if gmax:
        assert on_fp8.mean() >= 0.95, on_fp8.mean()
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode="fp8",
                                  q_descale=d["q"], k_descale=d["k"], v_descale=d["v"], rows=_rows(wl, 61))
    assert_within(compare(out, lse, ref))


@pytest.mark.parametrize("gmax", [False, True])
def test_pertensor_unit_descale_bit_identical(pertensor_wl, gmax):
    """Full size: descale None and a unit descale tensor give the same bits; 2 changes them. With
    K's group maxima the tiles take FP8 scores, without them mostly BF16 scores: both paths."""
    wl = pertensor_wl
    ops = _pertensor_ops(wl, "none")
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    q, k, v = (torch.from_numpy(ops[n]).to(dev) for n in ("pq", "pk", "pv"))
    gm = torch.from_numpy(e4m3_group_max(ops["pk"])).to(dev) if gmax else None
    o0, l0 = lp.lp_attn_varlen_fwd(q, k, v, mq, mq, pv_mode="fp8", k_group_max=gm)
    ones = torch.ones((2, 24), dtype=torch.float32, device=dev)
    o1, l1 = lp.lp_attn_varlen_fwd(q, k, v, mq, mq, pv_mode="fp8", q_descale=ones, k_descale=ones, v_descale=ones,
                                   k_group_max=gm)
    bcast = torch.ones((1, 1), dtype=torch.float32, device=dev)
    o2, l2 = lp.lp_attn_varlen_fwd(q, k, v, mq, mq, pv_mode="fp8", q_descale=bcast, k_descale=bcast,
                                   v_descale=bcast, k_group_max=gm)
    o3, l3 = lp.lp_attn_varlen_fwd(q, k, v, mq, mq, pv_mode="fp8", q_descale=2.0, k_group_max=gm)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    assert torch.equal(o0.view(torch.int16), o2.view(torch.int16)) and torch.equal(l0, l2)
    assert not torch.equal(o0.view(torch.int16), o3.view(torch.int16))
    assert not torch.equal(l0, l3)


# ---------------------------------------------------------------- exact invariants
def test_unit_descale_mx_mode_and_two_changes():
    wl = make_custom([300, 130], [200, 129], heads=2, seed=60)
    o0, l0, _, _ = _run_mx(wl, "fp8")
    dev = torch.device("cuda")
    ones = torch.ones((2, 2), dtype=torch.float32, device=dev)
    o1, l1, _, _ = _run_mx(wl, "fp8", q_descale=ones, k_descale=ones, v_descale=ones)
    o2, l2, _, _ = _run_mx(wl, "fp8", k_descale=2.0)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    assert not torch.equal(o0.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_packed_equals_each_sequence_alone(pv_mode):
    lq, lk = [130, 1, 300, 64], [257, 40, 3, 128]
    wl = make_custom(lq, lk, heads=2, seed=61)
    out, lse, _, _ = _run_mx(wl, pv_mode)
    for r in range(len(lq)):
        a, b = wl.cu_q[r], wl.cu_q[r + 1]
        c, d = wl.cu_k[r], wl.cu_k[r + 1]
        from synth import Workload
        alone = Workload("alone", [lq[r]], [lk[r]], 2, wl.q_bits[a:b], wl.k_bits[c:d], wl.v_bits[c:d])
        o1, l1, _, _ = _run_mx(alone, pv_mode)
        assert torch.equal(o1.view(torch.int16), out[a:b].view(torch.int16))
        assert torch.equal(l1, lse[:, a:b])


def test_v_times_two_doubles_output_bf16():
    wl = make_custom([200], [300], heads=2, seed=62)
    out, lse, _, _ = _run_mx(wl, "bf16")
    v2 = (wl.v_bits.astype(np.uint32) + 0x80).astype(np.uint16)        # exponent + 1: exactly 2x (no zeros/subnormals here)
    assert np.all((wl.v_bits & 0x7F80) != 0)
    from synth import Workload
    wl2 = Workload("x2", wl.lengths_q, wl.lengths_k, 2, wl.q_bits, wl.k_bits, v2)
    out2, lse2, _, _ = _run_mx(wl2, "bf16")
    assert torch.equal(out2.float(), 2 * out.float())
    assert torch.equal(lse, lse2)


def test_power_of_two_swap_between_q_and_k():
    """Q * 2^k with K * 2^-k: identical payloads, scales shifted by +-k, identical O and LSE bits."""
    wl = make_custom([150, 90], [140, 260], heads=2, seed=63)
    from synth import Workload
    up = (wl.q_bits.astype(np.int32) + (3 << 7)).astype(np.uint16)    # x 8 (normal values only)
    dn = (wl.k_bits.astype(np.int32) - (3 << 7)).astype(np.uint16)    # / 8
    assert np.all(((wl.q_bits >> 7) & 0xFF) < 250) and np.all(((wl.k_bits >> 7) & 0xFF) > 5)
    wl2 = Workload("swap", wl.lengths_q, wl.lengths_k, 2, up, dn, wl.v_bits)
    o1, l1, q1, k1 = _run_mx(wl, "fp8")
    o2, l2, q2, k2 = _run_mx(wl2, "fp8")
    assert torch.equal(q1.payload, q2.payload) and torch.equal(k1.payload, k2.payload)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_zero_queries_closed_form():
    """Q = 0: O = mean of V (BF16 V, P = 1 exactly), LSE = ln Sk."""
    wl = make_custom([100], [333], heads=2, seed=64)
    from synth import Workload
    wl0 = Workload("q0", wl.lengths_q, wl.lengths_k, 2, np.zeros_like(wl.q_bits), wl.k_bits, wl.v_bits)
    out, lse, _, _ = _run_mx(wl0, "bf16")
    from helpers import f64
    mean = f64(wl.v_bits).mean(axis=0)
    assert np.abs(out.float().cpu().numpy() - mean[None]).max() < 4e-3
    assert np.abs(lse.cpu().numpy() - math.log(333)).max() < 1e-5


def test_deterministic_and_tile_order_invariant():
    wl = make_workload("varlen", seed=3)
    o1, l1, _, _ = _run_mx(wl, "fp8")
    o2, l2, _, _ = _run_mx(wl, "fp8")
    o3, l3, _, _ = _run_mx(wl, "fp8", tile_order=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)


def test_timing_events_stamped_by_dispatch():
    """Events passed in the args are recorded by the kernel's own dispatch: the output is the same
    as without them, and their interval is positive and no longer than events recorded around
    the launch on the stream."""
    wl = make_custom([1000, 700], [900, 1200], heads=4, seed=71)
    ref_o, ref_l, _, _ = _run_mx(wl, "fp8")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in (e0, e1):
        e.record()
    torch.cuda.synchronize()
    b0.record()
    out, lse, _, _ = _run_mx(wl, "fp8", timing=(e0, e1))
    b1.record()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(lse, ref_l)
    kernel_ms, bracket_ms = e0.elapsed_time(e1), b0.elapsed_time(b1)
    assert 0.0 < kernel_ms <= bracket_ms
    with pytest.raises(ValueError):
        _run_mx(wl, "fp8", timing=(0, 0))


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_plan_and_reused_buffers_match_functional(pv_mode):
    """AttnPlan and the out= quantizer buffers give the functional API's bits, call after call,
    and a plan refuses operands that do not match what it was prepared for."""
    dev = torch.device("cuda")
    wl1 = make_custom([300, 77], [260, 500], heads=3, seed=81)
    wl2 = make_custom([300, 77], [260, 500], heads=3, seed=82)
    mq = lp.VarlenMeta.from_lengths(wl1.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl1.lengths_k, dev)
    plan = lp.AttnPlan(mq, mk, 3, pv_mode=pv_mode)
    qx = lp.quantize_mxfp8_varlen(bf16_to_device(wl2.q_bits), mq)     # buffers reused below
    kx = lp.quantize_mxfp8_varlen(bf16_to_device(wl2.k_bits), mk)
    vx = torch.empty((mk.total_tokens, 3, 128), dtype=torch.uint8, device=dev)
    for wl in (wl1, wl2, wl1):
        ref_o, ref_l, _, _ = _run_mx(wl, pv_mode)
        lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq, out=qx)
        lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk, out=kx)
        v = bf16_to_device(wl.v_bits)
        if pv_mode == "fp8":
            v = lp.cast_e4m3(v, out=vx)
        o, l = plan(qx, kx, v)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(l, ref_l)
    with pytest.raises(ValueError):
        plan(qx.payload, kx.payload, v)                   # raw codes into a block-scaled plan
    with pytest.raises(ValueError):
        plan(kx, qx, v)                                   # shapes swapped (Lq != Lk)
    with pytest.raises(ValueError):
        lp.cast_e4m3(bf16_to_device(wl1.v_bits), out=torch.empty((1, 3, 128), dtype=torch.uint8, device=dev))


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_graph_replay_matches_eager(pv_mode):
    """The whole step (quantize Q and K, cast V, attention) captured once into a HIP graph gives
    the eager bits on every replay. Between replays the static inputs are refilled with another
    workload's data and eager calls overwrite every output buffer, so each replay must recompute
    all of its outputs. The entry points record no memset and allocate nothing when given
    their output buffers."""
    dev = torch.device("cuda")
    wls = [make_custom([300, 77], [260, 500], heads=3, seed=s) for s in (91, 92)]
    mq = lp.VarlenMeta.from_lengths(wls[0].lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wls[0].lengths_k, dev)
    qin, kin, vin = (bf16_to_device(getattr(wls[0], f + "_bits")).clone() for f in "qkv")
    qx = lp.quantize_mxfp8_varlen(qin, mq)
    kx = lp.quantize_mxfp8_varlen(kin, mk)
    vx = lp.cast_e4m3(vin) if pv_mode == "fp8" else vin
    plan = lp.AttnPlan(mq, mk, 3, pv_mode=pv_mode)

    def step(q, k, v):
        lp.quantize_mxfp8_varlen(q, mq, out=qx)
        lp.quantize_mxfp8_varlen(k, mk, out=kx)
        vv = lp.cast_e4m3(v, out=vx) if pv_mode == "fp8" else v
        return plan(qx, kx, vv)

    refs = []
    for wl in wls:
        o, l, q, k = _run_mx(wl, pv_mode)
        refs.append((o.clone(), l.clone(), q.payload.clone(), q.scales.clone(), k.payload.clone(), k.scales.clone()))
    step(qin, kin, vin)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(qin, kin, vin)
    for r in range(4):
        wi = r % 2
        for dst, f in zip((qin, kin, vin), "qkv"):
            dst.copy_(bf16_to_device(getattr(wls[wi], f + "_bits")))
        other = wls[1 - wi]
        step(*(bf16_to_device(getattr(other, f + "_bits")) for f in "qkv"))   # eager: overwrite everything
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, l, pq, sq, pk, sk = refs[wi]
        assert torch.equal(qx.payload, pq) and torch.equal(qx.scales, sq), f"replay {r}: Q quantization"
        assert torch.equal(kx.payload, pk) and torch.equal(kx.scales, sk), f"replay {r}: K quantization"
        assert torch.equal(plan.out.view(torch.int16), o.view(torch.int16)), f"replay {r}: O"
        assert torch.equal(plan.lse, l), f"replay {r}: LSE"


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
@pytest.mark.parametrize("which", ["outliers", "dense"])
def test_k_group_max_same_results(pv_mode, which):
    """The precision guard takes the same decisions from the quantizer's K group maxima as from its
    own scan of the K scales: O and LSE are bit-identical with and without them. The outlier input
    mixes tiles on the FP8 and on the BF16 score path within one launch."""
    if which == "outliers":
        wl = make_custom([300, 640, 129, 900], [450, 640, 77, 1000], heads=3, seed=95, outlier_rate=2e-5)
    else:
        wl = make_workload("dense", seed=0)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    q = lp.quantize_mxfp8_varlen(bf16_to_device(wl.q_bits), mq)
    k = lp.quantize_mxfp8_varlen(bf16_to_device(wl.k_bits), mk)
    assert k.group_max is not None
    v = bf16_to_device(wl.v_bits)
    if pv_mode == "fp8":
        v = lp.cast_e4m3(v)
    o1, l1 = lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode=pv_mode)
    o1, l1 = o1.clone(), l1.clone()
    k_scan = lp.Mxfp8Tensor(k.payload, k.scales, mk)   # no group maxima: the kernel scans
    o2, l2 = lp.lp_attn_varlen_fwd(q, k_scan, v, mq, mk, pv_mode=pv_mode)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    with pytest.raises(ValueError):
        bad = lp.Mxfp8Tensor(k.payload, k.scales, mk, k.group_max[:1])
        lp.lp_attn_varlen_fwd(q, bad, v, mq, mk, pv_mode=pv_mode)


@pytest.mark.parametrize("pv_mode", ["bf16", "fp8"])
def test_fp8_score_guard_threshold_selects_the_path(pv_mode):
    """fp8_score_guard picks the score path: a negative threshold forces BF16 scores, a huge one
    FP8 scores, on the same dense inputs (where the default takes FP8). Both match the oracle;
    the default equals the forced-FP8 run bit for bit and differs from the forced-BF16 one (the
    FP8 instruction truncates inside its groups of 8 products)."""
    wl = make_workload("dense", seed=0)
    outs = {}
    for name, g in (("default", None), ("never", -1.0), ("always", 1e30)):
        o, l, _, _ = _run_mx(wl, pv_mode, fp8_score_guard=g)
        outs[name] = (o.clone(), l.clone())
    ops = oracle_operands(wl, pv_mode)
    ref = oracle.attention_varlen(ops["qhat"], ops["khat"], ops["vprime"], wl.cu_q, wl.cu_k, pv_mode=pv_mode,
                                  rows=_rows(wl, 31))
    for name in outs:
        assert_within(compare(*outs[name], ref))
    assert torch.equal(outs["default"][0].view(torch.int16), outs["always"][0].view(torch.int16))
    assert not torch.equal(outs["default"][1], outs["never"][1])
    with pytest.raises(ValueError):
        _run_mx(wl, pv_mode, fp8_score_guard=0.0)



# ---------------------------------------------------------------- a sequence with queries but no keys
@pytest.mark.parametrize("mode", ["bf16", "fp8", "bf16_fa"])
def test_sequence_without_keys_through_the_abi(mode):
    """The C ABI's contract for a sequence with queries but no keys: its O rows are 0 and its LSE is
    -inf, while the other sequences are unaffected. The Python wrapper rejects such metadata (the
    pages define no result for it), so the plan is built on metadata with one key there and its
    struct is then pointed at the real, keyless key offsets: the call itself goes through
    lp_attn_varlen_fwd as any caller of the library would make it. Covers the one-group kernel
    (bf16 PV, BF16 FlashAttention forward) and the two-group kernel (fp8 PV)."""
    from helpers import f64
    lq, lk, h = [130, 40, 200], [150, 0, 90], 2
    wl = make_custom(lq, lk, heads=h, seed=77)
    dev = torch.device("cuda")
    mq = lp.VarlenMeta.from_lengths(lq, dev)
    mk = lp.VarlenMeta.from_lengths(lk, dev)
    mk_one = lp.VarlenMeta.from_lengths([150, 1, 90], dev)
    qb, kb, vb = bf16_to_device(wl.q_bits), bf16_to_device(wl.k_bits), bf16_to_device(wl.v_bits)
    if mode == "bf16_fa":
        plan = lp.AttnPlan(mq, mk_one, h, pv_mode="bf16", mx=False, qk_bf16=True)
        q, k, v = qb, kb, vb
    else:
        plan = lp.AttnPlan(mq, mk_one, h, pv_mode=mode)
        q, k = lp.quantize_mxfp8_varlen(qb, mq), lp.quantize_mxfp8_varlen(kb, mk)
        v = lp.cast_e4m3(vb) if mode == "fp8" else vb
        plan._args.cu_scale_k = mk.cu_scale.data_ptr()
    a = plan._args
    a.cu_seqlens_k = mk.cu_seqlens.data_ptr()
    a.total_k, a.max_seqlen_k = mk.total_tokens, mk.max_seqlen
    plan.meta_k, plan._kshape = mk, (mk.total_tokens, h, 128)
    plan._keep = plan._keep + (mk,)
    plan.out.fill_(1.0)
    plan.lse.fill_(1.0)
    out, lse = plan(q, k, v)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(o[130:170] == 0.0)
    assert np.all(np.isneginf(l[:, 130:170]))
    # the other two sequences against the oracle, computed on them alone
    pv = "bf16" if mode == "bf16_fa" else mode
    if mode == "bf16_fa":
        qhat, khat, vprime = f64(wl.q_bits), f64(wl.k_bits), f64(wl.v_bits)
    else:
        ops = oracle_operands(wl, pv)
        qhat, khat, vprime = ops["qhat"], ops["khat"], ops["vprime"]
    keep = np.r_[0:130, 170:370]
    ref = oracle.attention_varlen(qhat[keep], khat, vprime, [0, 130, 330], [0, 150, 240], pv_mode=pv)
    st = compare(out[torch.as_tensor(keep, device=out.device)], lse[:, torch.as_tensor(keep, device=lse.device)], ref)
    assert_within(st)
