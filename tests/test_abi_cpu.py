"""CPU tests of the boundary: the library loads, exports what include/lpfa.h declares, the ctypes
mirror of lpfa_attn_args matches the C layout, and every host-side check returns its error code
before any device work (no GPU is touched: these calls fail validation first)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest
import torch

import precision_attention_mxfp8_amd as lp
from precision_attention_mxfp8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lpfa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liblpfa.so not built")
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(\w+)\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.lpfa_abi_version() == 9


@pytest.mark.parametrize("cname,pystruct", [("lpfa_attn_args", _lib.AttnArgs), ("lpfa_bwd_args", _lib.BwdArgs)])
def test_struct_layout_matches_c(cname, pystruct):
    fields = [f[0] for f in pystruct._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "lpfa.h"', "int main(void){",
           f'printf("size %zu\\n", sizeof({cname}));']
    src += [f'printf("{f} %zu\\n", offsetof({cname}, {f}));' for f in fields]
    src += ["return 0;}"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.split() for line in out if line.strip())
    assert int(got["size"]) == ctypes.sizeof(pystruct)
    for f in fields:
        assert int(got[f]) == getattr(pystruct, f).offset, f


@pytest.mark.parametrize("tq,tk,h", [(0, 0, 1), (2048, 2048, 16), (4096, 32768, 16), (5, 7, 3)])
def test_backward_workspace_macro_matches_python(tq, tk, h):
    src = ['#include <stdio.h>', '#include "lpfa.h"', "int main(void){",
           f'printf("%lld\\n", (long long)LPFA_BWD_WORK_BYTES({tq}, {tk}, {h}));', "return 0;}"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "w.c")
        exe = os.path.join(d, "w")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = int(subprocess.run([exe], capture_output=True, text=True, check=True).stdout)
    assert got == _lib.bwd_work_bytes(tq, tk, h)
    assert got % 256 == 0


FAKE = 0x10000  # an aligned non-NULL address: validation checks it, nothing dereferences it


def _quant(lib, **kw):
    args = dict(x=FAKE, x_dtype=0, stride_tok=256, stride_head=128, total_tokens=2, num_heads=2, head_dim=128,
                cu_seqlens=FAKE, cu_scale=FAKE, num_seqs=1, total_scale_rows=128, scaling_mode=0,
                payload=FAKE, scales=FAKE, deq=None)
    args.update(kw)
    return lib.mxfp8_quantize_varlen(args["x"], args["x_dtype"], args["stride_tok"], args["stride_head"],
                                     args["total_tokens"], args["num_heads"], args["head_dim"],
                                     args["cu_seqlens"], args["cu_scale"], args["num_seqs"],
                                     args["total_scale_rows"], args["scaling_mode"], args["payload"],
                                     args["scales"], None, args["deq"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), _lib.LPFA_ENOTSUP),
    (dict(scaling_mode=7), _lib.LPFA_EINVAL),
    (dict(x_dtype=5), _lib.LPFA_EINVAL),
    (dict(x=None), _lib.LPFA_EINVAL),
    (dict(x=FAKE + 2), _lib.LPFA_EINVAL),          # not 16-byte aligned
    (dict(stride_tok=100), _lib.LPFA_EINVAL),      # 200 bytes: not a 16-byte multiple
    (dict(stride_head=64), _lib.LPFA_EINVAL),      # heads overlap
    (dict(total_scale_rows=100), _lib.LPFA_EINVAL),  # not a multiple of 128
    (dict(total_scale_rows=0), _lib.LPFA_EINVAL),  # fewer scale rows than tokens
    (dict(num_heads=0), _lib.LPFA_EINVAL),
    (dict(cu_scale=None), _lib.LPFA_EINVAL),
    (dict(payload=None), _lib.LPFA_EINVAL),
    (dict(scales=FAKE + 1), _lib.LPFA_EINVAL),
    (dict(deq=FAKE + 8), _lib.LPFA_EINVAL),        # BF16 output not 16-byte aligned
])
def test_quantize_rejects(lib, kw, code):
    assert _quant(lib, **kw) == code
    assert lib.lpfa_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), _lib.LPFA_ENOTSUP),
    (dict(scaling_mode=7), _lib.LPFA_EINVAL),
    (dict(x=FAKE + 2), _lib.LPFA_EINVAL),
    (dict(total_scale_rows=100), _lib.LPFA_EINVAL),
    (dict(scales=None), _lib.LPFA_EINVAL),
])
def test_quantize_tokens_rejects(lib, kw, code):
    args = dict(x=FAKE, x_dtype=0, stride_tok=256, stride_head=128, total_tokens=2, num_heads=2, head_dim=128,
                cu_seqlens=FAKE, cu_scale=FAKE, num_seqs=1, total_scale_rows=128, scaling_mode=0,
                payload=FAKE, scales=FAKE)
    args.update(kw)
    rc = lib.mxfp8_quantize_varlen_tokens(*[args[k] for k in ("x", "x_dtype", "stride_tok", "stride_head",
                                                              "total_tokens", "num_heads", "head_dim", "cu_seqlens",
                                                              "cu_scale", "num_seqs", "total_scale_rows",
                                                              "scaling_mode", "payload", "scales")], None)
    assert rc == code
    assert lib.lpfa_last_error().decode()


def test_cast_current_rejects(lib):
    f = lib.lp_fp8_cast_current
    assert f(FAKE, 0, 256, 128, 2, 2, 96, FAKE, FAKE, FAKE, None) == _lib.LPFA_ENOTSUP
    assert f(FAKE, 0, 256, 128, 2, 2, 128, None, FAKE, FAKE, None) == _lib.LPFA_EINVAL    # work
    assert f(FAKE, 0, 256, 128, 2, 2, 128, FAKE, FAKE, None, None) == _lib.LPFA_EINVAL    # descale
    assert f(FAKE, 0, 256, 128, 2, 2, 128, FAKE + 2, FAKE, FAKE, None) == _lib.LPFA_EINVAL
    assert f(FAKE, 3, 256, 128, 2, 2, 128, FAKE, FAKE, FAKE, None) == _lib.LPFA_EINVAL     # dtype
    assert f(FAKE, 0, 256, 128, 2, 2, 128, FAKE, None, FAKE, None) == _lib.LPFA_EINVAL     # y
    assert lib.lpfa_last_error().decode()


def test_prepare_rejects(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=0, st=256, sh=128, tq=2, tk=2, h=2, d=128, cuq=FAKE, csq=FAKE,
                 cuk=FAKE, csk=FAKE, n=1, rq=128, rk=128, mode=0, qp=FAKE, qs=FAKE, kp=FAKE, ks=FAKE, kg=None,
                 vc=FAKE)
        a.update(kw)
        return lib.mxfp8_prepare_qkv(*a.values(), None)
    assert call(d=64) == _lib.LPFA_ENOTSUP
    assert call(mode=2) == _lib.LPFA_EINVAL
    assert call(dt=5) == _lib.LPFA_EINVAL
    assert call(qs=None) == _lib.LPFA_EINVAL
    assert call(ks=None) == _lib.LPFA_EINVAL
    assert call(csk=None) == _lib.LPFA_EINVAL
    assert call(vc=None) == _lib.LPFA_EINVAL
    assert call(v=FAKE + 8) == _lib.LPFA_EINVAL
    assert call(st=100) == _lib.LPFA_EINVAL
    assert lib.lpfa_last_error().decode()


def test_cast_rejects(lib):
    assert lib.lp_fp8_cast_e4m3(FAKE, 0, 256, 128, 2, 2, 96, FAKE, None, None) == _lib.LPFA_ENOTSUP
    assert lib.lp_fp8_cast_e4m3(FAKE, 2, 256, 128, 2, 2, 128, FAKE, None, None) == _lib.LPFA_EINVAL
    assert lib.lp_fp8_cast_e4m3(FAKE, 0, 256, 128, 2, 2, 128, None, None, None) == _lib.LPFA_EINVAL
    assert lib.lp_fp8_cast_e4m3(FAKE + 8, 0, 256, 128, 2, 2, 128, FAKE, None, None) == _lib.LPFA_EINVAL


def _args(**kw):
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.q = a.k = a.v = FAKE
    a.q_stride_tok = a.k_stride_tok = 256
    a.q_stride_head = a.k_stride_head = 128
    a.v_stride_tok, a.v_stride_head = 256, 128
    a.q_scale = a.k_scale = a.cu_scale_q = a.cu_scale_k = FAKE
    a.cu_seqlens_q = a.cu_seqlens_k = FAKE
    a.num_seqs, a.max_seqlen_q, a.max_seqlen_k = 1, 2, 2
    a.total_q = a.total_k = 2
    a.num_heads, a.head_dim = 2, 128
    a.softmax_scale = 0.088
    a.out = a.lse = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), _lib.LPFA_ENOTSUP),
    (dict(causal=1), _lib.LPFA_ENOTSUP),
    (dict(pv_mode=3), _lib.LPFA_EINVAL),
    (dict(pv_mode=2), _lib.LPFA_EINVAL),            # MX V without its scales
    (dict(pv_mode=1, v_scale=FAKE), _lib.LPFA_EINVAL),   # V scales outside the MX V mode
    (dict(pv_mode=2, v_scale=FAKE, q_scale=None, k_scale=None, cu_scale_q=None, cu_scale_k=None),
     _lib.LPFA_EINVAL),                             # MX V needs MX Q and K
    (dict(pv_mode=2, v_scale=FAKE + 2), _lib.LPFA_EINVAL),  # misaligned V scales
    (dict(qk_bf16=1), _lib.LPFA_EINVAL),            # BF16 Q/K with block scales
    (dict(qk_bf16=1, q_scale=None, k_scale=None, pv_mode=1), _lib.LPFA_EINVAL),   # BF16 Q/K need BF16 V
    (dict(qk_bf16=1, q_scale=None, k_scale=None, q_stride_tok=100), _lib.LPFA_EINVAL),  # 200 bytes
    (dict(qk_bf16=2, q_scale=None, k_scale=None), _lib.LPFA_EINVAL),
    (dict(struct_size=8), _lib.LPFA_EINVAL),
    (dict(k_scale=None), _lib.LPFA_EINVAL),         # Q scales without K scales
    (dict(q_scale=None), _lib.LPFA_EINVAL),
    (dict(cu_scale_k=None), _lib.LPFA_EINVAL),
    (dict(v_descale=FAKE), _lib.LPFA_EINVAL),       # v descale with BF16 V
    (dict(softmax_scale=0.0), _lib.LPFA_EINVAL),
    (dict(softmax_scale=float("nan")), _lib.LPFA_EINVAL),
    (dict(fp8_score_guard=float("nan")), _lib.LPFA_EINVAL),
    (dict(k_deq=FAKE + 8), _lib.LPFA_EINVAL),       # K's BF16 values not 16-byte aligned
    (dict(k_deq=FAKE, pv_mode=1), _lib.LPFA_EINVAL),  # only for BF16 V
    (dict(k_deq=FAKE, q_scale=None, k_scale=None, cu_scale_q=None, cu_scale_k=None), _lib.LPFA_EINVAL),  # MX only
    (dict(softmax_scale=float("inf")), _lib.LPFA_EINVAL),
    (dict(softmax_scale=-0.0), _lib.LPFA_EINVAL),
    (dict(q=None), _lib.LPFA_EINVAL),
    (dict(v=FAKE + 4), _lib.LPFA_EINVAL),
    (dict(k_stride_tok=100), _lib.LPFA_EINVAL),
    (dict(cu_seqlens_k=None), _lib.LPFA_EINVAL),
    (dict(out=None), _lib.LPFA_EINVAL),
    (dict(max_seqlen_q=3), _lib.LPFA_EINVAL),       # longer than the packed tensor
    (dict(num_tiles=4), _lib.LPFA_EINVAL),          # count without an order
    (dict(num_heads=0), _lib.LPFA_EINVAL),
])
def test_attention_rejects(lib, kw, code):
    a = _args(**kw)
    assert lib.lp_attn_varlen_fwd(ctypes.byref(a), None) == code
    assert lib.lpfa_last_error().decode()


def test_attention_rejects_null_args(lib):
    assert lib.lp_attn_varlen_fwd(None, None) == _lib.LPFA_EINVAL
    assert lib.lp_attn_varlen_bwd(None, None) == _lib.LPFA_EINVAL


def _bwd_args(**kw):
    a = _lib.BwdArgs()
    a.struct_size = ctypes.sizeof(_lib.BwdArgs)
    for f in ("q", "q_scale", "k", "k_scale", "v", "v_scale", "q_t", "q_t_scale", "k_t", "k_t_scale", "out",
              "dout", "lse", "cu_seqlens_q", "cu_seqlens_k", "cu_scale_q", "cu_scale_k", "work", "dq", "dk", "dv"):
        setattr(a, f, FAKE)
    a.num_seqs, a.num_heads, a.head_dim = 1, 2, 128
    a.total_q = a.total_k = 100
    a.total_scale_rows_q = a.total_scale_rows_k = 128
    a.softmax_scale = 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), _lib.LPFA_ENOTSUP),
    (dict(causal=1), _lib.LPFA_ENOTSUP),
    (dict(struct_size=8), _lib.LPFA_EINVAL),
    (dict(num_heads=0), _lib.LPFA_EINVAL),
    (dict(total_scale_rows_k=100), _lib.LPFA_EINVAL),     # not a multiple of 128
    (dict(total_q=200), _lib.LPFA_EINVAL),                # more tokens than scale rows
    (dict(softmax_scale=-1.0), _lib.LPFA_EINVAL),
    (dict(output_mxfp8_dkv=2), _lib.LPFA_EINVAL),
    (dict(scaling_mode=2), _lib.LPFA_EINVAL),
    (dict(output_mxfp8_dkv=1), _lib.LPFA_EINVAL),          # MXFP8 dK/dV without scale outputs
    (dict(output_mxfp8_dkv=1, dk_scale=FAKE), _lib.LPFA_EINVAL),
    (dict(dk_scale=FAKE, dv_scale=FAKE), _lib.LPFA_EINVAL),  # scale outputs for BF16 dK/dV
    (dict(q_t=None), _lib.LPFA_EINVAL),
    (dict(k_t_scale=FAKE + 4), _lib.LPFA_EINVAL),         # token scales are read 16 bytes at a time
    (dict(dq=FAKE + 2), _lib.LPFA_EINVAL),
    (dict(lse=FAKE + 2), _lib.LPFA_EINVAL),
    (dict(work=None), _lib.LPFA_EINVAL),
    (dict(work=FAKE + 16), _lib.LPFA_EINVAL),             # the workspace is 256-byte aligned
    (dict(cu_scale_k=None), _lib.LPFA_EINVAL),
    (dict(num_seqs=0), _lib.LPFA_EINVAL),                 # tokens without sequences
])
def test_backward_rejects(lib, kw, code):
    a = _bwd_args(**kw)
    assert lib.lp_attn_varlen_bwd(ctypes.byref(a), None) == code
    assert lib.lpfa_last_error().decode()


def test_varlen_meta_host_side():
    m = lp.VarlenMeta.from_lengths([5, 0, 128, 129], device="cpu")
    assert m.cu_seqlens_host == (0, 5, 5, 133, 262)
    assert m.cu_scale_host == (0, 128, 128, 256, 512)
    assert m.total_scale_rows == 512 and m.max_seqlen == 129 and m.num_seqs == 4
    assert m.cu_seqlens.dtype == torch.int32 and m.cu_seqlens.tolist() == list(m.cu_seqlens_host)
    d = lp.VarlenMeta.dense(3, 100, device="cpu")
    assert d.lengths == (100, 100, 100) and d.cu_seqlens_host == (0, 100, 200, 300)
    with pytest.raises(ValueError):
        lp.VarlenMeta.from_lengths([3, -1], device="cpu")


def test_longest_first_order():
    mq = lp.VarlenMeta.from_lengths([300, 100], device="cpu")
    mk = lp.VarlenMeta.from_lengths([50, 900], device="cpu")
    order = lp.longest_first_tile_order(mq, mk, heads=2).view(-1, 3).tolist()
    assert len(order) == (3 + 1) * 2
    assert order[0][0] == 1 and order[1][0] == 1                  # the sequence with 900 keys first
    assert sorted(map(tuple, order)) == sorted((r, h, t) for r, n in ((0, 3), (1, 1)) for t in range(n)
                                               for h in range(2))


def test_api_fails_loudly_on_host_tensors():
    m = lp.VarlenMeta.from_lengths([4], device="cpu")
    with pytest.raises(ValueError):
        lp.quantize_mxfp8_varlen(torch.zeros((4, 1, 128), dtype=torch.bfloat16), m)
    with pytest.raises(ValueError):
        lp.quantize_mxfp8_varlen(torch.zeros((4, 1, 64), dtype=torch.bfloat16), m)
    with pytest.raises(ValueError):
        lp.quantize_mxfp8_varlen(torch.zeros((4, 1, 128)), m, scaling_mode="nearest")
    with pytest.raises(ValueError):
        lp.lp_attn_varlen_fwd(torch.zeros((4, 1, 128), dtype=torch.uint8), torch.zeros((4, 1, 128), dtype=torch.uint8),
                              torch.zeros((4, 1, 128), dtype=torch.bfloat16), m, m, pv_mode="fp16")
