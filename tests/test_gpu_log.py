"""LPFA_LOG=1: the first forward call of each variant in a process prints one line naming the Q/K and
V types fed to the kernel (FastVideo fp8-PV PR: a once-per-process log of the V dtype the attention
received); repeated calls print nothing more, and without the variable nothing is printed."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys, numpy as np, torch
sys.path.insert(0, %r)
import precision_attention_mxfp8_amd as lp
from synth import make_custom
wl = make_custom([130], [200], heads=2, seed=5)
dev = torch.device("cuda")
up = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(dev)
mq, mk = lp.VarlenMeta.from_lengths(wl.lengths_q, dev), lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
q, k = lp.quantize_mxfp8_varlen(up(wl.q_bits), mq), lp.quantize_mxfp8_varlen(up(wl.k_bits), mk)
v = up(wl.v_bits)
for _ in range(3):
    lp.lp_attn_varlen_fwd(q, k, v, mq, mk, pv_mode="bf16")
for _ in range(2):
    lp.lp_attn_varlen_fwd(q, k, lp.cast_e4m3(v), mq, mk, pv_mode="fp8")
torch.cuda.synchronize()
print("done")
""" % ROOT


def _run(env_value):
    env = dict(os.environ)
    env.pop("LPFA_LOG", None)
    if env_value is not None:
        env["LPFA_LOG"] = env_value
    r = subprocess.run([sys.executable, "-c", SCRIPT], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr
    return [l for l in r.stderr.splitlines() if l.startswith("lpfa:")]


def test_variant_log_once_per_variant():
    lines = _run("1")
    assert len(lines) == 2, lines
    assert "V BF16" in lines[0] and "MXFP8" in lines[0]
    assert "V E4M3 unscaled, dequant scale 1.0" in lines[1]


def test_no_log_without_the_variable():
    assert _run(None) == []
