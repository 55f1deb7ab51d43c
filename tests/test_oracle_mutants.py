"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a copy of an oracle module's source (a dropped term, a
flipped sign, a wrong operand, orientation or index, a missing scale, a changed rounding or
boundary), loads the copy in place of the real module, and runs that module's pin tests (the
other ``test_oracle_*`` files): at least one must fail. The unmodified copy, loaded the same way,
must pass all of them, so a failure is the planted mistake's doing and not the harness's.

The mistakes are string edits of the real source; each edit must match exactly once, so a
rewrite of the oracle that moves the edited line makes this file fail loudly rather than test
nothing.
"""
from __future__ import annotations

import itertools
import pathlib
import sys
import types

import pytest

import oracle
import test_oracle_attention
import test_oracle_backward
import test_oracle_current
import test_oracle_fp8
import test_oracle_mx
import test_oracle_mx_tokens

ORACLE_DIR = pathlib.Path(oracle.__file__).parent

# pin tests that exercise each oracle module (every test function of those files)
PIN_MODULES = {
    "fp8": [test_oracle_fp8, test_oracle_mx, test_oracle_attention],
    "mx": [test_oracle_mx, test_oracle_mx_tokens],
    "attention": [test_oracle_attention],
    "backward": [test_oracle_backward],
    "current": [test_oracle_current],
}

# (module, old text, new text, the mistake)
MUTANTS = [
    # ---- backward: the pins name these in their docstring
    ("backward", "ds = p * (dp - D[:, None])", "ds = p * dp", "dropped D"),
    ("backward", "ds = p * (dp - D[:, None])", "ds = p * (D[:, None] - dp)", "flipped sign of dS"),
    ("backward", "dk[k0:k1, hh] = tau * (dsr.T @ Qt)", "dk[k0:k1, hh] = tau * (dsr.T @ Qd)", "dK from Q's head_dim orientation"),
    ("backward", "dq[q0:q1, hh] = tau * (dsr @ Kt)", "dq[q0:q1, hh] = tau * (dsr @ Kd)", "dQ from K's head_dim orientation"),
    ("backward", "dq[q0:q1, hh] = tau * (dsr @ Kt)", "dq[q0:q1, hh] = dsr @ Kt", "missing tau in dQ"),
    ("backward", "dk[k0:k1, hh] = tau * (dsr.T @ Qt)", "dk[k0:k1, hh] = dsr.T @ Qt", "missing tau in dK"),
    ("backward", "dv[k0:k1, hh] = pr.T @ dO", "dv[k0:k1, hh] = dsr.T @ dO", "dS in place of P in dV"),
    ("backward", "pr, dsr = _round_ops(p, round_ops), _round_ops(ds, round_ops)", "pr, dsr = p, ds", "no BF16 rounding"),
    ("backward", "D = np.sum(dO * O, axis=1)", "D = np.sum(dO * O, axis=1) * (1 + 2.0 ** -10)", "perturbed D"),
    ("backward", "p = np.exp(s - lse[hh, q0:q1][:, None])", "p = np.exp(s + lse[hh, q0:q1][:, None])", "wrong LSE sign"),
    ("backward", "s = tau * (Qd @ Kd.T)", "s = Qd @ Kd.T", "missing tau in the scores"),
    ("backward", "dp = dO @ Vd.T", "dp = O @ Vd.T", "O in place of dO in dP"),
    # ---- forward attention
    ("attention", "s = c * (Q @ K.T)", "s = softmax_scale * (Q @ K.T)", "descales dropped from the scores"),
    ("attention", "s = c * (Q @ K.T)", "s = (Q @ K.T)", "no softmax scale"),
    ("attention", "p = _round_pv(u, pv_mode)", "p = u", "probabilities not rounded"),
    ("attention", "out[q0 + sel, hh] = vd * (p @ V) / l[:, None]", "out[q0 + sel, hh] = vd * (p @ V) / p.sum(axis=1)[:, None]",
     "normalised by the rounded sum"),
    ("attention", "out[q0 + sel, hh] = vd * (p @ V) / l[:, None]", "out[q0 + sel, hh] = (p @ V) / l[:, None]", "v descale dropped"),
    ("attention", "lse[hh, q0 + sel] = m + np.log(l)", "lse[hh, q0 + sel] = np.log(l)", "row maximum missing from LSE"),
    ("attention", "lse[hh, q0 + sel] = m + np.log(l)", "lse[hh, q0 + sel] = m + np.log2(l)", "LSE in base 2"),
    ("attention", "m = s.max(axis=1)", "m = s.max(axis=1) + 1.0", "probabilities rounded against a shifted maximum"),
    ("attention", "return e4m3_decode(e4m3_encode(u))", "return bf16_round(u)", "fp8 mode rounds P to BF16"),
    ("attention", "V = vprime[k0:k1, hh]", "V = vprime[k0:k1, (hh + 1) % h]", "another head's V"),
    ("attention", "K = khat[k0:k1, hh]", "K = khat[q0:q0 + (k1 - k0), hh]", "keys indexed with the query offsets"),
    # ---- MX quantizer
    ("mx", "can_lower = a <= np.ldexp(E4M3_MAX, est - 1)", "can_lower = a <= np.ldexp(E4M3_MAX, est)",
     "RCEIL exponent one too small (the block maximum saturates)"),
    ("mx", "est = np.ceil(np.log2(a) - np.log2(E4M3_MAX)).astype(np.int64)\n        for _ in range(3):",
     "est = np.ceil(np.log2(a) - np.log2(E4M3_MAX)).astype(np.int64) + 1\n        for _ in range(0):",
     "RCEIL exponent one too large, no settling"),
    ("mx", "e[nz] = (ex - 1) - 8", "e[nz] = ex - 8", "FLOOR exponent off by one"),
    ("mx", "return np.clip(e, -127, 127)", "return np.clip(e, -126, 127)", "exponent clamp at -126"),
    ("mx", "scaled = blocks * np.ldexp(1.0, -e)[..., None]", "scaled = blocks * np.ldexp(1.0, e)[..., None]", "payload scaled the wrong way"),
    ("mx", "PAD_SCALE_BYTE = 0x7F", "PAD_SCALE_BYTE = 0x00", "pad rows zero"),
    ("mx", "out[1:] = np.cumsum([padded_len(v) for v in lengths])", "out[1:] = np.cumsum(lengths)", "scale rows not padded"),
    ("mx", "return -(-int(length) // PAD) * PAD", "return (int(length) // PAD) * PAD", "padding rounds down"),
    ("mx", "amax = np.abs(blocks).max(axis=3)", "amax = blocks.max(axis=3)", "block maximum without the absolute value"),
    ("mx", "c0 + min(BLOCK * (b + 1), int(length))", "c0 + BLOCK * (b + 1)", "token blocks run past the sequence"),
    ("mx", "out[c0 + j] = vals[c0 + j] * e8m0_decode(scales[row0 + j // BLOCK])",
     "out[c0 + j] = vals[c0 + j] * e8m0_decode(scales[row0 + j % BLOCK])", "token dequantization picks the wrong block"),
    # ---- number formats
    ("fp8", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))", "pick_hi = (d_hi <= d_lo)", "E4M3 ties round up"),
    ("fp8", "vals[c] = s * m * 2.0 ** -9", "vals[c] = s * m * 2.0 ** -10", "E4M3 subnormal step"),
    ("fp8", "vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 8)", "E4M3 exponent bias"),
    ("fp8", "code = np.where(a >= E4M3_MAX, 0x7E, code)", "code = np.where(a > 464.0, 0x7F, code)", "NaN above 464 instead of saturation"),
    ("fp8", "code = np.where(np.signbit(x), code | 0x80, code)", "code = np.where(x < 0, code | 0x80, code)", "negative zero loses its sign"),
    ("fp8", "return np.ldexp(1.0, b - 127)", "return np.ldexp(1.0, b - 128)", "E8M0 bias"),
    ("fp8", "quantum = np.ldexp(1.0, np.maximum(e - 8, -133))", "quantum = np.ldexp(1.0, np.maximum(e - 9, -133))", "BF16 with 9 bits"),
    ("fp8", "return np.rint(x / quantum) * quantum", "return np.floor(x / quantum + 0.5) * quantum", "BF16 ties away from zero"),
    # ---- current scaling
    ("current", "return np.float32(amax / np.float32(E4M3_MAX))", "return np.float32(amax / np.float32(E4M3_MAX)) * np.float32(1.001)",
     "scale with a margin"),
    ("current", "return np.float32(1.0)", "return np.float32(0.5)", "all-zero tensor scale"),
    ("current", "q = (np.asarray(x, dtype=np.float32) / s).astype(np.float32)",
     "q = (np.asarray(x, dtype=np.float32) * (np.float32(1) / s)).astype(np.float32)", "multiplication by a rounded reciprocal"),
]


def _load_copy(name: str, old: str = None, new: str = None) -> types.ModuleType:
    path = ORACLE_DIR / f"{name}.py"
    src = path.read_text()
    if old is not None:
        assert src.count(old) == 1, f"oracle/{name}.py: edit target must occur exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle._copy_{name}")
    mod.__package__ = "oracle"
    mod.__file__ = str(path)
    exec(compile(src, str(path), "exec"), mod.__dict__)
    return mod


def _install(copy: types.ModuleType, name: str, monkeypatch) -> None:
    """Replace every reference to the real module's objects (in the oracle package, its modules
    and the pin test modules) by the copy's objects of the same name."""
    real = sys.modules[f"oracle.{name}"]
    swaps = {id(getattr(real, a)): getattr(copy, a) for a in dir(real)
             if not a.startswith("__") and hasattr(copy, a) and callable(getattr(real, a))}
    for mname, mod in list(sys.modules.items()):
        if mod is None or not (mname == "oracle" or mname.startswith("oracle.") or mname.startswith("test_oracle")):
            continue
        if mname.startswith("oracle._copy"):
            continue
        for attr, val in list(vars(mod).items()):
            if id(val) in swaps:
                monkeypatch.setattr(mod, attr, swaps[id(val)])


def _calls(mod):
    """Every test function of a pin module, expanded over its parametrize marks."""
    out = []
    for fname in sorted(vars(mod)):
        fn = getattr(mod, fname)
        if not fname.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = [s.strip() for s in (m.args[0].split(",") if isinstance(m.args[0], str) else m.args[0])]
            vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        for combo in itertools.product(*grids) if grids else [()]:
            kw = {}
            for d in combo:
                kw.update(d)
            out.append((f"{mod.__name__}.{fname}{kw if kw else ''}", fn, kw))
    return out


def _failing(name: str, stop_at_first: bool):
    failed = []
    for mod in PIN_MODULES[name]:
        for label, fn, kw in _calls(mod):
            try:
                fn(**kw)
            except Exception:
                failed.append(label)
                if stop_at_first:
                    return failed
    return failed


@pytest.mark.parametrize("name", sorted(PIN_MODULES))
def test_unmodified_copy_passes_every_pin(name, monkeypatch):
    _install(_load_copy(name), name, monkeypatch)
    assert _failing(name, stop_at_first=False) == []


@pytest.mark.parametrize("case", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(case, monkeypatch):
    name, old, new, what = case
    _install(_load_copy(name, old, new), name, monkeypatch)
    assert _failing(name, stop_at_first=True), f"no pin catches the planted mistake: {what} (oracle/{name}.py)"
