"""The oracle pins catch planted mistakes (CPU only).

Each case rewrites one line of one oracle function -- a dropped term, a wrong sign, index or
operand, a swapped parameter -- installs the mutant in place of the original for the duration of
the case, and runs every pin of ``tests/test_oracle_pins.py`` in-process.  At least one pin must
fail; a mutation that every pin survives marks a part of the oracle that nothing holds down.
The mistakes are planted in the CPU oracle only.
"""
import importlib
import inspect
import itertools
import textwrap

import pytest

import oracle
from tests import test_oracle_pins as pins

# (module, function or Class.method, text to replace, replacement, what the mistake is)
MUTATIONS = [
    ("oracle.step", "attend", "g = h // group", "g = h % n_kv_heads", "GQA map h % Hkv"),
    ("oracle.step", "attend", "scale = F32(1.0) / np.sqrt(F32(hd))", "scale = F32(1.0) / F32(hd)",
     "softmax scale 1/hd"),
    ("oracle.step", "attend", "out[h] = seq_sum(e[:, None] * v) / den",
     "out[h] = seq_sum(e[:, None] * v)", "codec softmax without its denominator"),
    ("oracle.step", "attend", "p = e / den", "p = e", "talker softmax without its denominator"),
    ("oracle.step", "valid_slots", "(pos - P < window)", "(pos - P <= window)",
     "off-by-one window"),
    ("oracle.step", "valid_slots", "(P <= pos)", "(P <= pos + 1)", "non-causal mask"),
    ("oracle.step", "apply_rope", "a * cos - b * sin", "a * cos + b * sin", "rope sign"),
    ("oracle.step", "rope_cos_sin", "-2.0 * j / float(head_dim)", "-1.0 * j / float(head_dim)",
     "rope frequency"),
    ("oracle.step", "rope_pairs", "return j, j + head_dim // 2", "return 2 * j, 2 * j + 1",
     "rotate_half paired as interleaved"),
    ("oracle.step", "layer_norm", "(d * inv) * np.asarray(w, F32) + np.asarray(b, F32)",
     "(d * inv) * np.asarray(w, F32)", "LayerNorm bias dropped"),
    ("oracle.step", "rms_norm", "ss / F32(v.shape[-1]) + F32(eps)", "ss + F32(eps)",
     "RMS without the mean"),
    ("oracle.step", "gemv", "np.asarray(w, F32).T", "np.asarray(w, F32)", "transposed GEMV"),
    ("oracle.step", "silu_mul", "np.exp(-g)", "np.exp(g)", "SiLU sign"),
    ("oracle.step", "gelu_erf", "v64 / math.sqrt(2.0)", "v64 / 2.0", "GELU erf argument"),
    ("oracle.step", "seq_sum", "[-1]", "[0]", "sum keeps the first term only"),
    ("oracle.step", "OracleDecoder.step", 'lw["ls1"] * a_proj', 'lw["ls2"] * f_proj',
     "LayerScale of the wrong branch"),
    ("oracle.step", "OracleDecoder.step", 'rms_norm(q, lw["q_norm"]', 'rms_norm(q, lw["k_norm"]',
     "qk-norm gain swapped"),
    ("oracle.step", "OracleDecoder.step", "self.P[:, slot] = np.uint32(pos)",
     "self.P[:, slot] = np.uint32(pos + 1)", "wrong position stamp"),
    ("oracle.step", "OracleDecoder.step", "slot = pos % self.R", "slot = (pos + 1) % self.R",
     "wrong ring slot"),
    ("oracle.step", "OracleDecoder.prefill", "self.K[0, l, slots] = k", "self.K[0, l, slots] = q[:, ::2]",
     "prefill pushes the wrong key"),
    ("oracle.conv", "streamed_conv_transpose1d", "full[:, :np.asarray(x).shape[1] * stride]",
     "full[:, -np.asarray(x).shape[1] * stride:]", "streamed columns from the wrong end"),
    ("oracle.conv", "streamed_conv_transpose1d", "full[:, :np.asarray(x).shape[1] * stride]",
     "full[:, w.shape[2] - stride:w.shape[2] - stride + np.asarray(x).shape[1] * stride]",
     "streamed columns shifted by the pending tail"),
    ("oracle.conv", "causal_conv1d", "pad = K - stride", "pad = K - 1", "causal pad width"),
    ("oracle.conv", "elu", "np.exp(v.astype(np.float64)) - 1.0", "np.exp(v.astype(np.float64))",
     "ELU without its -1"),
    ("oracle.rvq", "OracleRVQ.project", "return gemv(self.in_first, x)[0], gemv(self.in_rest, x)[0]",
     "return gemv(self.in_rest, x)[0], gemv(self.in_first, x)[0]", "first/rest input projections swapped"),
    ("oracle.rvq", "OracleRVQ.decode",
     "gemv(self.out_first, acc_f)[0] + gemv(self.out_rest, acc_r)[0]",
     "gemv(self.out_rest, acc_f)[0] + gemv(self.out_first, acc_r)[0]",
     "first/rest output projections swapped"),
    ("oracle.rvq", "OracleRVQ.quantise", "r = (r - self.cb_rest[l, code]).astype(F32)",
     "r = (r + self.cb_rest[l, code]).astype(F32)", "residual update sign"),
    ("oracle.rvq", "sq_distances", "(cb[:, c] - r[c])", "(cb[:, c] - r[0])", "distance index"),
    ("oracle.rvq", "emb_sum", "cbs[l, int(code)]", "cbs[0, int(code)]", "code vector of level 0"),
    ("oracle.pocket", "decode_frames", "rows = np.ascontiguousarray(u.T)",
     "rows = np.ascontiguousarray(u.reshape(-1, u.shape[0]))",
     "channel-major to time-major as a reshape"),
    ("oracle.pocket", "decode_frames", "tr = np.ascontiguousarray(out.T)",
     "tr = np.ascontiguousarray(out.reshape(out.shape[1], -1))",
     "time-major back to channel-major as a reshape"),
    ("oracle.pocket", "decode_frames", 'conv["up.b"], stride, groups=dim)',
     'conv["up.b"], stride, pre_elu=True, groups=dim)', "ELU before the upsample"),
    ("oracle.pocket", "seanet_decode", "pre_elu=(i != 0)", "pre_elu=True",
     "ELU on the first conv's input"),
    ("oracle.pocket", "seanet_decode", "h = (block_in + causal_conv1d(h, W, B, stride, pre_elu=True))",
     "h = (causal_conv1d(h, W, B, stride, pre_elu=True))", "residual block without its skip"),
]


def _install(monkeypatch, modname, qualname, old, new):
    mod = importlib.import_module(modname)
    parts = qualname.split(".")
    owner = mod
    for p in parts[:-1]:
        owner = getattr(owner, p)
    fn = getattr(owner, parts[-1])
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, f"{qualname}: the text to mutate is not in its source"
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {qualname}>", "exec"), mod.__dict__, ns)
    mutant = ns[parts[-1]]
    monkeypatch.setattr(owner, parts[-1], mutant)
    if owner is mod and getattr(oracle, parts[-1], None) is fn:  # the package's re-export
        monkeypatch.setattr(oracle, parts[-1], mutant)


def _pin_calls():
    """Every pin of test_oracle_pins.py as (name, zero-argument callable), parametrisations
    expanded from their marks."""
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != pins.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        axes = []
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) \
                else list(m.args[0])
            vals = [v if len(argnames) > 1 else (v,) for v in m.args[1]]
            axes.append([dict(zip(argnames, v)) for v in vals])
        for combo in itertools.product(*axes):
            kw = {}
            for d in combo:
                kw.update(d)
            out.append((f"{name}{sorted(kw.items())}", lambda fn=fn, kw=kw: fn(**kw)))
    return out


@pytest.mark.parametrize("modname,qualname,old,new,what", MUTATIONS,
                         ids=[m[4] for m in MUTATIONS])
def test_some_pin_catches_the_mutation(monkeypatch, modname, qualname, old, new, what):
    _install(monkeypatch, modname, qualname, old, new)
    caught = []
    for name, call in _pin_calls():
        try:
            call()
        except pytest.skip.Exception:
            continue
        except Exception:  # an assertion, or an error the mistake provokes
            caught.append(name)
            break
    assert caught, f"no pin fails when the oracle has: {what}"
