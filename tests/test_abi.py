"""Host-only checks of the C ABI: exports, struct layout and argument validation (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from streaming_ar_transformer_amd import sdec, workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdec.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sdec.LIB_PATH),
                                reason="libsdec.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdec_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == sorted(sdec.EXPORTS)
    lib = sdec.lib()
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", sdec.LIB_PATH], capture_output=True,
                        text=True).stdout
    exported = set(re.findall(r" T (sdec_\w+)", nm))
    assert set(names) <= exported


def test_struct_layout_matches_header(tmp_path):
    fields = {
        "sdec_config": [f for f, _ in sdec.Config._fields_],
        "sdec_layer_weights": [f for f, _ in sdec.LayerWeights._fields_],
        "sdec_final_weights": [f for f, _ in sdec.FinalWeights._fields_],
        "sdec_rvq_config": [f for f, _ in sdec.RVQConfig._fields_],
        "sdec_rvq_weights": [f for f, _ in sdec.RVQWeights._fields_],
        "sdec_conv_config": [f for f, _ in sdec.ConvConfig._fields_],
    }
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "sdec.h"', "int main(void){"]
    for st, fs in fields.items():
        lines.append(f'printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True,
                                                 text=True).stdout.splitlines())
    for st, cls in (("sdec_config", sdec.Config), ("sdec_layer_weights", sdec.LayerWeights),
                    ("sdec_final_weights", sdec.FinalWeights), ("sdec_rvq_config", sdec.RVQConfig),
                    ("sdec_rvq_weights", sdec.RVQWeights), ("sdec_conv_config", sdec.ConvConfig)):
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f, _ in cls._fields_:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, f"{st}.{f}"


def _fake_layer(cfg, base=0x10000):
    lw = sdec.LayerWeights()
    for i, (name, _) in enumerate(sdec.LayerWeights._fields_):
        setattr(lw, name, base + 256 * i)  # aligned, never dereferenced
    return lw


def _create(c, layers, ring, final=None):
    h = ctypes.c_void_p()
    fw = final if final is not None else sdec.FinalWeights(0x20000, 0x20100)
    rc = sdec.lib().sdec_create(ctypes.byref(c), layers, ctypes.byref(fw), ring, ctypes.byref(h))
    return rc, sdec.lib().sdec_last_error().decode()


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 96, "head_dim"),
    ("n_kv_heads", 3, "multiple of n_kv_heads"),
    ("m", 9, "m must be"),
    ("m", 0, "m must be"),
    ("d_model", 510, "d_model"),
    ("window", 300, "window"),
    ("window", 0, "window"),
    ("norm", 7, "norm"),
    ("n_layers", 0, "n_layers"),
    ("max_prefill", 17, "max_prefill"),
])
def test_create_rejects_bad_config(field, value, msg):
    cfg = wl.CONFIGS[1]
    c = sdec.make_config(cfg)
    setattr(c, field, value)
    arr = (sdec.LayerWeights * max(cfg.n_layers, 1))(_fake_layer(cfg))
    rc, err = _create(c, arr, cfg.ring)
    assert rc == sdec.E_ARG and msg in err


def test_create_rejects_unbounded_window_and_bad_weights():
    cfg = wl.CONFIGS[4].replace(n_layers=1)
    c = sdec.make_config(cfg, window=100)  # talker: unbounded
    arr = (sdec.LayerWeights * 1)(_fake_layer(cfg))
    rc, err = _create(c, arr, 2048)
    assert rc == sdec.E_ARG and "unbounded" in err
    c = sdec.make_config(cfg)
    lw = _fake_layer(cfg)
    lw.w_gate = None
    rc, err = _create(c, (sdec.LayerWeights * 1)(lw), 2048)
    assert rc == sdec.E_ARG and "w_gate" in err
    lw = _fake_layer(cfg)
    lw.wk = 0x10004
    rc, err = _create(c, (sdec.LayerWeights * 1)(lw), 2048)
    assert rc == sdec.E_ARG and "aligned" in err
    rc, err = _create(c, (sdec.LayerWeights * 1)(_fake_layer(cfg)), 2048,
                      final=sdec.FinalWeights(0, 0))
    assert rc == sdec.E_ARG and "final" in err


def test_prefill_block_width_fits_the_staging_tile():
    # 16 rows of the 2048-wide talker would need 128 KiB of row staging; the codec's 512 fit
    cfg = wl.CONFIGS[4].replace(n_layers=1)
    c = sdec.make_config(cfg, max_prefill=16)
    rc, err = _create(c, (sdec.LayerWeights * 1)(_fake_layer(cfg)), 2048)
    assert rc == sdec.E_ARG and "staging" in err


def test_prefill_needs_one_stream():
    cfg = wl.CONFIGS[1].replace(m=2)
    c = sdec.make_config(cfg, max_prefill=4)
    arr = (sdec.LayerWeights * cfg.n_layers)(_fake_layer(cfg))
    rc, err = _create(c, arr, cfg.ring)
    assert rc == sdec.E_ARG and "one stream" in err
    assert sdec.lib().sdec_prefill(None, 16, 0, 1, 1, None) == sdec.E_ARG


def test_rvq_rejects_bad_config():
    L = sdec.lib()
    w = sdec.RVQWeights(*[0x10000 + 256 * i for i in range(6)])
    for kw, msg in ((dict(vq=100), "vq"), (dict(bins=100), "bins"), (dict(nq=1), "nq"),
                    (dict(dim=6), "dim"), (dict(max_frames=0), "max_frames")):
        c = dict(dim=512, vq=256, bins=2048, nq=8, max_frames=4)
        c.update(kw)
        h = ctypes.c_void_p()
        rc = L.sdec_rvq_create(ctypes.byref(sdec.RVQConfig(**c)), ctypes.byref(w), ctypes.byref(h))
        assert rc == sdec.E_ARG and msg in L.sdec_last_error().decode()
    w.cb_rest = 0x10004
    h = ctypes.c_void_p()
    rc = L.sdec_rvq_create(ctypes.byref(sdec.RVQConfig(512, 256, 2048, 8, 4)), ctypes.byref(w),
                           ctypes.byref(h))
    assert rc == sdec.E_ARG and "cb_rest" in L.sdec_last_error().decode()
    assert L.sdec_rvq_encode(None, 16, 1, 32, None) == sdec.E_ARG
    assert L.sdec_rvq_decode(None, 16, 1, 32, None) == sdec.E_ARG
    L.sdec_rvq_destroy(None)


def test_conv_rejects_bad_config():
    L = sdec.lib()
    base = dict(in_ch=8, out_ch=8, kernel=4, stride=2, groups=1, transposed=0, pre_elu=0,
                replicate_first=0, accumulate=0, max_t_in=16)
    for kw, msg in ((dict(kernel=1), "kernel >= stride"), (dict(groups=4), "groups"),
                    (dict(max_t_in=0), "max_t_in"), (dict(transposed=1, accumulate=1), "forward"),
                    (dict(out_ch=0), "channels")):
        c = dict(base)
        c.update(kw)
        h = ctypes.c_void_p()
        rc = L.sdec_conv_create(ctypes.byref(sdec.ConvConfig(**c)), 16, 32, ctypes.byref(h))
        assert rc == sdec.E_ARG and msg in L.sdec_last_error().decode()
    assert L.sdec_conv_step(None, 16, 4, 32, 1, None) == sdec.E_ARG
    L.sdec_conv_destroy(None)


def test_transpose_checks_on_the_host():
    L = sdec.lib()
    assert L.sdec_transpose(None, 4, 4, 4096, None) == sdec.E_ARG
    assert L.sdec_transpose(4096, 0, 4, 8192, None) == sdec.E_ARG
    # 16 x 512 floats from 0x10000 reach past 0x18000
    assert L.sdec_transpose(0x10000, 16, 512, 0x18000 - 256, None) == sdec.E_ARG
    assert "overlap" in L.sdec_last_error().decode()
    assert L.sdec_transpose(0x10000, 1, 1 << 22, 0x10000000, None) == sdec.E_ARG


def test_one_shot_entry_points_reject_bad_arguments():
    L = sdec.lib()
    assert L.sdec_gemv(None, 16, 32, 4, 4, 1, None) == sdec.E_ARG
    assert L.sdec_gemv(16, 16, 32, 4, 6, 1, None) == sdec.E_ARG  # k not a multiple of 4
    assert L.sdec_gemv(16, 16, 32, 4, 8, 9, None) == sdec.E_ARG  # m out of range
    assert L.sdec_ring_attention(16, 32, 48, 64, 80, 1, 4, 4, 96, 8, 8, 0, None) == sdec.E_ARG
    assert L.sdec_ring_attention(16, 32, 48, 64, 80, 1, 6, 4, 64, 8, 8, 0, None) == sdec.E_ARG
    assert L.sdec_step(None, 16, 0, 1, None) == sdec.E_ARG
    assert L.sdec_reset(None, None) == sdec.E_ARG
    L.sdec_destroy(None)


def test_static_scratch_attention_checks_on_the_host():
    # The entry point that allocates nothing refuses, before any HIP call, arguments the
    # allocating one refuses and any geometry whose scratch exceeds its fixed array.
    L = sdec.lib()
    assert L.sdec_ring_attention_static(16, 32, 48, 64, 80, 1, 4, 4, 96, 8, 8, 0, None) == sdec.E_ARG
    assert L.sdec_ring_attention_static(None, 32, 48, 64, 80, 1, 4, 4, 64, 8, 8, 0, None) == sdec.E_ARG
    # 8 streams x 16 heads of 128 over 100000 slots: about 52 MB of chunk partials
    rc = L.sdec_ring_attention_static(256, 512, 768, 1024, 1280, 8, 16, 8, 128, 100000, 100000, 5,
                                      None)
    assert rc == sdec.E_ARG and "static scratch" in L.sdec_last_error().decode()


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    # with no built library the binding refuses to run: there is no CPU path behind it
    from streaming_ar_transformer_amd import sdec
    monkeypatch.setattr(sdec, "_lib", None)
    monkeypatch.setattr(sdec, "LIB_PATH", str(tmp_path / "libsdec.so"))
    with pytest.raises(ImportError, match="is missing"):
        sdec.lib()
