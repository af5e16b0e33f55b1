"""The algorithmic byte counts bench.py divides by time (CPU).

Each weight is read once per step, each live K/V row once, each position-ring word once, and the
new K/V rows, the input row and the output row are moved once.  The counts are checked against
sums written out from the workload shapes (hidden 2048, 16 q / 8 kv heads x 128, SwiGLU 6144,
28 layers, float32), independently of how bench.py groups them.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from streaming_ar_transformer_amd import workloads as wl  # noqa: E402

F = 4  # bytes per float32


def talker_layer_weight_bytes():
    d, hd, hq, hkv, ff = 2048, 128, 16, 8, 6144
    mats = (hq * hd) * d + 2 * (hkv * hd) * d  # wq, wk, wv
    mats += d * (hq * hd)                       # wo
    mats += 2 * ff * d + d * ff                 # gate, up, down
    vecs = d + d + hd + hd                      # attention and FFN RMSNorm gains, q/k norm gains
    return F * (mats + vecs)


def test_talker_layer_bytes():
    assert talker_layer_weight_bytes() == 201_344_000
    assert bench.layer_weight_bytes(wl.CONFIGS[4]) == 201_344_000


@pytest.mark.parametrize("pos", [0, 1, 1023, 2047])
def test_talker_m1_step_bytes(pos):
    cfg = wl.CONFIGS[4]
    kv_row = 2 * F * 8 * 128                      # one position's K and V rows of one layer
    want = 28 * talker_layer_weight_bytes() + F * 2048  # + the final norm gain
    want += 28 * (kv_row * (pos + 1) + kv_row + F * 2048)  # live K/V rows, new rows, position ring
    want += 2 * F * 2048                          # input and output rows
    assert bench.step_bytes(cfg, pos, cfg.ring, cfg.window) == want


def test_talker_m1_run_figures():
    # 5.638 GB at p = 0, 6.108 GB at p = 2047, 5.873 GB on average over positions 0..2047
    cfg = wl.CONFIGS[4]
    b = [bench.step_bytes(cfg, p, cfg.ring, cfg.window) for p in range(cfg.ring)]
    assert round(b[0] / 1e9, 3) == 5.638
    assert round(b[-1] / 1e9, 3) == 6.108
    assert round(sum(b) / len(b) / 1e9, 3) == 5.873
    assert 28 * 201_344_000 + 8_192 == 5_637_640_192  # weights of the whole stack


def test_talker_m8_run_average():
    # weights once per step for all 8 streams; K/V per stream at positions 4096..4351
    cfg = wl.CONFIGS[5]
    b = [bench.step_bytes(cfg, 4096 + i, cfg.ring, cfg.window) for i in range(256)]
    avg = sum(b) / len(b)
    assert abs(avg / 1e9 - 13.39) < 0.01          # 5.64 GB of weights + 7.75 GB of K/V
    kv_row = 2 * F * 8 * 128
    live = 8 * 28 * kv_row * (4096 + 128.5)        # live rows, mean over positions 4096..4351
    other = 8 * (28 * (kv_row + F * 4352) + 2 * F * 2048)  # new rows, position rings, in/out rows
    assert avg == 5_637_640_192 + live + other


def test_codec_steady_state_bytes():
    # per layer: 12,595,200 B of weights, 4096 B per live position, 4R of position ring
    for cid, layers, want_mb in ((1, 1, 13.63), (2, 2, 27.25), (3, 8, 109.0)):
        cfg = wl.CONFIGS[cid]
        assert bench.layer_weight_bytes(cfg) == 12_595_200
        pos = 5000  # the ring is full
        b = bench.step_bytes(cfg, pos, cfg.ring, cfg.window)
        live = min(cfg.window, cfg.ring)
        want = layers * (12_595_200 + 4096 * live + 4096 + F * cfg.ring) + 2 * F * 512
        assert b == want
        assert round(b / 1e6, 2) == pytest.approx(want_mb, abs=0.01)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""  # no JSON line
