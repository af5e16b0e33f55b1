"""A Pocket-style codec frame on the GPU against the oracle's offline decode ([pocket] module doc
decode graph; PocketCodecGpu::new / decode_frame / reset).

Twenty latents go through ``PocketCodecFrame.decode_frame`` one at a time: 1x1 conv, channel-wise
transposed conv k32/s16, transpose, the 2-layer d512 transformer over 16 positions per frame
(one prefill block of 16; ring 266, window 250, so the run passes the ring's wrap at position
266), transpose, SEANet.  Every frame's transformer rows and samples must meet the per-row bar
(cosine >= 0.99999, max|delta| <= 1e-3); a restart with ``first`` must reproduce the first
frames.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_close_rows, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def frame_setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_ar_transformer_amd import sdec
    from streaming_ar_transformer_amd import workloads as wl
    sdec.lib()
    cfg = wl.POCKET_CONFIGS[1]
    conv, trl, sw = wl.make_pocket_frame(cfg)
    want = oracle.decode_frames(conv["latents"], conv, cfg.transformer, trl,
                                wl.seanet_layers(cfg.seanet), sw, cfg.up_stride)
    return cfg, conv, trl, sw, want


def test_pocket_frames_match_the_offline_decode(frame_setup):
    from streaming_ar_transformer_amd.device import upload_weights
    from streaming_ar_transformer_amd.pocket import PocketCodecFrame
    cfg, conv, trl, sw, want = frame_setup
    dconv = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in conv.items()}
    dtr, _ = upload_weights(trl, {})
    dsw = {k: torch.from_numpy(v).cuda() for k, v in sw.items()}
    fr = PocketCodecFrame(cfg, dconv, dtr, dsw)
    s, n = cfg.up_stride, cfg.samples_per_frame
    worst = (1.0, 0.0)
    for f in range(cfg.frames):
        log(f"{cfg.name}: frame {f} (positions {f * s}..{f * s + s - 1})")
        pcm = fr.decode_frame(dconv["latents"][f], first=(f == 0)).cpu().numpy()
        tr = fr.y_ct.cpu().numpy()
        assert_close_rows(tr.T, want["tr"][:, f * s:(f + 1) * s].T, f"frame {f} transformer")
        cos, mx = assert_close_rows(pcm, want["pcm"][:, f * n:(f + 1) * n], f"frame {f} samples")
        worst = (min(worst[0], cos), max(worst[1], mx))
    # a fresh stream on the same handles: the first frames again
    for f in range(2):
        pcm = fr.decode_frame(dconv["latents"][f], first=(f == 0)).cpu().numpy()
        assert_close_rows(pcm, want["pcm"][:, f * n:(f + 1) * n], f"restarted frame {f}")
    fr.close()
    log(f"{cfg.name}: {cfg.frames} frames of {n} samples, worst cos {worst[0]:.9f} "
        f"max|d| {worst[1]:.2e}")


def test_transpose_matches_numpy():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_ar_transformer_amd import sdec
    for rows, cols in ((512, 16), (16, 512), (33, 65), (1, 7), (100, 1)):
        x = torch.randn((rows, cols), device="cuda")
        y = torch.empty((cols, rows), device="cuda")
        sdec.transpose(x, y)
        assert torch.equal(y.cpu(), x.cpu().T.contiguous()), (rows, cols)
