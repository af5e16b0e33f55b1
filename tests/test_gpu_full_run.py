"""The 28-layer talker at one stream compared with the oracle at every position of its
2048-position run ([talker] src/qwen3tts_gpu.rs, module doc: the equality standard holds at
every position).

The oracle needs about ten minutes of CPU time per half of this run, so the tests run only with
SDEC_FULL_PARITY=1, one half per process: positions 0..1535 from an empty ring, and
1536..2047 over a seeded import of positions 0..1535 (the same import the oracle receives).  The
default GPU suite covers the same model at positions 0..39 and 22 further positions, and its
geometry with two layers at every one of the 2048 positions.
"""
import os

import numpy as np
import pytest

import oracle
from streaming_ar_transformer_amd import workloads as wl
from tests.gpu_helpers import assert_close_rows, log, weights
from tests.test_gpu_step import _import_prefill, make, read_pos_ring, run_parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("SDEC_FULL_PARITY") != "1",
                                 reason="minutes of oracle time: set SDEC_FULL_PARITY=1")]

torch = pytest.importorskip("torch")

SPLIT = 1536


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_ar_transformer_amd import sdec
    sdec.lib()
    return sdec


def test_talker_28_layers_first_positions_every_position(sd):
    run_parity(sd, wl.CONFIGS[4], SPLIT, ring_check=True, log_every=32)


def test_talker_28_layers_last_positions_every_position(sd):
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, SPLIT, [0])
    xs = wl.make_inputs(cfg, cfg.steps)
    x = torch.empty((1, cfg.d_model), device="cuda")
    worst = (1.0, 0.0)
    for p in range(SPLIT, cfg.steps):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p)
        want = orc.step(xs[p], p)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"talker pos {p}")
        np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0],
                                      err_msg=f"pos ring, pos {p}")
        worst = (min(worst[0], cos), max(worst[1], mx))
        if p % 32 == 31:
            log(f"{cfg.name}: positions {SPLIT}..{p} compared")
    dec.close()
    log(f"{cfg.name}: {SPLIT}..{cfg.steps - 1} over a {SPLIT}-position import, worst cos "
        f"{worst[0]:.9f} max|d| {worst[1]:.3e}")
