"""Parity of further configurations of the same step (GPU): the FlowLM backbone variant.

[pocket] ``PocketBackboneGpu::new`` runs the codec builder's layer with no LayerScale and no
window (window == ring == max_positions, unbounded), then an output LayerNorm and an EOS logit
whose bias is added on the host.  Every position meets the step bar (cos >= 0.99999, max|delta|
<= 1e-3); the logit, from ``sdec_gemv`` on the step's output row, is held to 1e-3.
"""
import numpy as np
import pytest

import oracle
from streaming_ar_transformer_amd import workloads as wl
from tests.gpu_helpers import assert_close_rows, device_weights, log, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_ar_transformer_amd import sdec
    sdec.lib()
    return sdec


def test_flowlm_variant_steps_and_eos_logit(sd):
    cfg = wl.CONFIGS[6]
    layers, final = weights(cfg)
    dl, df = device_weights(cfg)
    eos_w, eos_b = wl.make_eos(cfg)
    dec = sd.Decoder(cfg, dl, df)
    orc = oracle.OracleDecoder(cfg, layers, final)
    xs = wl.make_inputs(cfg, cfg.ring)
    x = torch.empty((1, cfg.d_model), device="cuda")
    w_dev = torch.from_numpy(eos_w).cuda()
    logit = torch.empty((1, 1), device="cuda")
    worst = (1.0, 0.0)
    worst_logit = 0.0
    for p in range(cfg.ring):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p, first=(p == 0))
        want = orc.step(xs[p], p, first=(p == 0))
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"{cfg.name} pos {p}")
        worst = (min(worst[0], cos), max(worst[1], mx))
        if p % 16 == 0 or p == cfg.ring - 1:
            sd.gemv(w_dev, x, logit)
            got = float(logit.cpu()[0, 0]) + eos_b
            ref = float(oracle.gemv(eos_w, want)[0, 0]) + eos_b
            worst_logit = max(worst_logit, abs(got - ref))
            assert abs(got - ref) <= 1e-3, f"EOS logit pos {p}: {got} vs {ref}"
    with pytest.raises(sd.SdecError) as e:  # unbounded: no position past the ring
        dec.step(x, cfg.ring)
    assert e.value.code == sd.E_CAPACITY
    dec.close()
    log(f"{cfg.name}: {cfg.ring} steps, worst cos {worst[0]:.9f} max|d| {worst[1]:.3e}, "
        f"EOS logit max|d| {worst_logit:.2e}")
