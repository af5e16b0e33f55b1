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


def test_flowlm_prefill_blocks_equal_single_steps(sd):
    # [pocket] PocketBackboneGpu's doc: the prompt may be fed in chunks or one position at a time
    # with the same hidden states.  Blocks of 8, 5, 16, 3 and 12 rows through sdec_prefill (the
    # k = 1024 eight- and sixteen-row GEMVs with LayerNorm prologues, the sixteen-row generic GEMV
    # for the k = 4096 down projection), then single steps, against the oracle stepping one
    # position at a time; up to the ring's end, where the unbounded stack refuses.
    cfg = wl.CONFIGS[6]
    layers, final = weights(cfg)
    dl, df = device_weights(cfg)
    dec = sd.Decoder(cfg, dl, df, max_prefill=16)
    orc = oracle.OracleDecoder(cfg, layers, final)
    xs = wl.make_inputs(cfg, cfg.ring)
    p = 0
    worst = (1.0, 0.0)
    for t in [8, 5, 16, 3, 12] * 9 + [8] * 4:
        xb = torch.from_numpy(np.ascontiguousarray(xs[p:p + t, 0])).cuda()
        dec.prefill(xb, p, first=(p == 0))
        got = xb.cpu().numpy()
        for r in range(t):
            want = orc.step(xs[p + r], p + r, first=(p + r == 0))
            cos, mx = assert_close_rows(got[r:r + 1], want, f"{cfg.name} prefill pos {p + r}")
            worst = (min(worst[0], cos), max(worst[1], mx))
        p += t
    x = torch.empty((1, cfg.d_model), device="cuda")
    for q in range(p, p + 4):
        x.copy_(torch.from_numpy(xs[q]))
        dec.step(x, q)
        assert_close_rows(x.cpu().numpy(), orc.step(xs[q], q), f"{cfg.name} step pos {q}")
    p += 4
    xb = torch.zeros((8, cfg.d_model), device="cuda")
    dec.set_next_position(cfg.ring - 4)
    with pytest.raises(sd.SdecError) as e:  # a block running past the unbounded ring
        dec.prefill(xb, cfg.ring - 4)
    assert e.value.code == sd.E_CAPACITY
    dec.close()
    log(f"{cfg.name}: {p} positions in blocks and steps, worst cos {worst[0]:.9f} max|d| {worst[1]:.3e}")
