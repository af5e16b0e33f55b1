"""Parity of the multi-position prefill (``sdec_prefill``) against the CPU oracle (GPU).

A block of t consecutive positions in one call must give, row by row, what t single decode steps
give ([talker] ``TalkerGpu::prefill``; [pocket] ``PocketBackboneGpu``: chunked and one-at-a-time
feeding agree), and leave the same rings, so decode steps can follow.  Same bar as the step
parity: cos >= 0.99999 and max|delta| <= 1e-3 per row, position rings bit-exact.
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


def make(sd, cfg, **kw):
    dl, df = device_weights(cfg)
    return sd.Decoder(cfg, dl, df, **kw)


def read_pos_ring(sd, dec, ring):
    _, _, p = dec.kv_view(0, 0)
    return sd.copy_from_device(p, ring * 4, np.uint32, (ring,))


def run_blocks(sd, cfg, blocks, decode_after, ring=None, check_kv=False):
    """Prefill `blocks` (sizes) from position 0, then `decode_after` single steps; every output
    row against the oracle stepping one position at a time."""
    ring = cfg.ring if ring is None else ring
    layers, final = weights(cfg)
    n = sum(blocks) + decode_after
    xs = wl.make_inputs(cfg, n)
    dec = make(sd, cfg, ring=ring, max_prefill=max(blocks))
    orc = oracle.OracleDecoder(cfg, layers, final, ring=ring)
    worst = (1.0, 0.0)
    p = 0
    for t in blocks:
        xb = torch.from_numpy(np.ascontiguousarray(xs[p:p + t, 0])).cuda()
        print(f"prefill {cfg.name} pos {p} t {t}", flush=True)
        dec.prefill(xb, p, first=(p == 0))
        got = xb.cpu().numpy()
        for r in range(t):
            want = orc.step(xs[p + r], p + r, first=(p + r == 0))
            cos, mx = assert_close_rows(got[r:r + 1], want, f"{cfg.name} prefill pos {p + r}")
            worst = (min(worst[0], cos), max(worst[1], mx))
        np.testing.assert_array_equal(read_pos_ring(sd, dec, ring), orc.P[0],
                                      err_msg=f"pos ring after block at {p}")
        p += t
    x = torch.empty((1, cfg.d_model), device="cuda")
    for q in range(p, n):
        x.copy_(torch.from_numpy(xs[q]))
        dec.step(x, q)
        want = orc.step(xs[q], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"{cfg.name} decode pos {q}")
        worst = (min(worst[0], cos), max(worst[1], mx))
    if check_kv:
        for li in range(cfg.n_layers):
            k, v, _ = dec.kv_view(0, li)
            shape = (ring, cfg.n_kv_heads, cfg.head_dim)
            nb = ring * cfg.n_kv_heads * cfg.head_dim * 4
            kk = sd.copy_from_device(k, nb, np.float32, shape)
            vv = sd.copy_from_device(v, nb, np.float32, shape)
            assert np.max(np.abs(kk - orc.K[0, li])) <= 1e-3
            assert np.max(np.abs(vv - orc.V[0, li])) <= 1e-3
    dec.close()
    log(f"{cfg.name} prefill blocks {blocks} + {decode_after} steps: worst cos {worst[0]:.9f} "
        f"max|d| {worst[1]:.3e}")


def test_talker_prefill_blocks_then_decode(sd):
    cfg = wl.CONFIGS[4]
    run_blocks(sd, cfg, [8, 3, 8, 1, 5], decode_after=4)


def test_talker_prefill_over_long_imported_history(sd):
    # Blocks whose rows attend 600+ legal slots: several attention chunks per row, merged.
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    start = 600
    pre = wl.make_prefill(cfg, n_pos=start, streams=[0])[0]
    dec = make(sd, cfg, max_prefill=8)
    orc = oracle.OracleDecoder(cfg, layers, final)
    orc.import_kv(0, pre[0], pre[1], np.arange(start))
    for li in range(cfg.n_layers):
        kp, vp, pp = dec.kv_view(0, li)
        sd.copy_to_device(kp, pre[0][li])
        sd.copy_to_device(vp, pre[1][li])
    sd.copy_to_device(pp, orc.P[0])
    dec.set_next_position(start)
    xs = wl.make_inputs(cfg, 13)
    p = start
    for t in (8, 5):
        xb = torch.from_numpy(np.ascontiguousarray(xs[p - start:p - start + t, 0])).cuda()
        print(f"prefill {cfg.name} pos {p} t {t}", flush=True)
        dec.prefill(xb, p)
        got = xb.cpu().numpy()
        want = orc.prefill(xs[p - start:p - start + t, 0], p)
        cos, mx = assert_close_rows(got, want, f"{cfg.name} prefill block at {p}")
        np.testing.assert_array_equal(read_pos_ring(sd, dec, cfg.ring), orc.P[0])
        p += t
    dec.close()
    log(f"{cfg.name} prefill over {start} imported positions: cos {cos:.9f} max|d| {mx:.3e}")


def test_codec_prefill_across_ring_wraps(sd):
    # ring = window + 7: any block of up to 8 rows is legal after the ring wraps (257, 514)
    cfg = wl.CONFIGS[3]
    sizes = [8, 7, 5, 8, 1, 6, 8, 3, 8, 2]
    blocks = (sizes * 8)[:70]
    while sum(blocks) > 560:
        blocks.pop()
    run_blocks(sd, cfg, blocks, decode_after=6, ring=cfg.window + 7, check_kv=True)


def test_prefill_restart_with_first(sd):
    # first != 0 on a later block starts a fresh stream at that position
    cfg = wl.CONFIGS[1]
    ring = cfg.window + 7
    layers, final = weights(cfg)
    xs = wl.make_inputs(cfg, 40)
    dec = make(sd, cfg, ring=ring, max_prefill=8)
    orc = oracle.OracleDecoder(cfg, layers, final, ring=ring)
    xb = torch.from_numpy(np.ascontiguousarray(xs[0:8, 0])).cuda()
    dec.prefill(xb, 0, first=True)
    for r in range(8):
        orc.step(xs[r], r, first=(r == 0))
    xb = torch.from_numpy(np.ascontiguousarray(xs[8:14, 0])).cuda()
    dec.prefill(xb, 100, first=True)
    got = xb.cpu().numpy()
    for r in range(6):
        want = orc.step(xs[8 + r], 100 + r, first=(r == 0))
        assert_close_rows(got[r:r + 1], want, f"restart pos {100 + r}")
    np.testing.assert_array_equal(read_pos_ring(sd, dec, ring), orc.P[0])
    dec.close()


def test_prefill_argument_errors(sd):
    cfg = wl.CONFIGS[1]
    x8 = torch.zeros((8, cfg.d_model), device="cuda")
    x2 = torch.zeros((2, cfg.d_model), device="cuda")
    # the workload's ring == window: a block past the first ring turn would evict a live position
    dec = make(sd, cfg, max_prefill=8)
    dec.prefill(x8, 0, first=True)  # inside the first ring turn
    with pytest.raises(sd.SdecError) as e:
        dec.prefill(x8, 9)  # not the next position
    assert e.value.code == sd.E_POS
    xs = torch.zeros((1, cfg.d_model), device="cuda")
    for p in range(8, cfg.ring - 1):
        dec.step(xs, p)
    with pytest.raises(sd.SdecError) as e:
        dec.prefill(x2, cfg.ring - 1)
    assert e.value.code == sd.E_CAPACITY
    dec.prefill(x2[:1], cfg.ring - 1)  # one row never evicts a live position
    with pytest.raises(sd.SdecError) as e:
        dec.prefill(torch.zeros((9, cfg.d_model), device="cuda"), cfg.ring)
    assert e.value.code == sd.E_ARG  # more rows than max_prefill
    dec.close()
    # the talker's unbounded cache refuses a block reaching past its capacity
    tcfg = wl.CONFIGS[4].replace(n_layers=2)
    dl, df = device_weights(wl.CONFIGS[4])
    tdec = sd.Decoder(tcfg, dl[:2], df, max_prefill=8)
    tdec.set_next_position(tcfg.ring - 4)
    with pytest.raises(sd.SdecError) as e:
        tdec.prefill(torch.zeros((8, tcfg.d_model), device="cuda"), tcfg.ring - 4)
    assert e.value.code == sd.E_CAPACITY
    tdec.close()


def test_codec_prefill_end_in_down_equals_end_launch(sd, monkeypatch):
    # A stack without a final norm: the last down projection writing the caller's rows (the
    # default) and a separate end launch give bit-identical blocks, ring wraps included.
    cfg = wl.CONFIGS[2]
    ring = cfg.window + 7
    monkeypatch.setenv("SDEC_END_IN_DOWN", "0")
    sep = make(sd, cfg, ring=ring, max_prefill=8)
    monkeypatch.delenv("SDEC_END_IN_DOWN")
    fused = make(sd, cfg, ring=ring, max_prefill=8)
    xs = wl.make_inputs(cfg, 296)
    p = 0
    for t in [8, 3, 8, 5] * 10:
        a = torch.from_numpy(np.ascontiguousarray(xs[p:p + t, 0])).cuda()
        b = a.clone()
        sep.prefill(a, p, first=(p == 0))
        fused.prefill(b, p, first=(p == 0))
        torch.testing.assert_close(a, b, rtol=0, atol=0)
        p += t
    sep.close()
    fused.close()
    log(f"{cfg.name}: {p} positions in blocks, fused and separate end bit-identical")


def test_codec_prefill_blocks_of_sixteen(sd):
    # Blocks of 9..16 rows take the sixteen-row GEMV shapes (k = 512 and 2048, one float4 per lane
    # and row); ring = window + 15 so every block stays legal after the ring wraps (265, 530).
    cfg = wl.CONFIGS[2]
    blocks = [16, 9, 16, 12, 16, 15, 1, 16, 13, 10] * 6
    while sum(blocks) > 620:
        blocks.pop()
    run_blocks(sd, cfg, blocks, decode_after=4, ring=cfg.window + 15, check_kv=True)
