"""Whole-step parity of the HIP path against the CPU oracle on the five workloads (GPU).

Every position of every stream must meet cos >= 0.99999 and max|delta| <= 1e-3; the position
rings must match the oracle bit for bit, including past the ring wrap.  For the LayerScale stacks
the same bar is also applied to the branch taps (attention output, and both projections before
LayerScale), which a 0.01 LayerScale would otherwise hide inside the residual.
"""
import numpy as np
import pytest

import oracle
from oracle import INVALID_POS
from streaming_ar_transformer_amd import workloads as wl
from tests.gpu_helpers import assert_close_rows, cos_maxabs, device_weights, log, weights

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


def read_pos_ring(sd, dec, stream, ring):
    _, _, p = dec.kv_view(stream, 0)
    return sd.copy_from_device(p, ring * 4, np.uint32, (ring,))


def read_kv(sd, dec, cfg, stream, layer, ring):
    k, v, _ = dec.kv_view(stream, layer)
    shape = (ring, cfg.n_kv_heads, cfg.head_dim)
    n = ring * cfg.n_kv_heads * cfg.head_dim * 4
    return sd.copy_from_device(k, n, np.float32, shape), sd.copy_from_device(v, n, np.float32, shape)


def run_parity(sd, cfg, steps, check_every=1, taps=False, ring_check=True, log_every=256):
    layers, final = weights(cfg)
    xs = wl.make_inputs(cfg, steps)
    dec = make(sd, cfg, taps=taps)
    orc = oracle.OracleDecoder(cfg, layers, final)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    worst = (1.0, 0.0)
    for p in range(steps):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p, first=(p == 0))
        t = {} if taps else None
        want = orc.step(xs[p], p, first=(p == 0), taps=t)
        if p % check_every and p != steps - 1:
            continue
        got = x.cpu().numpy()
        cos, mx = assert_close_rows(got, want, f"{cfg.name} pos {p}")
        if p % log_every == log_every - 1:
            log(f"{cfg.name}: {p + 1} positions compared")
        worst = (min(worst[0], cos), max(worst[1], mx))
        if taps:
            for li in range(cfg.n_layers):
                for which, key in enumerate(("attn", "attn_proj", "ffn_proj")):
                    ptr = dec.tap_view(li, which)
                    w_ = t[key][li]
                    g_ = sd.copy_from_device(ptr, w_.nbytes, np.float32, w_.shape)
                    assert_close_rows(g_, w_, f"{cfg.name} pos {p} layer {li} tap {key}")
            # the residual update itself, y - x
            assert_close_rows(got - xs[p], want - xs[p], f"{cfg.name} pos {p} y-x")
        if ring_check:
            for s in range(cfg.m):
                np.testing.assert_array_equal(read_pos_ring(sd, dec, s, cfg.ring), orc.P[s],
                                              err_msg=f"pos ring, pos {p}")
    path = dec.path
    dec.close()
    log(f"{cfg.name} path {path}: {steps} steps, worst cos {worst[0]:.9f} max|d| {worst[1]:.3e}")
    return dec, orc


def test_codec1_full_run_with_taps_and_ring_state(sd):
    cfg = wl.CONFIGS[1]
    run_parity(sd, cfg, cfg.steps, taps=True)


def test_codec1_full_run(sd):
    cfg = wl.CONFIGS[1]
    run_parity(sd, cfg, cfg.steps)


def test_codec2_full_run(sd):
    cfg = wl.CONFIGS[2]
    run_parity(sd, cfg, cfg.steps, ring_check=True)



def test_codec8_full_run(sd):
    cfg = wl.CONFIGS[3]
    run_parity(sd, cfg, cfg.steps, ring_check=True)


def test_codec_kv_ring_contents_past_wrap(sd):
    # K (roped) and V ring rows equal the oracle's, slot by slot, around each wrap.
    cfg = wl.CONFIGS[2]
    layers, final = weights(cfg)
    xs = wl.make_inputs(cfg, 520)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for p in range(520):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p, first=(p == 0))
        orc.step(xs[p], p, first=(p == 0))
        if p in (249, 250, 251, 252, 501, 502, 519):
            for li in range(cfg.n_layers):
                k, v = read_kv(sd, dec, cfg, 0, li, cfg.ring)
                assert np.max(np.abs(k - orc.K[0, li])) <= 1e-3
                assert np.max(np.abs(v - orc.V[0, li])) <= 1e-3
            np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    dec.close()


def test_talker_first_positions(sd):
    # Positions 0..39: up to 20 the attention runs inside the o-projection launch (at most 21
    # legal slots), from 21 on in its own launch.
    cfg = wl.CONFIGS[4]
    run_parity(sd, cfg, 40, ring_check=True)


def test_talker_geometry_two_layers_every_position(sd):
    # The talker's geometry (hidden 2048, 16/8 heads of 128, SwiGLU 6144, qk-norm, rotate_half
    # rope) with two of its layers, over its whole 2048-position run from a fresh stream, compared
    # at every position: the short-context form up to position 20, then the attention launch
    # with 1 to 16 chunks of 128 slots and the o prologue's combine of each count.
    cfg = wl.CONFIGS[4].replace(name="talker2_h2048_m1", n_layers=2)
    run_parity(sd, cfg, cfg.steps, ring_check=True)


def test_talker_m8_two_layers_every_step(sd):
    # The eight-stream talker geometry with two layers over the first 64 steps of its run
    # (positions 4096..4159 after a seeded 4096-position import into every stream), compared at
    # every step (the oracle takes about a second per step here).
    cfg = wl.CONFIGS[5].replace(name="talker2_h2048_m8", n_layers=2, steps=64)
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, cfg.start_pos, list(range(cfg.m)))
    xs = wl.make_inputs(cfg, cfg.steps)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    worst = (1.0, 0.0)
    for i in range(cfg.steps):
        q = cfg.start_pos + i
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, q)
        want = orc.step(xs[i], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"m8 two layers pos {q}")
        worst = (min(worst[0], cos), max(worst[1], mx))
        if i % 16 == 15:
            log(f"m8 two layers: {i + 1} steps compared")
    for s in range(cfg.m):
        np.testing.assert_array_equal(read_pos_ring(sd, dec, s, cfg.ring), orc.P[s])
    assert dec.attention_form == sd.ATTN_SPLIT
    log(f"m8 two layers, {cfg.steps} steps: worst cos {worst[0]:.9f} max|d| {worst[1]:.3e}")
    dec.close()


@pytest.mark.parametrize("short", ["1", "0"])
def test_talker_short_context_over_an_import(sd, short, monkeypatch):
    # Positions 20..21 over a seeded import of 0..19 (the step cannot know the imported history,
    # so it bounds the legal slots by pos + 1 = 21): with the attention inside the o launch and,
    # for comparison, with the attention launch kept.
    monkeypatch.setenv("SDEC_SHORT_ATTN", short)
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, 20, [0])
    xs = wl.make_inputs(cfg, 22)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for q in (20, 21):
        x.copy_(torch.from_numpy(xs[q]))
        dec.step(x, q)
        want = orc.step(xs[q], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"talker short={short} pos {q}")
        assert dec.attention_form == (sd.ATTN_SHORT if short == "1" and q == 20 else sd.ATTN_LIST)
        np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    log(f"talker short={short} over an import: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


def _import_prefill(sd, dec, orc, cfg, n_pos, streams):
    pre = wl.make_prefill(cfg, n_pos=n_pos, streams=streams)
    for s in streams:
        K, V = pre[s]
        positions = np.arange(n_pos)
        orc.import_kv(s, K, V, positions)
        for li in range(cfg.n_layers):
            kp, vp, pp = dec.kv_view(s, li)
            sd.copy_to_device(kp, orc.K[s, li])
            sd.copy_to_device(vp, orc.V[s, li])
        sd.copy_to_device(pp, orc.P[s])
    dec.set_next_position(n_pos)


def test_talker_last_positions_from_prefill(sd):
    # Positions 2040..2047 of the 2048-slot talker, over a seeded prefill of 0..2039.
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, 2040, [0])
    xs = wl.make_inputs(cfg, cfg.steps)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for p in range(2040, 2048):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p)
        want = orc.step(xs[p], p)
        assert_close_rows(x.cpu().numpy(), want, f"talker pos {p}")
        assert dec.attention_form == sd.ATTN_LIST
    np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    with pytest.raises(sd.SdecError) as e:  # the unbounded cache refuses position 2048
        dec.step(x, 2048)
    assert e.value.code == sd.E_CAPACITY
    dec.close()


@pytest.mark.parametrize("p", [130, 300, 600, 1030, 1500])
def test_talker_mid_positions_from_prefill(sd, p):
    # Over a seeded import of positions 0..p-1 the step at p attends p+1 slots: 2, 3, 5, 9 and 12
    # chunks of 128, whose partials the o projection's prologue combines in batches of 4, 8 and 16
    # (the last two partly filled).
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, p, [0])
    xs = wl.make_inputs(cfg, p + 2)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for q in (p, p + 1):
        log(f"talker step at {q} over a {p}-position import")
        x.copy_(torch.from_numpy(xs[q]))
        dec.step(x, q)
        want = orc.step(xs[q], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"talker pos {q}")
        np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    log(f"talker pos {p}..{p + 1}: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


def test_talker_over_a_gapped_import(sd):
    # An imported history with holes (positions 0..99 and 180..299 only; the slots of 100..179
    # keep the empty stamp) and a stamp ahead of the step (position 1900 in slot 1900, which no
    # step before 1900 may attend): the legal lists must leave out exactly those slots.
    cfg = wl.CONFIGS[4]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    K, V = wl.make_prefill(cfg, n_pos=300, streams=[0])[0]
    keep = np.r_[0:100, 180:300]
    orc.import_kv(0, K[:, keep], V[:, keep], keep)
    orc.import_kv(0, K[:, :1], V[:, :1], [1900])  # a stamp ahead of every step below
    orc.next_pos = 300
    for li in range(cfg.n_layers):
        kp, vp, pp = dec.kv_view(0, li)
        sd.copy_to_device(kp, orc.K[0, li])
        sd.copy_to_device(vp, orc.V[0, li])
    sd.copy_to_device(pp, orc.P[0])
    dec.set_next_position(300)
    xs = wl.make_inputs(cfg, 2)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for i, q in enumerate((300, 301)):
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, q)
        want = orc.step(xs[i], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"talker gapped pos {q}")
        np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    log(f"talker gapped import: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


def test_talker_one_stream_long_ring_combines_batches(sd):
    # The talker at one stream over config 5's 4352-slot ring: at positions 4350-4351 the o
    # prologue combines 34 chunk partials (two full batches of 16, then 2); 4352 is refused.
    cfg = wl.CONFIGS[5].replace(m=1)
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, 4350, [0])
    xs = wl.make_inputs(cfg, 2)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for i, q in enumerate((4350, 4351)):
        log(f"one-stream talker step at {q}")
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, q)
        want = orc.step(xs[i], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"talker R4352 pos {q}")
    np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    with pytest.raises(sd.SdecError) as e:
        dec.step(x, 4352)
    assert e.value.code == sd.E_CAPACITY
    log(f"one-stream talker R4352: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


LONG_C = wl.small_config("C", n_layers=2, ring=8320, window=8320, steps=8202)


def test_codec_one_stream_more_than_64_chunks(sd):
    # An 8-head, head_dim-64 stack at one stream with an 8320-slot ring: past position 8191 more
    # than 64 chunks of 128 slots are legal, more than the o prologue's combine takes, so the
    # chunks merge in the attention launch; the outputs still match the oracle.
    cfg = LONG_C
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, 8200, [0])
    xs = wl.make_inputs(cfg, 2)
    x = torch.empty((1, cfg.d_model), device="cuda")
    for i, q in enumerate((8200, 8201)):
        log(f"codec R8320 step at {q}")
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, q)
        want = orc.step(xs[i], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"codec R8320 pos {q}")
        assert_close_rows(x.cpu().numpy() - xs[i], want - xs[i], f"codec R8320 pos {q} y-x")
    np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    log(f"codec R8320: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


def test_talker_m8_last_positions_and_capacity(sd):
    # All 8 streams at positions 4350-4351 over a seeded 4350-position import (the last two steps
    # of the m=8 run); position 4352 is past the 4352-slot ring and is refused.
    cfg = wl.CONFIGS[5]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, 4350, list(range(cfg.m)))
    xs = wl.make_inputs(cfg, 256)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    for q in (4350, 4351):
        log(f"m8 step at {q}")
        x.copy_(torch.from_numpy(xs[q - cfg.start_pos]))
        dec.step(x, q)
        want = orc.step(xs[q - cfg.start_pos], q)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"m8 pos {q}")
        for s in range(cfg.m):
            np.testing.assert_array_equal(read_pos_ring(sd, dec, s, cfg.ring), orc.P[s])
    with pytest.raises(sd.SdecError) as e:
        dec.step(x, 4352)
    assert e.value.code == sd.E_CAPACITY
    log(f"m8 pos 4350..4351: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()
    del orc


def test_talker_m8_from_prefill(sd):
    cfg = wl.CONFIGS[5]
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    _import_prefill(sd, dec, orc, cfg, cfg.start_pos, list(range(cfg.m)))
    xs = wl.make_inputs(cfg, 2)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    for i, p in enumerate((4096, 4097)):
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, p)
        want = orc.step(xs[i], p)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"m8 pos {p}")
        log(f"m8 pos {p}: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


SPLIT_T = wl.small_config("T", n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=2,
                          head_dim=128, d_ff=1024, ring=600, window=520, steps=700).replace(m=3, unbounded=False)


@pytest.mark.parametrize("items", ["2", "8"])
def test_streams_split_attention_long_windowed_ring(sd, items, monkeypatch):
    # Several streams: each stream's legal slots are split evenly over a fixed number of items
    # that walk them in double-buffered passes of 64 slots.  Two items per kv head put up to 260
    # slots (five passes) in one item; the 520-slot window over a 600-slot ring wraps at 600.
    monkeypatch.setenv("SDEC_ATTN_ITEMS", items)
    cfg = SPLIT_T
    layers, final = weights(cfg)
    dec = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    xs = wl.make_inputs(cfg, cfg.steps)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    check = set(range(0, cfg.steps, 37)) | {63, 64, 65, 519, 520, 521, 599, 600, 601, cfg.steps - 1}
    for p in range(cfg.steps):
        want = orc.step(xs[p], p, first=(p == 0))
        if p in check:
            x.copy_(torch.from_numpy(xs[p]))
            dec.step(x, p, first=(p == 0))
            cos, mx = assert_close_rows(x.cpu().numpy(), want, f"split items={items} pos {p}")
        else:
            x.copy_(torch.from_numpy(xs[p]))
            dec.step(x, p, first=(p == 0))
    log(f"split items={items}: last pos cos {cos:.9f} max|d| {mx:.3e}")
    for s in range(cfg.m):
        np.testing.assert_array_equal(read_pos_ring(sd, dec, s, cfg.ring), orc.P[s])
    dec.close()


# ---------------------------------------------------------------------------------------------
# cross-checks on the GPU path itself
# ---------------------------------------------------------------------------------------------

SMALL_T = wl.small_config("T", n_layers=3, d_model=1024, n_q_heads=8, n_kv_heads=4,
                          head_dim=128, d_ff=2816, ring=40, window=40, steps=50)
SMALL_C = wl.small_config("C", n_layers=2, ring=21, window=20, steps=50)


def collect(dec, cfg, xs, positions, firsts=()):
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    outs = []
    for i, p in enumerate(positions):
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, p, first=(i == 0 or p in firsts))
        outs.append(x.cpu().numpy().copy())
    return outs


@pytest.mark.parametrize("cfg", [SMALL_T, SMALL_C], ids=["T", "C"])
def test_graph_replay_equals_eager_and_is_deterministic(sd, cfg):
    # 40 positions: both recorded plans (attention inside the o launch up to 32 legal slots, in its
    # own launch after) replay bit for bit like the eager launches
    xs = wl.make_inputs(cfg, 40)
    pos = list(range(40))
    g1 = collect(make(sd, cfg), cfg, xs, pos)
    g2 = collect(make(sd, cfg), cfg, xs, pos)
    e1 = collect(make(sd, cfg, eager=True), cfg, xs, pos)
    for a, b, c in zip(g1, g2, e1):
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(a, c)


@pytest.mark.parametrize("cfg", [SMALL_T, SMALL_C], ids=["T", "C"])
def test_reset_replays_bitwise_and_first_restarts(sd, cfg):
    xs = wl.make_inputs(cfg, 30)
    dec = make(sd, cfg)
    a = collect(dec, cfg, xs, list(range(30)))
    dec.reset()
    b = collect(dec, cfg, xs, list(range(30)))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    # first=1 in the middle of a stream equals a fresh handle started there
    start = 20 if cfg.family == "T" else 100  # the talker-family ring refuses pos >= ring
    c = collect(dec, cfg, xs, list(range(start, start + 15)))
    fresh = collect(make(sd, cfg), cfg, xs, list(range(start, start + 15)))
    for u, v in zip(c, fresh):
        np.testing.assert_array_equal(u, v)


def test_streams_equal_separate_handles(sd):
    cfg8 = SMALL_T.replace(m=8)
    cfg1 = SMALL_T.replace(m=1)
    xs = wl.make_inputs(cfg8, 12)
    multi = collect(make(sd, cfg8), cfg8, xs, list(range(12)))
    for s in (0, 3, 7):
        single = collect(make(sd, cfg1), cfg1, xs[:, s:s + 1], list(range(12)))
        for p in range(12):
            cos, mx = cos_maxabs(multi[p][s], single[p][0])
            assert cos >= 0.99999 and mx <= 1e-4, (s, p, cos, mx)


def test_position_errors_leave_state_unchanged(sd):
    cfg = SMALL_T
    xs = wl.make_inputs(cfg, 10)
    dec = make(sd, cfg)
    ref = collect(make(sd, cfg), cfg, xs, list(range(10)))
    collect(dec, cfg, xs, list(range(5)))
    x = torch.zeros((cfg.m, cfg.d_model), device="cuda")
    for bad in (7, 4):
        with pytest.raises(sd.SdecError) as e:
            dec.step(x, bad)
        assert e.value.code == sd.E_POS and "contiguous" in str(e.value)
    for p in range(5, 10):
        x.copy_(torch.from_numpy(xs[p]))
        dec.step(x, p)
        np.testing.assert_array_equal(x.cpu().numpy(), ref[p])
    with pytest.raises(sd.SdecError) as e:  # the handle also refuses a bad pointer
        dec.step(x[:, 1:], 10)
    assert e.value.code == sd.E_ARG


def test_resume_from_exported_rings(sd):
    cfg = SMALL_C
    xs = wl.make_inputs(cfg, 40)
    a = make(sd, cfg)
    collect(a, cfg, xs, list(range(25)))
    b = make(sd, cfg)
    for li in range(cfg.n_layers):
        ka, va, pa = a.kv_view(0, li)
        kb, vb, pb = b.kv_view(0, li)
        n = cfg.ring * cfg.n_kv_heads * cfg.head_dim
        sd.copy_to_device(kb, sd.copy_from_device(ka, n * 4, np.float32, (n,)))
        sd.copy_to_device(vb, sd.copy_from_device(va, n * 4, np.float32, (n,)))
    sd.copy_to_device(pb, sd.copy_from_device(pa, cfg.ring * 4, np.uint32, (cfg.ring,)))
    b.set_next_position(25)
    x1 = torch.empty((1, cfg.d_model), device="cuda")
    x2 = torch.empty((1, cfg.d_model), device="cuda")
    for p in range(25, 40):
        x1.copy_(torch.from_numpy(xs[p]))
        x2.copy_(torch.from_numpy(xs[p]))
        a.step(x1, p)
        b.step(x2, p)
        np.testing.assert_array_equal(x1.cpu().numpy(), x2.cpu().numpy())
    assert read_pos_ring(sd, b, 0, cfg.ring).tolist().count(INVALID_POS) == 0


def test_repeated_step_at_one_position_matches_single_steps(sd):
    # bench.py times fixed positions by stepping p again and again after set_next_position(p):
    # each repetition re-stamps slot p with p and rewrites its K/V rows, so every repetition must
    # equal a single step at p over the same imported history (the oracle's import + one step).
    cfg = SMALL_T
    layers, final = weights(cfg)
    p = 23
    pre = wl.make_prefill(cfg, n_pos=p, streams=[0])[0]
    dec = make(sd, cfg)
    pos_ring = np.full(cfg.ring, INVALID_POS, np.uint32)
    pos_ring[:p] = np.arange(p, dtype=np.uint32)
    for li in range(cfg.n_layers):
        kp, vp, pp = dec.kv_view(0, li)
        sd.copy_to_device(kp, pre[0][li])
        sd.copy_to_device(vp, pre[1][li])
    sd.copy_to_device(pp, pos_ring)
    xs = wl.make_inputs(cfg, 4)
    x = torch.empty((cfg.m, cfg.d_model), device="cuda")
    for i in range(4):
        orc = oracle.OracleDecoder(cfg, layers, final)
        orc.import_kv(0, pre[0], pre[1], np.arange(p))
        want = orc.step(xs[i], p)
        dec.set_next_position(p)
        x.copy_(torch.from_numpy(xs[i]))
        dec.step(x, p)
        cos, mx = assert_close_rows(x.cpu().numpy(), want, f"repeat {i} at pos {p}")
        np.testing.assert_array_equal(read_pos_ring(sd, dec, 0, cfg.ring), orc.P[0])
    log(f"repeated steps at pos {p}: cos {cos:.9f} max|d| {mx:.3e}")
    dec.close()


@pytest.mark.parametrize("cid", [4, 2])
def test_begin_in_qkv_launch_equals_separate_begin(sd, cid, monkeypatch):
    # The step begin inside layer 0's q/k/v launch (the default at one stream: the talker's
    # row-stream projection, the codec's register GEMV) and as a launch of its own give
    # bit-identical outputs over positions 0..24 (both forms of the attention).
    cfg = wl.CONFIGS[cid]
    layers, final = weights(cfg)
    monkeypatch.setenv("SDEC_BEGIN_IN_QKV", "0")
    sep = make(sd, cfg)
    monkeypatch.delenv("SDEC_BEGIN_IN_QKV")
    fused = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    xs = wl.make_inputs(cfg, 25)
    a = torch.empty((1, cfg.d_model), device="cuda")
    b = torch.empty((1, cfg.d_model), device="cuda")
    for p in range(25):
        a.copy_(torch.from_numpy(xs[p]))
        b.copy_(torch.from_numpy(xs[p]))
        sep.step(a, p, first=(p == 0))
        fused.step(b, p, first=(p == 0))
        want = orc.step(xs[p], p, first=(p == 0))
        torch.testing.assert_close(a, b, rtol=0, atol=0)
    assert_close_rows(b.cpu().numpy(), want, f"{cfg.name} begin in qkv, pos 24")
    np.testing.assert_array_equal(read_pos_ring(sd, fused, 0, cfg.ring), orc.P[0])
    sep.close()
    fused.close()


def test_codec_end_in_down_equals_end_launch(sd, monkeypatch):
    # A stack without a final norm: the last down projection writing the caller's rows itself
    # (the default at one stream) and a separate end launch give bit-identical outputs.
    cfg = wl.CONFIGS[2]
    layers, final = weights(cfg)
    monkeypatch.setenv("SDEC_END_IN_DOWN", "0")
    sep = make(sd, cfg)
    monkeypatch.delenv("SDEC_END_IN_DOWN")
    fused = make(sd, cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    xs = wl.make_inputs(cfg, 30)
    a = torch.empty((1, cfg.d_model), device="cuda")
    b = torch.empty((1, cfg.d_model), device="cuda")
    for p in range(30):
        a.copy_(torch.from_numpy(xs[p]))
        b.copy_(torch.from_numpy(xs[p]))
        sep.step(a, p, first=(p == 0))
        fused.step(b, p, first=(p == 0))
        want = orc.step(xs[p], p, first=(p == 0))
        torch.testing.assert_close(a, b, rtol=0, atol=0)
        assert_close_rows(b.cpu().numpy(), want, f"codec end in down, pos {p}")
    sep.close()
    fused.close()
