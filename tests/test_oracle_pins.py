"""Pins of the CPU oracle against facts fixed by the pages and by mathematics (no GPU).

Each test holds one part of ``oracle/`` to something other than itself: closed forms, textbook
values, identities, exact small-integer arithmetic, or the independent float64 brute force in
``tests/brute.py``.  They are chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import F32, INVALID_POS
from streaming_ar_transformer_amd import workloads as wl
from tests.brute import BruteDecoder

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# sums and GEMV
# ---------------------------------------------------------------------------------------------

def test_seq_sum_is_left_to_right():
    # A pairwise or blocked sum of this vector differs from the sequential one.
    a = np.array([1e8, 1.0, 1.0, 1.0, 1.0, -1e8, 3.0, 0.5], dtype=F32)
    acc = F32(0.0)
    for t in a:
        acc = F32(acc + t)
    assert oracle.seq_sum(a) == acc
    assert oracle.seq_sum(a) == F32(3.5)  # every +1 is absorbed by 1e8 in f32


def test_seq_sum_rows():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((300, 7)).astype(F32)
    acc = np.zeros(7, F32)
    for row in a:
        acc = (acc + row).astype(F32)
    np.testing.assert_array_equal(oracle.seq_sum(a), acc)


def test_gemv_small_integers_exact():
    # |w|,|x| <= 4 and k = 6144: every partial sum is an integer below 2^24, so any order is exact.
    rng = np.random.default_rng(1)
    w = rng.integers(-4, 5, size=(96, 6144)).astype(F32)
    x = rng.integers(-4, 5, size=(3, 6144)).astype(F32)
    exact = x.astype(np.int64) @ w.astype(np.int64).T
    np.testing.assert_array_equal(oracle.gemv(w, x), exact.astype(F32))


def test_gemv_orientation_brute():
    # Non-square W catches a transposed operand; the reference is an explicit double loop.
    rng = np.random.default_rng(2)
    w = rng.standard_normal((5, 3)).astype(F32)
    x = rng.standard_normal((2, 3)).astype(F32)
    ref = [[math.fsum(float(w[n, k]) * float(x[r, k]) for k in range(3)) for n in range(5)]
           for r in range(2)]
    np.testing.assert_allclose(oracle.gemv(w, x), np.array(ref), rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------------------------
# norms
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("c", [0.5, 3.0, -2.0])
def test_rms_norm_constant_row(c):
    g = np.random.default_rng(3).standard_normal(64).astype(F32)
    y = oracle.rms_norm(np.full(64, c, F32), g, 1e-6)
    np.testing.assert_allclose(y, c * g / math.sqrt(c * c + 1e-6), rtol=2e-6)


def test_rms_norm_unit_gain_has_unit_rms():
    x = np.random.default_rng(4).standard_normal(2048).astype(F32) * 7
    y = oracle.rms_norm(x, np.ones(2048, F32), 1e-6)
    ms = float(np.mean(x.astype(np.float64) ** 2))
    assert abs(float(np.mean(y.astype(np.float64) ** 2)) - ms / (ms + 1e-6)) < 1e-5


def test_qk_norm_never_mixes_heads():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((16, 128)).astype(F32)
    g = rng.standard_normal(128).astype(F32)
    a = oracle.rms_norm(q, g, 1e-6)
    q2 = q.copy()
    q2[3] *= 10
    q2[7, 5] += 1
    b = oracle.rms_norm(q2, g, 1e-6)
    keep = [h for h in range(16) if h not in (3, 7)]
    np.testing.assert_array_equal(a[keep], b[keep])
    np.testing.assert_allclose(a[3], b[3], rtol=1e-5, atol=1e-6)  # scale invariance


def test_layer_norm_constant_row_gives_bias_exactly():
    rng = np.random.default_rng(6)
    w, b = rng.standard_normal(512).astype(F32), rng.standard_normal(512).astype(F32)
    np.testing.assert_array_equal(oracle.layer_norm(np.full(512, 2.5, F32), w, b, 1e-5), b)


def test_layer_norm_moments_and_shift_invariance():
    x = np.random.default_rng(7).standard_normal(512).astype(F32) * 3 + 5
    y = oracle.layer_norm(x, np.ones(512, F32), np.zeros(512, F32), 1e-5).astype(np.float64)
    var = float(np.var(x.astype(np.float64)))
    assert abs(y.mean()) < 1e-6
    assert abs(y.var() - var / (var + 1e-5)) < 1e-5
    y2 = oracle.layer_norm(x - F32(5), np.ones(512, F32), np.zeros(512, F32), 1e-5)
    np.testing.assert_allclose(y2, y, atol=2e-5)


# ---------------------------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------------------------

def test_gelu_textbook_values():
    # GELU(x) = x * Phi(x); Phi(1), Phi(2), Phi(-1) from the standard normal table.
    v = np.array([0.0, 1.0, 2.0, -1.0], F32)
    ref = [0.0, 0.8413447460685429, 2 * 0.9772498680518208, -0.15865525393145707]
    np.testing.assert_allclose(oracle.gelu_erf(v), ref, rtol=1e-7, atol=0)
    x = np.linspace(-6, 6, 97).astype(F32)
    np.testing.assert_allclose(oracle.gelu_erf(x) - oracle.gelu_erf(-x), x, atol=1e-6)


def test_silu_closed_forms():
    # sigma(ln 3) = 3/4, silu(0) = 0, silu(x) - silu(-x) = x.
    g = np.array([math.log(3.0), 0.0], F32)
    y = oracle.silu_mul(g, np.ones(2, F32))
    assert abs(float(y[0]) - 0.75 * math.log(3.0)) < 1e-7 and y[1] == 0
    x = np.linspace(-8, 8, 65).astype(F32)
    one = np.ones_like(x)
    np.testing.assert_allclose(oracle.silu_mul(x, one) - oracle.silu_mul(-x, one), x, atol=2e-6)
    np.testing.assert_allclose(oracle.silu_mul(x, 2 * one), 2 * oracle.silu_mul(x, one), rtol=0)


# ---------------------------------------------------------------------------------------------
# rope
# ---------------------------------------------------------------------------------------------

def test_rope_frequencies_closed_form():
    # hd = 64, theta = 1e4: frequency index 16 has inverse frequency 1e4^(-1/2) = 0.01.
    c, s = oracle.rope_cos_sin(7, 64, 1e4)
    assert c[0] == F32(math.cos(7.0)) and s[0] == F32(math.sin(7.0))
    assert c[16] == F32(math.cos(0.07)) and s[16] == F32(math.sin(0.07))
    # hd = 128, theta = 1e6: index 32 has inverse frequency 1e6^(-1/2) = 1e-3.
    c, s = oracle.rope_cos_sin(1000, 128, 1e6)
    assert c[32] == F32(math.cos(1.0)) and s[32] == F32(math.sin(1.0))


@pytest.mark.parametrize("style", [oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED])
def test_rope_identity_at_zero_and_norm(style):
    x = np.random.default_rng(8).standard_normal((4, 128)).astype(F32)
    c, s = oracle.rope_cos_sin(0, 128, 1e6)
    np.testing.assert_array_equal(oracle.apply_rope(x, c, s, style), x)
    c, s = oracle.rope_cos_sin(1234, 128, 1e6)
    y = oracle.apply_rope(x, c, s, style)
    ia, ib = oracle.rope_pairs(128, style)
    np.testing.assert_allclose(y[:, ia] ** 2 + y[:, ib] ** 2, x[:, ia] ** 2 + x[:, ib] ** 2,
                               rtol=1e-5)


def test_rope_interleaved_is_complex_multiplication():
    x = np.random.default_rng(9).standard_normal(64).astype(F32)
    pos, theta = 37, 1e4
    c, s = oracle.rope_cos_sin(pos, 64, theta)
    y = oracle.apply_rope(x, c, s, oracle.ROPE_INTERLEAVED)
    z = (x[0::2] + 1j * x[1::2]).astype(np.complex128)
    w = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(32) / 64))
    np.testing.assert_allclose(y[0::2], w.real, atol=2e-6)
    np.testing.assert_allclose(y[1::2], w.imag, atol=2e-6)


def test_rope_half_is_permuted_interleaved():
    # Reordering (j, j+hd/2) -> (2j, 2j+1) turns rotate_half into the interleaved form, exactly.
    x = np.random.default_rng(10).standard_normal(128).astype(F32)
    c, s = oracle.rope_cos_sin(999, 128, 1e6)
    perm = np.empty(128, np.int64)
    perm[0::2] = np.arange(64)
    perm[1::2] = np.arange(64) + 64
    np.testing.assert_array_equal(oracle.apply_rope(x, c, s, oracle.ROPE_HALF)[perm],
                                  oracle.apply_rope(x[perm], c, s, oracle.ROPE_INTERLEAVED))


def test_rope_relative_position():
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal(128).astype(F32), rng.standard_normal(128).astype(F32)

    def dot(m, n):
        cm, sm = oracle.rope_cos_sin(m, 128, 1e6)
        cn, sn = oracle.rope_cos_sin(n, 128, 1e6)
        return float(np.dot(oracle.apply_rope(q, cm, sm, 0).astype(np.float64),
                            oracle.apply_rope(k, cn, sn, 0).astype(np.float64)))

    assert abs(dot(10, 3) - dot(1010, 1003)) < 2e-4
    assert abs(dot(10, 3) - dot(10, 4)) > 1e-3  # and it does depend on the offset


@pytest.mark.parametrize("sections", ["contiguous", "interleaved"])
def test_mrope_uniform_positions_equal_1d(sections):
    # Multimodal rope assigns each frequency index to one of three position streams (temporal,
    # height, width).  With the three positions equal it is 1-D rope, bit for bit.
    hd, theta, pos = 128, 1e6, 517
    half = hd // 2
    rng = np.random.default_rng(12)
    if sections == "contiguous":
        cut = np.sort(rng.choice(np.arange(1, half), 2, replace=False))
        stream = np.searchsorted(cut, np.arange(half), side="right")
    else:
        stream = np.arange(half) % 3
    positions = np.array([pos, pos, pos], np.float64)
    j = np.arange(half, dtype=np.float64)
    ang = positions[stream] * np.power(theta, -2.0 * j / hd)
    c1, s1 = oracle.rope_cos_sin(pos, hd, theta)
    np.testing.assert_array_equal(np.cos(ang).astype(F32), c1)
    np.testing.assert_array_equal(np.sin(ang).astype(F32), s1)


# ---------------------------------------------------------------------------------------------
# ring attention
# ---------------------------------------------------------------------------------------------

def test_attention_closed_form_mean_of_valid_positions():
    # q = 0 makes every legal score 0; with V[s, 0] = P[s] dim 0 of the output is the mean of
    # the legal positions -- pos - (W - 1) / 2 once the window is full.
    R, W, hd = 7, 5, 8
    for pos in range(0, 30):
        P = np.full(R, INVALID_POS, np.uint32)
        for p in range(max(0, pos - R + 1), pos + 1):
            P[p % R] = p
        K = np.random.default_rng(pos).standard_normal((R, 1, hd)).astype(F32)
        V = np.zeros((R, 1, hd), F32)
        V[:, 0, 0] = np.where(P == INVALID_POS, 1e6, P.astype(np.float64))
        o = oracle.attend(np.zeros((1, hd), F32), K, V, P, pos, W, 1, False)
        lo = max(0, pos - W + 1)
        assert o[0, 0] == F32((lo + pos) / 2.0)


def test_attention_sequential_order_bit_exact():
    # Scores from small integers are exact, so e, den and the value sums can be replayed with
    # explicit float32 loops in ascending position order.
    rng = np.random.default_rng(13)
    R, hd = 9, 4
    P = np.array([5, 6, 7, 8, 0, 1, 2, 3, 4], np.uint32)  # wrapped: slot 4 holds position 0
    K = rng.integers(-2, 3, size=(R, 1, hd)).astype(F32)
    V = rng.standard_normal((R, 1, hd)).astype(F32)
    q = rng.integers(-2, 3, size=(1, hd)).astype(F32)
    order = np.argsort(P)
    s = np.array([float(K[j, 0] @ q[0]) for j in order], F32) * (F32(1) / np.sqrt(F32(hd)))
    e = np.exp(s - s.max()).astype(F32)
    den = F32(0)
    for t in e:
        den = F32(den + t)
    acc_t = np.zeros(hd, F32)
    acc_c = np.zeros(hd, F32)
    for t, j in zip(e, order):
        acc_t = (acc_t + (t / den) * V[j, 0]).astype(F32)
        acc_c = (acc_c + t * V[j, 0]).astype(F32)
    np.testing.assert_array_equal(oracle.attend(q, K, V, P, 8, 100, 1, True)[0], acc_t)
    np.testing.assert_array_equal(oracle.attend(q, K, V, P, 8, 100, 1, False)[0], acc_c / den)


def test_attention_mask_rules():
    P = np.array([3, INVALID_POS, 9, 10, 4], np.uint32)
    assert list(oracle.valid_slots(P, 9, 100)) == [0, 4, 2]  # 10 > pos, INVALID skipped
    assert list(oracle.valid_slots(P, 9, 6)) == [4, 2]  # 9 - 3 = 6 is outside a 6-window
    assert list(oracle.valid_slots(P, 2, 100)) == []


# ---------------------------------------------------------------------------------------------
# whole-step pins against the independent float64 brute force
# ---------------------------------------------------------------------------------------------

def tiny(family, **kw):
    if family == "T":
        base = dict(n_layers=2, d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=4, d_ff=24,
                    ring=64, window=64, steps=12)
    else:
        base = dict(n_layers=2, d_model=16, n_q_heads=2, n_kv_heads=2, head_dim=8, d_ff=32,
                    ring=5, window=4, steps=15, layer_scale_init=0.5)
    base.update(kw)
    return wl.small_config(family, **base)


@pytest.mark.parametrize("family,kw", [
    ("T", {}),
    ("C", {}),                       # ring 5 > window 4: the mask, not the overwrite, hides keys
    ("C", dict(ring=4, window=4)),   # ring == window: exact at one position per step
    ("C", dict(layer_scale=False)),
    ("C", dict(random_ls=True)),     # distinct LayerScale vectors per branch and layer
])
def test_step_matches_brute_force(family, kw):
    kw = dict(kw)
    random_ls = kw.pop("random_ls", False)
    cfg = tiny(family, **kw)
    layers, final = wl.make_weights(cfg)
    if random_ls:
        rng = np.random.default_rng(14)
        for lw in layers:
            lw["ls1"] = rng.uniform(0.1, 1.0, cfg.d_model).astype(F32)
            lw["ls2"] = rng.uniform(-1.0, -0.1, cfg.d_model).astype(F32)
    xs = wl.make_inputs(cfg)
    orc = oracle.OracleDecoder(cfg, layers, final)
    bru = BruteDecoder(cfg, layers, final, cfg.window)
    for p in range(cfg.steps):
        y = orc.step(xs[p], p, first=(p == 0))
        ref = np.array(bru.step(xs[p, 0], p))
        np.testing.assert_allclose(y[0], ref, rtol=2e-5, atol=2e-5, err_msg=f"pos {p}")


@pytest.mark.parametrize("family,kw,blocks", [
    ("T", {}, [5, 1, 3, 3]),
    ("C", dict(ring=7, window=4), [4, 2, 4, 1, 3, 4, 2]),  # wraps the 7-slot ring several times
])
def test_prefill_blocks_match_brute_force(family, kw, blocks):
    # A block of t positions in one pass ([talker] forward_rows: append the block's K/V, then
    # causal attention) equals the float64 brute force fed one position at a time.
    cfg = tiny(family, **kw)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, sum(blocks))
    orc = oracle.OracleDecoder(cfg, layers, final)
    bru = BruteDecoder(cfg, layers, final, cfg.window)
    p = 0
    for t in blocks:
        y = orc.prefill(xs[p:p + t, 0], p, first=(p == 0))
        assert y.shape == (t, cfg.d_model)
        for r in range(t):
            ref = np.array(bru.step(xs[p + r, 0], p + r))
            np.testing.assert_allclose(y[r], ref, rtol=2e-5, atol=2e-5, err_msg=f"pos {p + r}")
        p += t
    assert orc.next_pos == p


def test_prefill_equals_single_steps_and_keeps_the_ring():
    # Chunk invariance ([pocket] PocketBackboneGpu doc): blocks and single steps give the same
    # outputs and leave the same rings, and a decode continues from a prefilled ring.
    cfg = tiny("C", ring=9, window=6)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, 30)
    a = oracle.OracleDecoder(cfg, layers, final)
    b = oracle.OracleDecoder(cfg, layers, final)
    p = 0
    for t in (4, 4, 1, 3, 4, 2):
        ya = a.prefill(xs[p:p + t, 0], p, first=(p == 0))
        yb = np.concatenate([b.step(xs[p + r], p + r, first=(p + r == 0)) for r in range(t)])
        np.testing.assert_allclose(ya, yb, rtol=1e-5, atol=1e-6)
        p += t
    np.testing.assert_array_equal(a.P, b.P)
    np.testing.assert_allclose(a.K, b.K, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(a.V, b.V, rtol=1e-5, atol=1e-6)
    for q in range(p, 30):
        np.testing.assert_allclose(a.step(xs[q], q), b.step(xs[q], q), rtol=1e-5, atol=1e-6)


def test_prefill_argument_errors():
    cfg = tiny("C", ring=5, window=4)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, 8)
    d = oracle.OracleDecoder(cfg, layers, final)
    d.prefill(xs[:3, 0], 0, first=True)  # inside the first ring turn nothing is evicted
    with pytest.raises(ValueError, match="window"):
        d.prefill(xs[3:6, 0], 3)  # position 5 evicts 0, which row 3 (pos 3, window 4) attends
    d.prefill(xs[3:5, 0], 3)       # 5 slots >= window 4 + 1
    with pytest.raises(ValueError, match="contiguous"):
        d.prefill(xs[5:7, 0], 6)
    multi = oracle.OracleDecoder(tiny("C", m=2), *wl.make_weights(tiny("C", m=2)))
    with pytest.raises(ValueError, match="single-stream"):
        multi.prefill(xs[:1, 0], 0, first=True)


def test_ring_bookkeeping_closed_form():
    # After step p of a stream that started at p0: P[s] = max{p' <= p : p' = s mod R, p' >= p0}.
    cfg = tiny("C", ring=5, window=4)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, 40)
    orc = oracle.OracleDecoder(cfg, layers, final)
    p0 = 3
    for p in range(p0, p0 + 37):
        orc.step(xs[p - p0], p, first=(p == p0))
        for s in range(5):
            cands = [t for t in range(p0, p + 1) if t % 5 == s]
            want = max(cands) if cands else int(INVALID_POS)
            assert int(orc.P[0, s]) == want, (p, s)


def test_streams_are_independent():
    # m streams in lockstep equal m separate single-stream decoders.
    cfg = tiny("T", m=3)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg)
    multi = oracle.OracleDecoder(cfg, layers, final)
    singles = [oracle.OracleDecoder(cfg.replace(m=1), layers, final) for _ in range(3)]
    for p in range(6):
        y = multi.step(xs[p], p, first=(p == 0))
        for s in range(3):
            ys = singles[s].step(xs[p, s:s + 1], p, first=(p == 0))
            np.testing.assert_allclose(y[s], ys[0], rtol=1e-6, atol=1e-6)


def test_layerscale_zero_passes_residual_through():
    cfg = tiny("C", layer_scale_init=0.0)
    layers, final = wl.make_weights(cfg)
    x = wl.make_inputs(cfg, 1)[0]
    y = oracle.OracleDecoder(cfg, layers, final).step(x, 0, first=True)
    np.testing.assert_array_equal(y, x)
    cfg1 = tiny("C", layer_scale_init=1.0)
    cfg0 = tiny("C", layer_scale=False)
    l1, f1 = wl.make_weights(cfg1)
    l0, f0 = wl.make_weights(cfg0)
    np.testing.assert_array_equal(oracle.OracleDecoder(cfg1, l1, f1).step(x, 0, True),
                                  oracle.OracleDecoder(cfg0, l0, f0).step(x, 0, True))


def test_reset_replays_bitwise_and_resume_from_import():
    cfg = tiny("C", ring=6, window=5)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, 20)
    a = oracle.OracleDecoder(cfg, layers, final)
    first_run = [a.step(xs[p], p, p == 0) for p in range(9)]
    a.reset()
    again = [a.step(xs[p], p, p == 0) for p in range(9)]
    for u, v in zip(first_run, again):
        np.testing.assert_array_equal(u, v)
    # Resume: hand the ring contents of `a` to a fresh decoder and continue both.
    b = oracle.OracleDecoder(cfg, layers, final)
    live = [int(t) for t in a.P[0] if t != INVALID_POS]
    slots = [t % 6 for t in live]
    b.import_kv(0, a.K[0][:, slots], a.V[0][:, slots], live)
    for p in range(9, 20):
        np.testing.assert_array_equal(a.step(xs[p], p), b.step(xs[p], p))


def test_step_argument_errors():
    cfg = tiny("T", ring=4, window=4)
    layers, final = wl.make_weights(cfg)
    xs = wl.make_inputs(cfg, 6)
    d = oracle.OracleDecoder(cfg, layers, final)
    d.step(xs[0], 0, True)
    with pytest.raises(ValueError, match="contiguous"):
        d.step(xs[1], 2)
    for p in range(1, 4):
        d.step(xs[p], p)
    with pytest.raises(ValueError, match="ring"):
        d.step(xs[4], 4)  # unbounded (talker) cache refuses a position past its capacity


# ---------------------------------------------------------------------------------------------
# the pages' fixed constants
# ---------------------------------------------------------------------------------------------

def test_page_facts():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    assert int(INVALID_POS) == facts["invalid_pos"]["value"] == wl.INVALID_POS
    ctx = facts["codec_context"]["value"]
    for i in (1, 2, 3):
        c = wl.CONFIGS[i]
        assert c.window == ctx and c.ring in (ctx, ctx + 1)  # ctx + one position per call
        assert c.d_model == facts["codec_dim"]["value"]
        assert c.n_q_heads == facts["codec_heads"]["value"]
        assert c.d_ff == facts["codec_ffn"]["value"]
        assert c.norm_eps == facts["codec_ln_eps"]["value"]
        assert c.rope_theta == facts["codec_rope_theta"]["value"]
    for i in (4, 5):
        c = wl.CONFIGS[i]
        assert c.rope_theta == facts["talker_rope_theta"]["value"]
        assert c.head_dim <= facts["talker_max_head_dim"]["value"]


# ---------------------------------------------------------------------------------------------
# split RVQ ([mimi] NEAREST, SUB_EMB, EMB_SUM and the encode / decode plans)
# ---------------------------------------------------------------------------------------------

def test_rvq_distances_exact_on_small_integers():
    # |cb|, |r| <= 8 integers: every difference, square and partial sum is exact in float32.
    rng = np.random.default_rng(30)
    cb = rng.integers(-8, 9, size=(300, 64)).astype(F32)
    r = rng.integers(-8, 9, size=64).astype(F32)
    exact = ((cb.astype(np.int64) - r.astype(np.int64)) ** 2).sum(axis=1)
    np.testing.assert_array_equal(oracle.sq_distances(cb, r), exact.astype(F32))


def test_rvq_distances_sequential_order_no_fma():
    # The float32 sum runs over c in ascending order with the square rounded first: equal to an
    # explicit scalar loop, and different from a float64 sum on data where order matters.
    rng = np.random.default_rng(31)
    cb = (rng.standard_normal((40, 256)) * 100).astype(F32)
    r = rng.standard_normal(256).astype(F32)
    d = oracle.sq_distances(cb, r)
    for b in (0, 17, 39):
        acc = F32(0)
        for c in range(256):
            df = F32(cb[b, c] - r[c])
            acc = F32(acc + F32(df * df))
        assert d[b] == acc
    d64 = ((cb.astype(np.float64) - r.astype(np.float64)) ** 2).sum(axis=1)
    np.testing.assert_allclose(d, d64, rtol=1e-5)


def test_rvq_nearest_first_wins_and_brute_force():
    rng = np.random.default_rng(32)
    cb = rng.standard_normal((256, 32)).astype(F32)
    r = rng.standard_normal(32).astype(F32)
    d64 = ((cb.astype(np.float64) - r) ** 2).sum(axis=1)
    assert oracle.nearest(cb, r) == int(np.argmin(d64))
    # exact ties: duplicated rows (and an exactly equidistant pair) go to the lower bin
    cb2 = cb.copy()
    best = oracle.nearest(cb, r)
    cb2[3] = cb[best]
    cb2[200] = cb[best]
    assert oracle.nearest(cb2, r) == min(3, best)
    cbi = np.array([[2, 0], [0, 2], [-2, 0], [1, 1]], F32)  # distances 4, 4, 4, 2 from (0, 0)
    assert oracle.nearest(cbi, np.zeros(2, F32)) == 3
    assert oracle.nearest(cbi[:3], np.zeros(2, F32)) == 0


def test_rvq_emb_sum_order_and_values():
    cbs = np.zeros((3, 4, 2), F32)
    cbs[0, 1] = [1e8, 1.0]
    cbs[1, 2] = [1.0, 2.0]
    cbs[2, 3] = [-1e8, 3.0]
    acc = oracle.emb_sum(cbs, [1, 2, 3])
    # sequential: (1e8 + 1) rounds to 1e8, then - 1e8 -> 0 (a pairwise sum would give 1)
    assert acc[0] == F32(0.0) and acc[1] == F32(6.0)


def _rvq_identity(nq=4, vq=16, bins=32, seed=33):
    # identity projections (dim == vq) and well-separated codebooks: codes are recoverable
    rng = np.random.default_rng(seed)
    eye = np.eye(vq, dtype=F32)
    cb_first = (rng.standard_normal((1, bins, vq)) * 4).astype(F32)
    cb_rest = (rng.standard_normal((nq - 1, bins, vq)) * 4 / np.arange(1, nq)[:, None, None]).astype(F32)
    return oracle.OracleRVQ(eye, eye, eye, eye, cb_first, cb_rest), cb_first, cb_rest


def test_rvq_encode_recovers_planted_codes_and_decode_inverts():
    # latent = cb_rest[0][a] + cb_rest[1][b] + cb_rest[2][c] (shrinking scales) with identity
    # projections: the rest chain finds a, b, c in turn; the first codebook sees the latent itself.
    q, cb_first, cb_rest = _rvq_identity()
    planted = [5, 17, 30]
    x = (cb_rest[0, 5] + cb_rest[1, 17] + cb_rest[2, 30]).astype(F32)
    codes = q.encode(x)
    assert list(codes[1:]) == planted
    assert codes[0] == oracle.nearest(cb_first[0], x)
    y = q.decode(codes)
    want = (cb_first[0, codes[0]] + (cb_rest[0, 5] + cb_rest[1, 17] + cb_rest[2, 30]))
    np.testing.assert_allclose(y, want, rtol=1e-6, atol=1e-6)


def test_rvq_last_level_skips_the_residual_update():
    # nq = 2: one rest level; quantise never subtracts after it (changing the rest codebook's
    # rows other than the chosen one cannot change the result)
    q, _, cb_rest = _rvq_identity(nq=2)
    x = cb_rest[0, 9].copy()
    codes, margins = q.quantise(x, x)
    assert codes[1] == 9 and len(margins) == 2


def test_rvq_workload_margins_exceed_rounding():
    # Every decision of the seeded RVQ workload has a relative margin far above what rounding in
    # the projections can move a distance by, so the GPU must reproduce the codes bit for bit.
    cfg = wl.RVQ_CONFIGS[1]
    R = wl.make_rvq(cfg.replace(frames=16))
    q = oracle.OracleRVQ(R["in_first"], R["in_rest"], R["out_first"], R["out_rest"],
                         R["cb_first"], R["cb_rest"])
    for f in range(16):
        _, margins = q.quantise(*q.project(R["latents"][f]))
        for best, second in margins:
            assert (second - best) / best > 1e-6


# ---------------------------------------------------------------------------------------------
# streaming codec convolutions, offline ([mimi] CONV1D, convtr_src, ELU_IP, REPLICATE)
# ---------------------------------------------------------------------------------------------

def test_elu_closed_forms():
    v = np.array([0.0, 1.0, -1.0, -50.0, 3.5], F32)
    np.testing.assert_array_equal(oracle.elu(v)[[0, 1, 4]], v[[0, 1, 4]])
    assert oracle.elu(v)[2] == F32(math.exp(-1.0) - 1.0)
    assert oracle.elu(v)[3] == F32(-1.0)


@pytest.mark.parametrize("stride,k,groups,replicate,pre_elu", [
    (1, 7, 1, False, False), (2, 4, 1, True, False), (1, 3, 1, False, True),
    (4, 8, 1, True, True), (1, 5, 6, False, False),
])
def test_causal_conv1d_is_the_library_convolution(stride, k, groups, replicate, pre_elu):
    torch = pytest.importorskip("torch")
    torch_f = torch.nn.functional
    rng = np.random.default_rng(40 + k)
    cin, cout, T = 6, 6 if groups > 1 else 5, 24
    x = rng.standard_normal((cin, T)).astype(F32)
    w = rng.standard_normal((cout, cin // groups, k)).astype(F32)
    b = rng.standard_normal(cout).astype(F32)
    y = oracle.causal_conv1d(x, w, b, stride, replicate=replicate, pre_elu=pre_elu, groups=groups)
    xt = torch.from_numpy(x)[None].double()
    xt = torch_f.pad(xt, (k - stride, 0), mode="replicate" if replicate else "constant")
    if pre_elu:
        xt = torch_f.elu(xt)
    ref = torch_f.conv1d(xt, torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                         stride=stride, groups=groups)[0].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("stride,k,groups,pre_elu", [(4, 8, 1, False), (2, 4, 6, True),
                                                     (3, 3, 1, True), (16, 32, 6, False)])
def test_conv_transpose1d_is_the_library_convolution(stride, k, groups, pre_elu):
    torch = pytest.importorskip("torch")
    torch_f = torch.nn.functional
    rng = np.random.default_rng(50 + k)
    cin, T = 6, 5
    cout = cin if groups > 1 else 4
    x = rng.standard_normal((cin, T)).astype(F32)
    w = rng.standard_normal((cin, cout // groups, k)).astype(F32)
    b = rng.standard_normal(cout).astype(F32)
    y = oracle.conv_transpose1d_full(x, w, b, stride, pre_elu=pre_elu, groups=groups)
    xt = torch.from_numpy(x)[None].double()
    if pre_elu:
        xt = torch_f.elu(xt)
    ref = torch_f.conv_transpose1d(xt, torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                                   stride=stride, groups=groups)[0].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)
    assert oracle.streamed_conv_transpose1d(x, w, b, stride, pre_elu, groups).shape == (cout, T * stride)


def _overlap_add_frames(x, w, b, stride, frame_cols):
    # Frame-by-frame transposed convolution written from the definition with scalar float64
    # loops: input column t adds w[i, o, k] * x[i, t] to output column t*stride + k; a column is
    # emitted once no later input column can reach it (column j < (t_end) * stride after a frame
    # ending at input column t_end), the rest stays pending.  Single group, no ELU.
    c_in, T = x.shape
    _, c_out, K = w.shape
    acc = {}  # output column -> per-channel float64 sums (bias added when emitted)
    out = []
    t0 = 0
    while t0 < T:
        t1 = min(T, t0 + frame_cols)
        for t in range(t0, t1):
            for k in range(K):
                col = acc.setdefault(t * stride + k, [0.0] * c_out)
                for o in range(c_out):
                    col[o] += sum(float(w[i, o, k]) * float(x[i, t]) for i in range(c_in))
        for j in range(t0 * stride, t1 * stride):
            col = acc.pop(j, [0.0] * c_out)
            out.append([float(b[o]) + col[o] for o in range(c_out)])
        t0 = t1
    return np.array(out, np.float64).T  # [c_out, T * stride]


@pytest.mark.parametrize("stride,k,frame_cols", [(2, 4, 1), (3, 7, 2), (4, 4, 3), (2, 5, 5)])
def test_streamed_conv_transpose1d_is_frame_by_frame_overlap_add(stride, k, frame_cols):
    # The streamed result is what frame-by-frame overlap-add emits: its first T*stride columns,
    # not its last ones, and not shifted by the K - stride pending columns.
    rng = np.random.default_rng(70 + k)
    cin, cout, T = 3, 2, 6
    x = rng.standard_normal((cin, T)).astype(F32)
    w = rng.standard_normal((cin, cout, k)).astype(F32)
    b = rng.standard_normal(cout).astype(F32)
    y = oracle.streamed_conv_transpose1d(x, w, b, stride)
    ref = _overlap_add_frames(x, w, b, stride, frame_cols)
    assert y.shape == ref.shape == (cout, T * stride)
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)
    # a prefix of the input emits a prefix of the output
    y3 = oracle.streamed_conv_transpose1d(x[:, :3], w, b, stride)
    np.testing.assert_allclose(y3, y[:, :3 * stride], rtol=1e-6, atol=1e-6)


def test_streamed_conv_transpose1d_is_a_prefix_of_the_library_convolution():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    cin, cout, T, stride, k = 4, 3, 7, 5, 10
    x = rng.standard_normal((cin, T)).astype(F32)
    w = rng.standard_normal((cin, cout, k)).astype(F32)
    b = rng.standard_normal(cout).astype(F32)
    ref = torch.nn.functional.conv_transpose1d(
        torch.from_numpy(x)[None].double(), torch.from_numpy(w).double(),
        torch.from_numpy(b).double(), stride=stride)[0].numpy()
    y = oracle.streamed_conv_transpose1d(x, w, b, stride)
    np.testing.assert_allclose(y, ref[:, :T * stride], rtol=1e-6, atol=1e-6)


def test_rvq_first_and_rest_projections_are_not_interchangeable():
    # Distinct, non-identity projections on a latent twice the quantiser width: in_first = [2I | 0]
    # sees the first half doubled, in_rest = [0 | P] a permutation of the second half; out_first =
    # [2I ; 0] writes the first group's code vector doubled into the first half, out_rest = [0 ; Q]
    # the rest group's sum permuted into the second half.  Codes are planted in both halves, so
    # swapping a first projection with its rest one changes the codes or the decoded latent.
    vq, bins, nq = 16, 32, 4
    _, cb_first, cb_rest = _rvq_identity(nq=nq, vq=vq, bins=bins)
    rng = np.random.default_rng(34)
    perm = rng.permutation(vq)
    qperm = rng.permutation(vq)
    z = np.zeros((vq, vq), F32)
    in_first = np.concatenate([2 * np.eye(vq, dtype=F32), z], axis=1)
    P = np.eye(vq, dtype=F32)[perm]  # (P w)[i] = w[perm[i]]
    in_rest = np.concatenate([z, P], axis=1)
    out_first = np.concatenate([2 * np.eye(vq, dtype=F32), z], axis=0)
    Q = np.eye(vq, dtype=F32)[qperm]
    out_rest = np.concatenate([z, Q], axis=0)
    q = oracle.OracleRVQ(in_first, in_rest, out_first, out_rest, cb_first, cb_rest)
    c0, planted = 11, [5, 17, 30]
    s = ((cb_rest[0, 5] + cb_rest[1, 17]).astype(F32) + cb_rest[2, 30]).astype(F32)
    x = np.zeros(2 * vq, F32)
    x[:vq] = cb_first[0, c0] / F32(2)
    x[vq + perm] = s  # so that (P x_rest)[i] = s[i]
    codes = q.encode(x)
    assert list(codes) == [c0] + planted
    y = q.decode(codes)
    want = np.concatenate([2 * cb_first[0, c0], s[qperm]]).astype(F32)
    np.testing.assert_array_equal(y, want)


# ---- the Pocket-style codec frame ([pocket] module doc decode graph; PocketCodecGpu) ----

def _tiny_pocket():
    from streaming_ar_transformer_amd import workloads as wl
    sc = wl.SEANetConfig("seanet_tiny", 31, channels=8, ratios=(2,), frame_cols=4)
    # weights large enough that the transformer moves the signal by O(1)
    return wl.PocketFrameConfig("pocket_tiny", 32, latent_dim=3, dim=8, heads=2, ffn=16,
                                tr_layers=2, up_kernel=8, up_stride=4, context=10, frames=6,
                                seanet=sc, tr_weight_std=0.4, tr_layer_scale=0.7)


def test_pocket_frame_offline_equals_brute_stream():
    # The oracle decodes all frames offline (whole-sequence convs, the ring-buffer stack one
    # position at a time); the brute force streams one latent at a time with explicit carries,
    # a history-list transformer and scalar sums.  6 frames of 4 positions pass the 14-slot ring.
    from streaming_ar_transformer_amd import workloads as wl
    from tests.brute import BrutePocketFrame
    cfg = _tiny_pocket()
    conv, trl, sw = wl.make_pocket_frame(cfg)
    layers = wl.seanet_layers(cfg.seanet)
    got = oracle.decode_frames(conv["latents"], conv, cfg.transformer, trl, layers, sw,
                               cfg.up_stride)
    bru = BrutePocketFrame(cfg, conv, trl, layers, sw)
    frames = [bru.frame(conv["latents"][f]) for f in range(cfg.frames)]
    want = {k: np.array([c for fr in frames for c in fr[k]], np.float64).T
            for k in ("quant", "up", "tr", "pcm")}
    assert got["pcm"].shape == (1, cfg.frames * cfg.samples_per_frame) == want["pcm"].shape
    for k in ("quant", "up", "tr", "pcm"):
        np.testing.assert_allclose(got[k], want[k], rtol=2e-5, atol=2e-5, err_msg=k)
    # the transformer does move the signal (a dropped stack would not pass unnoticed)
    assert np.max(np.abs(want["tr"] - want["up"])) > 0.1
