"""Kernel-level parity through the one-shot C entry points (GPU)."""
import math

import numpy as np
import pytest

import oracle
from oracle import F32, INVALID_POS
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_ar_transformer_amd import sdec
    sdec.lib()
    return sdec


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,m", [(1000, 6144, 1), (4096, 2048, 1), (777, 2048, 3),
                                   (2048, 6144, 8), (1536, 512, 1), (33, 1000, 5),
                                   (1001, 1024, 1), (1023, 4096, 1)])
def test_gemv_small_integers_bit_exact(sd, n, k, m):
    # |w|, |x| <= 4 with k <= 6144 keeps every partial sum an exact integer below 2^24.
    log(f"gemv exact n={n} k={k} m={m}")
    rng = np.random.default_rng(n * 7 + k + m)
    w = rng.integers(-4, 5, size=(n, k)).astype(F32)
    x = rng.integers(-4, 5, size=(m, k)).astype(F32)
    y = torch.full((m, n), float("nan"), device="cuda")
    sd.gemv(dev(w), dev(x), y)
    exact = (x.astype(np.int64) @ w.astype(np.int64).T).astype(F32)
    np.testing.assert_array_equal(y.cpu().numpy(), exact)


@pytest.mark.parametrize("n,k,m", [(4096, 2048, 1), (2048, 6144, 1), (12288, 2048, 1),
                                   (2048, 2048, 8), (2048, 6144, 8), (1, 4, 1), (5, 260, 2),
                                   (3072, 1024, 1), (1024, 4096, 1), (1, 1024, 1)])
def test_gemv_random_within_error_bound(sd, n, k, m):
    log(f"gemv random n={n} k={k} m={m}")
    rng = np.random.default_rng(k + n + m)
    w = (rng.standard_normal((n, k)) / math.sqrt(k)).astype(F32)
    x = rng.standard_normal((m, k)).astype(F32)
    y = torch.empty((m, n), device="cuda")
    sd.gemv(dev(w), dev(x), y)
    got = y.cpu().numpy().astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    # Higham: |fl(w.x) - w.x| <= gamma_k sum |w_i x_i|, gamma_k = k u / (1 - k u), u = 2^-24.
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    bound = gamma * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    want = oracle.gemv(w, x)
    assert np.max(np.abs(got - want)) <= 1e-4


# ---------------------------------------------------------------------------------------------
# ring attention
# ---------------------------------------------------------------------------------------------

def ring_state(R, pos, start, m=1):
    """Position ring of a contiguous stream that started at `start` and has pushed `pos`."""
    P = np.full((m, R), INVALID_POS, np.uint32)
    for p in range(max(start, pos - R + 1), pos + 1):
        P[:, p % R] = p
    return P


@pytest.mark.parametrize("hd,hq,hkv,R,W", [(128, 16, 8, 2048, 2048), (64, 8, 8, 250, 250),
                                           (64, 8, 8, 251, 250), (128, 4, 1, 300, 100),
                                           (64, 2, 2, 7, 5)])
def test_attention_closed_form_mean_position(sd, hd, hq, hkv, R, W):
    # q = 0: every legal slot scores 0, so dim 0 of the output (V[s, 0] = P[s]) is the mean legal
    # position, exactly: pos - (W - 1) / 2 once the window is full.
    log(f"attention closed form hd={hd} R={R} W={W}")
    m = 2
    for pos in sorted({0, 1, W - 1, W, R - 1, R, R + 1, 2 * R + 3, 3 * R - 1}):
        P = ring_state(R, pos, 0, m)
        K = np.random.default_rng(pos).standard_normal((m, R, hkv, hd)).astype(F32)
        V = np.zeros((m, R, hkv, hd), F32)
        V[..., 0] = np.where(P == INVALID_POS, 1e9, P.astype(np.float64))[:, :, None]
        q = np.zeros((m, hq * hd), F32)
        out = torch.full((m, hq * hd), float("nan"), device="cuda")
        sd.ring_attention(dev(q), dev(K), dev(V), dev(P.view(np.int32)), out, hq, hkv, hd, R, W, pos)
        o = out.cpu().numpy().reshape(m, hq, hd)
        lo = max(0, pos - min(W, R) + 1)
        np.testing.assert_array_equal(o[:, :, 0], np.float32((lo + pos) / 2.0))
        np.testing.assert_array_equal(o[:, :, 1:], 0.0)


@pytest.mark.parametrize("hd,hq,hkv,R,W,m", [(128, 16, 8, 2048, 2048, 1), (128, 16, 8, 4352, 4352, 8),
                                             (64, 8, 8, 250, 250, 1), (64, 8, 8, 251, 250, 2),
                                             (128, 8, 2, 97, 40, 3)])
def test_attention_random_matches_oracle(sd, hd, hq, hkv, R, W, m):
    log(f"attention random hd={hd} hq={hq} hkv={hkv} R={R} W={W} m={m}")
    rng = np.random.default_rng(R + m)
    for pos in sorted({1, R // 2, R - 1, R + 17}):
        P = ring_state(R, pos, 0, m)
        K = rng.standard_normal((m, R, hkv, hd)).astype(F32)
        V = rng.standard_normal((m, R, hkv, hd)).astype(F32)
        q = (rng.standard_normal((m, hq, hd)) * 0.3).astype(F32)
        out = torch.empty((m, hq * hd), device="cuda")
        sd.ring_attention(dev(q.reshape(m, -1)), dev(K), dev(V), dev(P.view(np.int32)), out, hq,
                          hkv, hd, R, W, pos)
        got = out.cpu().numpy().reshape(m, hq, hd)
        for s in range(m):
            want = oracle.attend(q[s], K[s], V[s], P[s], pos, W, hkv, True)
            assert np.max(np.abs(got[s] - want)) <= 2e-5, (pos, s)


def test_attention_no_legal_slot_gives_zeros(sd):
    hd, hq, hkv, R = 128, 4, 2, 64
    P = np.full((1, R), INVALID_POS, np.uint32)
    P[0, :5] = [10, 11, 12, 13, 14]  # all in the future of pos 3
    K = np.ones((1, R, hkv, hd), F32)
    out = torch.full((1, hq * hd), float("nan"), device="cuda")
    sd.ring_attention(dev(np.ones((1, hq * hd), F32)), dev(K), dev(K), dev(P.view(np.int32)), out,
                      hq, hkv, hd, R, R, 3)
    assert np.all(out.cpu().numpy() == 0)
