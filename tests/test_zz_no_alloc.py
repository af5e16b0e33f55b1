"""The one-shot ring attention that allocates nothing (GPU).

``sdec_ring_attention_static`` runs the same kernels as ``sdec_ring_attention`` with its scratch in
a fixed device array instead of library-allocated buffers.  Two calls in a row -- the second with
a smaller input -- must give what the allocating entry point gives on the same inputs (and the
oracle's attention within the kernel tolerance); a call whose scratch would not fit is refused on
the host.
"""
import numpy as np
import pytest

import oracle
from oracle import F32, INVALID_POS
from tests.gpu_helpers import assert_close_rows, log

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


def ring_state(R, pos, m):
    P = np.full((m, R), INVALID_POS, np.uint32)
    for p in range(max(0, pos - R + 1), pos + 1):
        P[:, p % R] = p
    return P


# (m, hq, hkv, hd, R, W, pos): the first call spans several chunks and wraps a windowed ring; the
# second is smaller in every dimension
CASES = [(3, 8, 4, 128, 600, 520, 1000), (1, 4, 2, 64, 100, 100, 50)]


def test_static_scratch_matches_the_allocating_entry_point(sd):
    for (m, hq, hkv, hd, R, W, pos) in CASES:
        log(f"static attention m={m} hq={hq} hkv={hkv} hd={hd} R={R} W={W} pos={pos}")
        rng = np.random.default_rng(R + m)
        P = ring_state(R, pos, m)
        K = rng.standard_normal((m, R, hkv, hd)).astype(F32)
        V = rng.standard_normal((m, R, hkv, hd)).astype(F32)
        q = (rng.standard_normal((m, hq, hd)) * 0.3).astype(F32)
        args = (dev(q.reshape(m, -1)), dev(K), dev(V), dev(P.view(np.int32)))
        ref = torch.full((m, hq * hd), float("nan"), device="cuda")
        got = torch.full((m, hq * hd), float("nan"), device="cuda")
        sd.ring_attention(*args, ref, hq, hkv, hd, R, W, pos)
        sd.ring_attention_static(*args, got, hq, hkv, hd, R, W, pos)
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        assert_close_rows(g, r, f"static vs allocating m={m} R={R}")
        np.testing.assert_array_equal(g, r)  # the same kernels over the same inputs
        for s in range(m):
            want = oracle.attend(q[s], K[s], V[s], P[s], pos, W, hkv, True)
            assert np.max(np.abs(g[s].reshape(hq, hd) - want)) <= 2e-5, s


def test_static_scratch_refuses_inputs_past_its_size(sd):
    q = torch.zeros((8, 16 * 128), device="cuda")
    ring = torch.zeros(16, device="cuda")
    pr = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = torch.zeros((8, 16 * 128), device="cuda")
    with pytest.raises(sd.SdecError) as e:
        # 8 streams x 16 heads over 100000 slots: about 52 MB of chunk partials
        sd.ring_attention_static(q, ring, ring, pr, out, 16, 8, 128, 100000, 100000, 5)
    assert e.value.code == sd.E_ARG and "static scratch" in str(e.value)
