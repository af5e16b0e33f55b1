"""Split RVQ on the GPU against the CPU oracle ([mimi] NEAREST, SUB_EMB, EMB_SUM).

Codes are integers decided by float32 distances that both sides compute in the same order and
precision, so from the same projected residuals the codes must match bit for bit (and ties must
go to the lower bin).  From the latent frames, the GPU's projection rounds differently from the
oracle's; every decision of the seeded workload has a margin far above that (asserted on the CPU
in the oracle pins), so the codes must still match exactly.  Decoded latents meet the step bar
(cos >= 0.99999, max|delta| <= 1e-3).
"""
import numpy as np
import pytest

import oracle
from streaming_ar_transformer_amd import workloads as wl
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


@pytest.fixture(scope="module")
def setup(sd):
    cfg = wl.RVQ_CONFIGS[1]
    R = wl.make_rvq(cfg)
    orc = oracle.OracleRVQ(R["in_first"], R["in_rest"], R["out_first"], R["out_rest"],
                           R["cb_first"], R["cb_rest"])
    proj = [orc.project(R["latents"][f]) for f in range(cfg.frames)]
    want = np.stack([orc.quantise(*p)[0] for p in proj])
    return cfg, R, orc, proj, want


def device(R):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in R.items()
            if k != "latents"}


def test_rvq_quantise_bit_exact(sd, setup):
    cfg, R, orc, proj, want = setup
    q = sd.RVQ(cfg.dim, cfg.vq, cfg.bins, cfg.nq, cfg.frames, device(R))
    rf = torch.from_numpy(np.stack([p[0] for p in proj])).cuda()
    rr = torch.from_numpy(np.stack([p[1] for p in proj])).cuda()
    codes = torch.full((cfg.frames, cfg.nq), -1, dtype=torch.int32, device="cuda")
    print(f"rvq quantise {cfg.name} frames {cfg.frames}", flush=True)
    q.quantise(rf, rr, codes)
    np.testing.assert_array_equal(codes.cpu().numpy().astype(np.uint32), want)
    # a single frame, and a smaller batch, give the same codes
    q.quantise(rf[5:6].contiguous(), rr[5:6].contiguous(), codes[:1])
    np.testing.assert_array_equal(codes[:1].cpu().numpy().astype(np.uint32), want[5:6])
    q.close()


def test_rvq_encode_and_decode(sd, setup):
    cfg, R, orc, proj, want = setup
    q = sd.RVQ(cfg.dim, cfg.vq, cfg.bins, cfg.nq, cfg.frames, device(R))
    lat = torch.from_numpy(R["latents"]).cuda()
    codes = torch.full((cfg.frames, cfg.nq), -1, dtype=torch.int32, device="cuda")
    print(f"rvq encode {cfg.name} frames {cfg.frames}", flush=True)
    q.encode(lat, codes)
    got = codes.cpu().numpy().astype(np.uint32)
    np.testing.assert_array_equal(got, want)
    out = torch.empty((cfg.frames, cfg.dim), device="cuda")
    q.decode(codes, out)
    ref = np.stack([orc.decode(want[f]) for f in range(cfg.frames)])
    cos, mx = assert_close_rows(out.cpu().numpy(), ref, "rvq decode")
    q.close()
    log(f"{cfg.name}: {cfg.frames} frames, codes bit-exact, decode cos {cos:.9f} max|d| {mx:.2e}")


def test_rvq_ties_go_to_the_lower_bin(sd, setup):
    cfg, R, orc, proj, want = setup
    # plant exact ties: bin 1 of the first rest codebook copies frame 0's chosen code vector, and
    # bin 0 of the first codebook copies frame 1's chosen first code (each chosen bin > the copy)
    R2 = {k: v.copy() for k, v in R.items()}
    c1, c0 = int(want[0, 1]), int(want[1, 0])
    assert c1 > 1 and c0 > 0
    R2["cb_rest"][0, 1] = R2["cb_rest"][0, c1]
    R2["cb_first"][0, 0] = R2["cb_first"][0, c0]
    orc2 = oracle.OracleRVQ(R2["in_first"], R2["in_rest"], R2["out_first"], R2["out_rest"],
                            R2["cb_first"], R2["cb_rest"])
    want2 = np.stack([orc2.quantise(*p)[0] for p in proj])
    assert want2[0, 1] == 1 and want2[1, 0] == 0
    q = sd.RVQ(cfg.dim, cfg.vq, cfg.bins, cfg.nq, cfg.frames, device(R2))
    rf = torch.from_numpy(np.stack([p[0] for p in proj])).cuda()
    rr = torch.from_numpy(np.stack([p[1] for p in proj])).cuda()
    codes = torch.empty((cfg.frames, cfg.nq), dtype=torch.int32, device="cuda")
    q.quantise(rf, rr, codes)
    np.testing.assert_array_equal(codes.cpu().numpy().astype(np.uint32), want2)
    with pytest.raises(sd.SdecError) as e:
        q.quantise(rf[:0], rr[:0], codes)  # zero frames
    assert e.value.code == sd.E_ARG
    big = torch.zeros((cfg.frames + 1, cfg.dim), device="cuda")
    with pytest.raises(sd.SdecError) as e:
        q.encode(big, torch.empty((cfg.frames + 1, cfg.nq), dtype=torch.int32, device="cuda"))
    assert e.value.code == sd.E_ARG
    q.close()
