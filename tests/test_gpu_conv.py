"""Streaming codec convolutions on the GPU against the offline oracle ([mimi] CONV1D with its
carried prefix, convtr_src with its bias-subtracted overlap tail, ELU folded into the reads).

Frames of assorted sizes go through ``sdec_conv_step`` one at a time; the concatenated outputs
must equal the offline convolution of the concatenated input (max|delta| <= 1e-4 on unit-scale
outputs), including a restart with ``first`` mid-stream and an accumulating conv.
"""
import numpy as np
import pytest

import oracle
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


CASES = [
    dict(tr=False, cin=64, cout=48, k=7, s=1),
    dict(tr=False, cin=32, cout=32, k=4, s=2, replicate=True),
    dict(tr=False, cin=40, cout=24, k=3, s=1, pre_elu=True),
    dict(tr=False, cin=24, cout=16, k=1, s=1),
    dict(tr=False, cin=32, cout=32, k=5, s=1, groups=32, replicate=True, pre_elu=True),
    dict(tr=True, cin=48, cout=32, k=8, s=4),
    dict(tr=True, cin=64, cout=64, k=32, s=16, groups=64),
    dict(tr=True, cin=32, cout=16, k=10, s=5, pre_elu=True),
    dict(tr=True, cin=16, cout=8, k=3, s=3),
]


def make_case(c, seed):
    rng = np.random.default_rng(seed)
    groups = c.get("groups", 1)
    fan = (c["cin"] // groups) * c["k"]
    if c["tr"]:
        w = rng.standard_normal((c["cin"], c["cout"] // groups, c["k"])).astype(np.float32)
    else:
        w = rng.standard_normal((c["cout"], c["cin"] // groups, c["k"])).astype(np.float32)
    w /= np.float32(np.sqrt(fan))
    b = rng.standard_normal(c["cout"]).astype(np.float32)
    return w, b, groups


def offline(c, x, w, b, groups):
    if c["tr"]:
        return oracle.streamed_conv_transpose1d(x, w, b, c["s"], c.get("pre_elu", False), groups)
    return oracle.causal_conv1d(x, w, b, c["s"], c.get("replicate", False),
                                c.get("pre_elu", False), groups)


def run_stream(sd, conv, c, x, sizes, first=True):
    outs = []
    p = 0
    for i, n in enumerate(sizes):
        xf = torch.from_numpy(np.ascontiguousarray(x[:, p:p + n])).cuda()
        yf = torch.empty((c["cout"], conv.out_cols(n)), device="cuda")
        conv.step(xf, yf, first=(first and i == 0))
        outs.append(yf.cpu().numpy())
        p += n
    return np.concatenate(outs, axis=1)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_streaming_equals_offline(sd, ci):
    c = CASES[ci]
    w, b, groups = make_case(c, 60 + ci)
    unit = 1 if c["tr"] else c["s"]
    sizes = [u * unit for u in (4, 1, 8, 2, 5, 3, 1, 6)]
    x = np.random.default_rng(70 + ci).standard_normal((c["cin"], sum(sizes))).astype(np.float32)
    wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    conv = sd.StreamConv(wd, bd, c["s"], transposed=c["tr"], groups=groups,
                         pre_elu=c.get("pre_elu", False), replicate_first=c.get("replicate", False),
                         max_t_in=64)
    print(f"conv case {ci}: {c}", flush=True)
    got = run_stream(sd, conv, c, x, sizes)
    want = offline(c, x, w, b, groups)
    assert got.shape == want.shape
    mx = float(np.max(np.abs(got - want)))
    assert mx <= 1e-4, f"case {ci}: max|d| {mx:.3e}"
    # a restart with `first` mid-stream behaves like a fresh stream
    got2 = run_stream(sd, conv, c, x[:, :sum(sizes[:3])], sizes[:3])
    np.testing.assert_allclose(got2, offline(c, x[:, :sum(sizes[:3])], w, b, groups), atol=1e-4)
    conv.close()
    log(f"conv case {ci} {'convtr' if c['tr'] else 'conv'} k{c['k']} s{c['s']}: max|d| {mx:.2e}")


def test_accumulating_conv_and_errors(sd):
    c = dict(tr=False, cin=16, cout=16, k=3, s=1)
    w, b, _ = make_case(c, 80)
    x = np.random.default_rng(81).standard_normal((16, 12)).astype(np.float32)
    z = np.random.default_rng(82).standard_normal((16, 12)).astype(np.float32)
    conv = sd.StreamConv(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), 1,
                         pre_elu=True, accumulate=True, max_t_in=16)
    y = torch.from_numpy(z).cuda()
    conv.step(torch.from_numpy(x).cuda(), y, first=True)
    want = z + oracle.causal_conv1d(x, w, b, 1, pre_elu=True)
    np.testing.assert_allclose(y.cpu().numpy(), want, atol=1e-4)
    with pytest.raises(sd.SdecError) as e:
        conv.step(torch.zeros((16, 20), device="cuda"), y)  # more columns than max_t_in
    assert e.value.code == sd.E_ARG
    conv.close()
    c2 = sd.StreamConv(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), 1, max_t_in=16)
    with pytest.raises(sd.SdecError) as e:
        c2.step(torch.zeros((16, 4), device="cuda"), y)  # a stream must start with first
    assert e.value.code == sd.E_POS
    c2.close()


def offline_seanet(cfg, w, X):
    from streaming_ar_transformer_amd import workloads as wl
    h = None
    for name, kind, shape, stride in wl.seanet_layers(cfg):
        W, B = w[name + ".w"], w[name + ".b"]
        if kind == "conv":
            h = oracle.causal_conv1d(X if h is None else h, W, B, stride,
                                     pre_elu=(name != "conv_in"))
        elif kind == "convtr":
            h = oracle.streamed_conv_transpose1d(h, W, B, stride, pre_elu=True)
        elif kind == "res0":
            block_in, h = h, oracle.causal_conv1d(h, W, B, 1, pre_elu=True)
        else:
            h = (block_in + oracle.causal_conv1d(h, W, B, 1, pre_elu=True)).astype(np.float32)
    return h


def test_seanet_decoder_streaming_equals_offline(sd):
    # conv k7 -> (ELU, convtr, residual block) x [6, 5, 4] -> ELU, conv k3: 16 columns per frame
    # become 1920 samples; frame by frame through the library == offline over all frames
    from streaming_ar_transformer_amd import workloads as wl
    from streaming_ar_transformer_amd.seanet import SEANetDecoder
    from tests.gpu_helpers import assert_close_rows
    cfg = wl.SEANET_CONFIGS[1]
    w, x = wl.make_seanet(cfg)
    dev = {k: torch.from_numpy(v).cuda() for k, v in w.items()}
    dec = SEANetDecoder(cfg, dev)
    outs = []
    for f in range(cfg.frames):
        print(f"seanet frame {f}", flush=True)
        y = dec.step(torch.from_numpy(x[f]).cuda(), first=(f == 0))
        outs.append(y.cpu().numpy())
    got = np.concatenate(outs, axis=1)
    want = offline_seanet(cfg, w, np.concatenate(list(x), axis=1))
    assert got.shape == want.shape == (1, cfg.frames * 1920)
    cos, mx = assert_close_rows(got, want, "seanet")
    dec.close()
    log(f"{cfg.name}: {cfg.frames} frames x 1920 samples, cos {cos:.9f} max|d| {mx:.2e}")
