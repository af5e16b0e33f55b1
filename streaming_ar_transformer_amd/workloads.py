"""Seeded synthetic workloads for the streaming decode step.

This module only *describes* and *draws* inputs: layer geometry, the per-step input rows, the
weights and the optional K/V prefill.  It holds none of the step's arithmetic, so both the CPU
oracle (``oracle/``) and the HIP path can take their inputs from it without sharing any of the
method.

Shapes follow the pages' two layer families:

* the talker family (``qwen3tts_gpu.rs``, inferencelayer 0.2.8: ``GpuLayer``/``Dims`` and the
  ``build_step_plan`` pass list): RMSNorm, per-head qk-RMSNorm, rotate_half rope, GQA,
  SwiGLU, final RMSNorm;
* the codec family (``mimi_gpu.rs``, inferencelayer 0.2.1: ``LayerView``/``TrShape`` and
  ``Builder::transformer_shaped``; ``pocket_tts_gpu.rs``, inferencelayer 0.2.4: the codec
  decode plan): pre-LayerNorm, packed in_proj, interleaved rope, MHA, GELU(erf), LayerScale,
  no final norm.

Seeds: ``numpy.random.default_rng([cfg_id, role, ...])`` with role 0 = weights
(``[cfg_id, 0, layer, matrix]``; the m=8 talker reuses the m=1 talker's weights), role 1 = per-step inputs (``[cfg_id, 1, stream]``), role 2 =
K/V prefill (``[cfg_id, 2, stream, layer, 0 for K / 1 for V]``).  Every draw is float32
``standard_normal`` scaled by the stated std, so each array can be drawn on its own thread.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

INVALID_POS = 0xFFFFFFFF  # empty position-ring slot (mimi_gpu.rs, INVALID_POS)

NORM_RMS, NORM_LAYER = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
FFN_SWIGLU, FFN_GELU = 0, 1


@dataclasses.dataclass(frozen=True)
class StepConfig:
    """Geometry and options of one streaming decoder stack, plus the workload drawn for it."""

    name: str
    cfg_id: int
    family: str  # "T" (talker family) or "C" (codec family)
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    m: int  # independent streams advanced in lockstep, one row each
    norm: int
    norm_eps: float
    qk_norm: bool
    qk_norm_eps: float
    rope: int
    rope_theta: float
    ffn: int
    layer_scale: bool
    layer_scale_init: float
    final_norm: bool
    ring: int  # KV ring capacity in slots
    window: int  # causal window; == ring means unbounded
    steps: int
    start_pos: int = 0  # first decoded position (>0 when the rings are prefilled)
    weight_std: float | None = None  # fixed std, or None for 1/sqrt(k)
    bf16_round: bool = False
    weight_seed: int | None = None  # cfg_id whose weights this stack shares (None: its own)
    unbounded: bool | None = None  # refuse positions past the ring (None: the talker family does)
    eos: bool = False  # an EOS logit row [1, d_model] (+ scalar bias) reads the output row

    @property
    def is_unbounded(self) -> bool:
        return (self.family == "T") if self.unbounded is None else self.unbounded

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "StepConfig":
        return dataclasses.replace(self, **kw)


def _codec(name, cfg_id, layers, ring, window, steps):
    return StepConfig(
        name=name, cfg_id=cfg_id, family="C", n_layers=layers, d_model=512, n_q_heads=8,
        n_kv_heads=8, head_dim=64, d_ff=2048, m=1, norm=NORM_LAYER, norm_eps=1e-5,
        qk_norm=False, qk_norm_eps=0.0, rope=ROPE_INTERLEAVED, rope_theta=10000.0,
        ffn=FFN_GELU, layer_scale=True, layer_scale_init=0.01, final_norm=False, ring=ring,
        window=window, steps=steps, weight_std=0.02)


def _talker(name, cfg_id, m, ring, steps, start_pos, weight_seed=None):
    return StepConfig(
        name=name, cfg_id=cfg_id, family="T", n_layers=28, d_model=2048, n_q_heads=16,
        n_kv_heads=8, head_dim=128, d_ff=6144, m=m, norm=NORM_RMS, norm_eps=1e-6, qk_norm=True,
        qk_norm_eps=1e-6, rope=ROPE_HALF, rope_theta=1e6, ffn=FFN_SWIGLU, layer_scale=False,
        layer_scale_init=1.0, final_norm=True, ring=ring, window=ring, steps=steps,
        start_pos=start_pos, weight_std=None, bf16_round=True, weight_seed=weight_seed)


def _flowlm(name, cfg_id, ring, steps):
    # [pocket] PocketBackboneGpu::new: the codec builder's layer (LayerNorm eps 1e-5, packed
    # in_proj, interleaved rope, GELU FFN) with no LayerScale and no window (window == ring ==
    # max_positions), then the output LayerNorm and the EOS logit.  6 layers, d1024, 16 heads as
    # the page states; the FFN width (4 * d) and the rope base (the codec builder's 1e4) are
    # readings.
    return StepConfig(
        name=name, cfg_id=cfg_id, family="C", n_layers=6, d_model=1024, n_q_heads=16,
        n_kv_heads=16, head_dim=64, d_ff=4096, m=1, norm=NORM_LAYER, norm_eps=1e-5,
        qk_norm=False, qk_norm_eps=0.0, rope=ROPE_INTERLEAVED, rope_theta=10000.0,
        ffn=FFN_GELU, layer_scale=False, layer_scale_init=1.0, final_norm=True, ring=ring,
        window=ring, steps=steps, weight_std=0.02, unbounded=True, eos=True)


# The five workloads.  Ring/window readings: a ring that holds exactly the window is exact at one
# position per step; config 2 keeps the codec plan's "window + positions per call" capacity so the
# window mask, not the overwrite, is what hides the oldest slot.
CONFIGS = {
    1: _codec("codec1_d512_r250", 1, 1, 250, 250, 300),
    2: _codec("codec2_d512_r251w250", 2, 2, 251, 250, 1000),
    3: _codec("codec8_d512_r250", 3, 8, 250, 250, 2000),
    4: _talker("talker28_h2048_m1", 4, 1, 2048, 2048, 0),
    # The m=8 workload runs the same talker as config 4, so it shares config 4's weights.
    5: _talker("talker28_h2048_m8_prefill4096", 5, 8, 4352, 256, 4096, weight_seed=4),
    # Next to the five: the FlowLM backbone variant of the same step (unbounded, no LayerScale,
    # final LayerNorm and an EOS logit).
    6: _flowlm("flowlm6_d1024_r512", 6, 512, 512),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and widen back to float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _normal(seed, shape, std, mean=0.0, bf16=False):
    a = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    if mean:
        a += np.float32(mean)
    return bf16_round(a) if bf16 else a


def layer_weight_specs(cfg: StepConfig):
    """(name, shape, std, mean) of every per-layer parameter, in draw order.

    Matrices are row-major ``[n_out, k]``.  Norm gains are 1 + N(0, 0.02), LayerNorm biases
    N(0, 0.02).  LayerScale vectors are constants (``layer_scale_init``), not drawn."""
    d, f = cfg.d_model, cfg.d_ff
    ws = (lambda k: cfg.weight_std) if cfg.weight_std is not None else (lambda k: 1.0 / np.sqrt(k))
    specs = [("attn_norm_w", (d,), 0.02, 1.0)]
    if cfg.norm == NORM_LAYER:
        specs.append(("attn_norm_b", (d,), 0.02, 0.0))
    if cfg.family == "C":
        specs.append(("in_proj", (cfg.q_width + 2 * cfg.kv_width, d), ws(d), 0.0))
    else:
        specs += [("wq", (cfg.q_width, d), ws(d), 0.0), ("wk", (cfg.kv_width, d), ws(d), 0.0),
                  ("wv", (cfg.kv_width, d), ws(d), 0.0)]
    specs.append(("wo", (d, cfg.q_width), ws(cfg.q_width), 0.0))
    if cfg.qk_norm:
        specs += [("q_norm", (cfg.head_dim,), 0.02, 1.0), ("k_norm", (cfg.head_dim,), 0.02, 1.0)]
    specs.append(("ffn_norm_w", (d,), 0.02, 1.0))
    if cfg.norm == NORM_LAYER:
        specs.append(("ffn_norm_b", (d,), 0.02, 0.0))
    if cfg.ffn == FFN_SWIGLU:
        specs += [("w_gate", (f, d), ws(d), 0.0), ("w_up", (f, d), ws(d), 0.0)]
    else:
        specs.append(("w_up", (f, d), ws(d), 0.0))
    specs.append(("w_down", (d, f), ws(f), 0.0))
    return specs


def make_weights(cfg: StepConfig, threads: int = 8):
    """Draw every layer's parameters and the final norm.

    Returns ``(layers, final)``: ``layers[l]`` maps a parameter name to a float32 array; for the
    codec family ``wq``/``wk``/``wv`` are row-block views of the packed ``in_proj`` (rows
    ``[q; k; v]``).  ``final`` holds ``norm_w`` (and ``norm_b`` for LayerNorm) when the stack has
    a final norm, else it is empty."""
    specs = layer_weight_specs(cfg)
    wid = cfg.cfg_id if cfg.weight_seed is None else cfg.weight_seed
    jobs = []
    for l in range(cfg.n_layers):
        for i, (name, shape, std, mean) in enumerate(specs):
            jobs.append((l, name, [wid, 0, l, i], shape, std, mean))
    if cfg.final_norm:
        jobs.append((cfg.n_layers, "norm_w", [wid, 0, cfg.n_layers, 0], (cfg.d_model,),
                     0.02, 1.0))
        if cfg.norm == NORM_LAYER:
            jobs.append((cfg.n_layers, "norm_b", [wid, 0, cfg.n_layers, 1],
                         (cfg.d_model,), 0.02, 0.0))

    def run(job):
        l, name, seed, shape, std, mean = job
        return l, name, _normal(seed, shape, std, mean, cfg.bf16_round)

    layers = [dict() for _ in range(cfg.n_layers)]
    final = {}
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for l, name, arr in ex.map(run, jobs):
            (final if l == cfg.n_layers else layers[l])[name] = arr
    for lw in layers:
        if cfg.layer_scale:
            lw["ls1"] = np.full(cfg.d_model, cfg.layer_scale_init, dtype=np.float32)
            lw["ls2"] = np.full(cfg.d_model, cfg.layer_scale_init, dtype=np.float32)
        if "in_proj" in lw:
            qw, kw = cfg.q_width, cfg.kv_width
            lw["wq"] = lw["in_proj"][:qw]
            lw["wk"] = lw["in_proj"][qw:qw + kw]
            lw["wv"] = lw["in_proj"][qw + kw:]
    return layers, final


def make_eos(cfg: StepConfig):
    """The EOS logit row ``[1, d_model]`` (std 0.02) and its scalar bias (N(0, 1)), seeded
    ``[cfg_id, 3]``; the bias is applied on the host ([pocket] PocketBackboneGpu: ``eos_bias``)."""
    w = _normal([cfg.cfg_id, 3, 0], (1, cfg.d_model), 0.02)
    b = float(_normal([cfg.cfg_id, 3, 1], (1,), 1.0)[0])
    return w, b


def make_inputs(cfg: StepConfig, steps: int | None = None) -> np.ndarray:
    """Per-step input rows, ``[steps, m, d_model]`` float32, N(0, 1), one seed per stream."""
    steps = cfg.steps if steps is None else steps
    out = np.empty((steps, cfg.m, cfg.d_model), dtype=np.float32)
    for s in range(cfg.m):
        out[:, s, :] = np.random.default_rng([cfg.cfg_id, 1, s]).standard_normal(
            (steps, cfg.d_model), dtype=np.float32)
    return out


def make_prefill(cfg: StepConfig, n_pos: int | None = None, streams=None, threads: int = 8):
    """K/V prefill rows for positions ``0 .. n_pos-1``: N(0, 1), neither normed nor roped.

    Returns ``{stream: (K, V)}`` with ``K, V`` of shape ``[n_layers, n_pos, n_kv_heads,
    head_dim]`` (the slot-major ``[positions][heads][head_dim]`` cache layout)."""
    n_pos = cfg.start_pos if n_pos is None else n_pos
    streams = range(cfg.m) if streams is None else streams
    shape = (n_pos, cfg.n_kv_heads, cfg.head_dim)
    jobs = [(s, l, kv) for s in streams for l in range(cfg.n_layers) for kv in (0, 1)]
    out = {s: (np.empty((cfg.n_layers,) + shape, np.float32),
               np.empty((cfg.n_layers,) + shape, np.float32)) for s in streams}

    def run(job):
        s, l, kv = job
        out[s][kv][l] = np.random.default_rng([cfg.cfg_id, 2, s, l, kv]).standard_normal(
            shape, dtype=np.float32)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, jobs))
    return out


def small_config(family: str = "T", **kw) -> StepConfig:
    """A reduced geometry of either family for fast tests (several tiles, ragged where asked)."""
    base = CONFIGS[4] if family == "T" else CONFIGS[1]
    base = base.replace(name=f"small_{family}", cfg_id=100 + (1 if family == "T" else 0))
    return base.replace(**kw)


@dataclasses.dataclass(frozen=True)
class RVQConfig:
    """Split RVQ geometry ([mimi] ``MimiGpu``: latent DIM 512, VQ_DIM 256, 2048-bin codebooks, one
    first codebook and NQ - 1 rest codebooks) and the frames drawn for it."""

    name: str
    seed: int
    dim: int = 512
    vq: int = 256
    bins: int = 2048
    nq: int = 8
    frames: int = 64

    def replace(self, **kw) -> "RVQConfig":
        return dataclasses.replace(self, **kw)


RVQ_CONFIGS = {1: RVQConfig("rvq8_d512_v256_b2048", 7)}


def make_rvq(cfg: RVQConfig):
    """Projections N(0, 1/sqrt(k)), codebooks N(0, 1), latent frames N(0, 1), seeded
    ``[seed, 4, part]``.  Returns a dict of float32 arrays."""
    d, v, b, nq = cfg.dim, cfg.vq, cfg.bins, cfg.nq
    s = cfg.seed
    return {
        "in_first": _normal([s, 4, 0], (v, d), 1.0 / np.sqrt(d)),
        "in_rest": _normal([s, 4, 1], (v, d), 1.0 / np.sqrt(d)),
        "out_first": _normal([s, 4, 2], (d, v), 1.0 / np.sqrt(v)),
        "out_rest": _normal([s, 4, 3], (d, v), 1.0 / np.sqrt(v)),
        "cb_first": _normal([s, 4, 4], (1, b, v), 1.0),
        "cb_rest": _normal([s, 4, 5], (nq - 1, b, v), 1.0),
        "latents": _normal([s, 4, 6], (cfg.frames, d), 1.0),
    }


@dataclasses.dataclass(frozen=True)
class SEANetConfig:
    """A streaming SEANet-style codec decoder ([pocket] module doc: conv k7, then per ratio ELU,
    transposed conv and a residual block, then ELU and conv k3; 16 input columns per 80 ms frame
    become 16 * 6 * 5 * 4 = 1920 samples).  Channels halve at each transposed conv (kernel
    2 * ratio); a residual block is ELU, conv k3 to half the channels, ELU, conv k1 back, plus
    the block's input.  The channel counts are readings."""

    name: str
    seed: int
    channels: int = 512
    ratios: tuple = (6, 5, 4)
    frame_cols: int = 16
    frames: int = 4

    def replace(self, **kw) -> "SEANetConfig":
        return dataclasses.replace(self, **kw)


SEANET_CONFIGS = {1: SEANetConfig("seanet_c512_r654", 11)}


def seanet_layers(cfg: SEANetConfig):
    """(name, kind, weight shape, stride) in execution order: kind "conv" (weights [out][in][k]),
    "convtr" ([in][out][k]), "res0"/"res1" (the residual block's two convs)."""
    c = cfg.channels
    out = [("conv_in", "conv", (c, c, 7), 1)]
    for s, r in enumerate(cfg.ratios):
        d = c // 2
        out += [(f"up{s}", "convtr", (c, d, 2 * r), r),
                (f"res{s}_0", "res0", (d // 2, d, 3), 1),
                (f"res{s}_1", "res1", (d, d // 2, 1), 1)]
        c = d
    out.append(("conv_out", "conv", (1, c, 3), 1))
    return out


def make_seanet(cfg: SEANetConfig):
    """Weights N(0, 1/fan_in) per layer (``[seed, 5, layer, 0]``), biases N(0, 0.1)
    (``[seed, 5, layer, 1]``), input frames N(0, 1) ``[frames][channels][frame_cols]``."""
    w = {}
    for i, (name, kind, shape, _) in enumerate(seanet_layers(cfg)):
        fan = shape[0] * shape[2] if kind == "convtr" else shape[1] * shape[2]
        w[name + ".w"] = _normal([cfg.seed, 5, i, 0], shape, 1.0 / np.sqrt(fan))
        n_out = shape[1] if kind == "convtr" else shape[0]
        w[name + ".b"] = _normal([cfg.seed, 5, i, 1], (n_out,), 0.1)
    x = _normal([cfg.seed, 5, 999, 0], (cfg.frames, cfg.channels, cfg.frame_cols), 1.0)
    return w, x



@dataclasses.dataclass(frozen=True)
class PocketFrameConfig:
    """A Pocket-style codec decode frame ([pocket] module doc, the decode graph, and
    ``PocketCodecGpu::new``): one latent column ``[latent_dim, 1]`` -> 1x1 conv to ``dim``
    channels -> channel-wise transposed conv (kernel ``up_kernel``, stride ``up_stride``) giving
    ``up_stride`` positions -> time-major -> the codec transformer over those positions (window
    ``context``, ring ``context + up_stride``) -> channel-major -> SEANet.  The transformer's
    rope/ring position advances by ``up_stride`` per frame."""

    name: str
    seed: int
    latent_dim: int = 32
    dim: int = 512
    heads: int = 8
    ffn: int = 2048
    tr_layers: int = 2
    up_kernel: int = 32
    up_stride: int = 16
    context: int = 250
    frames: int = 20
    seanet: SEANetConfig = SEANET_CONFIGS[1]
    tr_weight_std: float = 0.02
    tr_layer_scale: float = 0.01

    def replace(self, **kw) -> "PocketFrameConfig":
        return dataclasses.replace(self, **kw)

    @property
    def transformer(self) -> StepConfig:
        """The codec-family stack of the frame (LayerNorm eps 1e-5, interleaved rope, GELU FFN,
        LayerScale, no final norm), its weights seeded with ``cfg_id = seed``."""
        return _codec(f"{self.name}_tr", self.seed, self.tr_layers, self.context + self.up_stride,
                      self.context, self.frames * self.up_stride).replace(
            d_model=self.dim, n_q_heads=self.heads, n_kv_heads=self.heads,
            head_dim=self.dim // self.heads, d_ff=self.ffn, weight_std=self.tr_weight_std,
            layer_scale_init=self.tr_layer_scale)

    @property
    def samples_per_frame(self) -> int:
        return self.up_stride * int(np.prod(self.seanet.ratios))


POCKET_CONFIGS = {1: PocketFrameConfig("pocket_frame_l32_d512_tr2_r654", 21)}


def make_pocket_frame(cfg: PocketFrameConfig):
    """The frame's parameters and inputs.  Returns ``(conv, tr_layers, seanet_w)``: ``conv`` holds
    ``quant.w`` ``[dim, latent_dim, 1]`` (std 1/sqrt(latent_dim)), ``up.w`` ``[dim, 1, up_kernel]``
    (std sqrt(up_stride / up_kernel): each output column sums up_kernel / up_stride taps), their
    biases N(0, 0.1) and the latents ``[frames, latent_dim, 1]`` N(0, 1), seeded
    ``[seed, 6, part]``; ``tr_layers`` come from ``make_weights(cfg.transformer)`` and
    ``seanet_w`` from ``make_seanet(cfg.seanet)``."""
    s, d = cfg.seed, cfg.dim
    conv = {
        "quant.w": _normal([s, 6, 0], (d, cfg.latent_dim, 1), 1.0 / np.sqrt(cfg.latent_dim)),
        "quant.b": _normal([s, 6, 1], (d,), 0.1),
        "up.w": _normal([s, 6, 2], (d, 1, cfg.up_kernel), np.sqrt(cfg.up_stride / cfg.up_kernel)),
        "up.b": _normal([s, 6, 3], (d,), 0.1),
        "latents": _normal([s, 6, 4], (cfg.frames, cfg.latent_dim, 1), 1.0),
    }
    tr_layers, _ = make_weights(cfg.transformer)
    seanet_w, _ = make_seanet(cfg.seanet)
    return conv, tr_layers, seanet_w
