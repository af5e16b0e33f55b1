"""CPU oracle of a Pocket-style codec decode frame, computed offline over all frames at once.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[pocket] inferencelayer 0.2.4, ``src/pocket_tts_gpu.rs``: the module doc's decode graph and
``PocketCodecGpu::new`` / ``decode_frame``.  One latent column becomes one frame of samples:

  latent ``[latent_dim, 1]`` -> 1x1 conv to ``dim`` channels -> channel-wise transposed conv
  (kernel 2 * stride here, groups = dim) -> ``stride`` columns -> time-major rows -> the codec
  transformer at positions ``frame * stride + r`` (window ``context``, ring ``context + stride``)
  -> channel-major -> SEANet (conv k7; per ratio ELU, transposed conv, residual block; ELU,
  conv k3).

Streaming changes nothing: every stage is causal, so the frames decoded one after another give,
concatenated, the offline result over the concatenated latents.  This module is that offline
result, built from the pinned pieces in ``conv.py`` and ``step.py``.
"""
from __future__ import annotations

import numpy as np

from .conv import causal_conv1d, streamed_conv_transpose1d
from .step import F32, OracleDecoder


def seanet_decode(x: np.ndarray, layers, w: dict) -> np.ndarray:
    """Offline SEANet-style decoder over channel-major ``x`` ``[channels, T]``.

    ``layers`` lists ``(name, kind, weight shape, stride)`` in execution order: "conv" (ELU on
    its input unless it is the first layer), "convtr" (ELU on its input, the streamed part of
    the transposed conv), "res0"/"res1" (a residual block: ELU, conv; ELU, conv; plus the
    block's input).  ``w`` maps ``<name>.w`` / ``<name>.b`` to float32 arrays."""
    h = np.asarray(x, F32)
    block_in = None
    for i, (name, kind, _, stride) in enumerate(layers):
        W, B = w[name + ".w"], w[name + ".b"]
        if kind == "conv":
            h = causal_conv1d(h, W, B, stride, pre_elu=(i != 0))
        elif kind == "convtr":
            h = streamed_conv_transpose1d(h, W, B, stride, pre_elu=True)
        elif kind == "res0":
            block_in, h = h, causal_conv1d(h, W, B, stride, pre_elu=True)
        elif kind == "res1":
            h = (block_in + causal_conv1d(h, W, B, stride, pre_elu=True)).astype(F32)
        else:
            raise ValueError(f"unknown layer kind {kind}")
    return h


def decode_frames(latents: np.ndarray, conv: dict, tr_cfg, tr_layers, seanet_layers,
                  seanet_w: dict, stride: int) -> dict:
    """Every stage of the decode of ``latents`` ``[frames, latent_dim, 1]``.

    Returns ``quant`` ``[dim, frames]``, ``up`` ``[dim, frames * stride]`` (channel-major),
    ``tr`` ``[dim, frames * stride]`` (the transformer's output rows, back in channel-major) and
    ``pcm`` ``[1, frames * samples_per_frame]``."""
    lat = np.asarray(latents, F32)
    X = np.concatenate(list(lat), axis=1)  # [latent_dim, frames]
    z = causal_conv1d(X, conv["quant.w"], conv["quant.b"], 1)
    dim = z.shape[0]
    u = streamed_conv_transpose1d(z, conv["up.w"], conv["up.b"], stride, groups=dim)
    dec = OracleDecoder(tr_cfg, tr_layers, {})
    rows = np.ascontiguousarray(u.T)  # time-major: one row per position
    out = np.empty_like(rows)
    for t in range(rows.shape[0]):
        out[t] = dec.step(rows[t][None, :], t, first=(t == 0))[0]
    tr = np.ascontiguousarray(out.T)
    pcm = seanet_decode(tr, seanet_layers, seanet_w)
    return {"quant": z, "up": u, "tr": tr, "pcm": pcm}
