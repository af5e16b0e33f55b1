"""A Pocket-style codec decode frame assembled from the library's entry points.

Argument marshalling only: every convolution, layout change and transformer layer runs in the
library's kernels.  One latent column becomes one frame of samples ([pocket] module doc, the
decode graph; ``PocketCodecGpu::new`` and ``decode_frame``):

  1x1 conv (``sdec_conv_step``) -> channel-wise transposed conv -> ``sdec_transpose`` to
  time-major rows -> the codec transformer over the frame's ``up_stride`` positions
  (``sdec_prefill``, one block of up to 16 rows) -> ``sdec_transpose`` back -> SEANet.

The transformer's ring holds ``context + up_stride`` slots so that the frame's pushes never evict
a position its earlier rows still attend ([pocket] ``PocketCodecGpu::new``); its position
advances by ``up_stride`` per frame.
"""
from __future__ import annotations

import torch

from . import sdec
from .seanet import SEANetDecoder
from .workloads import PocketFrameConfig

MAX_BLOCK = 16  # rows per sdec_prefill call (the library's max_prefill bound)


class PocketCodecFrame:
    def __init__(self, cfg: PocketFrameConfig, conv: dict, tr_layers: list, seanet_w: dict):
        """``conv`` maps ``quant.w``/``quant.b``/``up.w``/``up.b`` to device float32 tensors,
        ``tr_layers`` is a list of per-layer dicts of device tensors keyed like
        ``sdec_layer_weights``, ``seanet_w`` maps the SEANet layers' ``<name>.w``/``<name>.b``;
        all borrowed."""
        assert cfg.seanet.channels == cfg.dim and cfg.seanet.frame_cols == cfg.up_stride
        self.cfg = cfg
        d, s = cfg.dim, cfg.up_stride
        self.quant = sdec.StreamConv(conv["quant.w"], conv["quant.b"], 1, max_t_in=1)
        self.up = sdec.StreamConv(conv["up.w"], conv["up.b"], s, transposed=True, groups=d,
                                  max_t_in=1)
        self.block = min(MAX_BLOCK, s)
        self.tr = sdec.Decoder(cfg.transformer, tr_layers, None, max_prefill=self.block)
        self.seanet = SEANetDecoder(cfg.seanet, seanet_w)
        self.z = torch.empty((d, 1), device="cuda")
        self.y_up = torch.empty((d, s), device="cuda")
        self.rows = torch.empty((s, d), device="cuda")
        self.y_ct = torch.empty((d, s), device="cuda")
        self.pos = 0

    def decode_frame(self, latent, first: bool = False, stream=None):
        """One latent ``[latent_dim, 1]`` (device) -> the frame's ``[1, samples]`` output (a
        buffer the next frame overwrites).  ``first`` starts a fresh stream at position 0."""
        if first:
            self.pos = 0
        self.quant.step(latent, self.z, first=first, stream=stream)
        self.up.step(self.z, self.y_up, first=first, stream=stream)
        sdec.transpose(self.y_up, self.rows, stream=stream)
        s = self.cfg.up_stride
        for r in range(0, s, self.block):
            n = min(self.block, s - r)
            self.tr.prefill(self.rows[r:r + n], self.pos + r, first=(first and r == 0),
                            stream=stream)
        sdec.transpose(self.rows, self.y_ct, stream=stream)
        out = self.seanet.step(self.y_ct, first=first, stream=stream)
        self.pos += s
        return out

    def close(self):
        for part in (self.quant, self.up, self.tr, self.seanet):
            part.close()

