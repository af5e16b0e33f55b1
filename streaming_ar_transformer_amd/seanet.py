"""A streaming SEANet-style codec decoder assembled from ``sdec_conv`` handles.

Argument marshalling only: every convolution, transposed convolution and ELU runs in the
library's kernels (``sdec_conv_step``); this module owns the per-layer handles and the
intermediate device buffers and calls them in order ([pocket] module doc: conv k7, then per
ratio ELU + transposed conv + residual block, then ELU + conv k3).  A residual block's second
conv accumulates into its input buffer, so the block needs no copy.
"""
from __future__ import annotations

import torch

from . import sdec
from .workloads import SEANetConfig, seanet_layers


class SEANetDecoder:
    def __init__(self, cfg: SEANetConfig, weights: dict):
        """``weights`` maps ``<layer>.w`` / ``<layer>.b`` to device float32 tensors (borrowed)."""
        self.cfg = cfg
        self.layers = []
        cols = cfg.frame_cols
        for name, kind, shape, stride in seanet_layers(cfg):
            w, b = weights[name + ".w"], weights[name + ".b"]
            if kind == "convtr":
                conv = sdec.StreamConv(w, b, stride, transposed=True, pre_elu=True, max_t_in=cols)
                cols *= stride
                out_ch = shape[1]
            else:
                conv = sdec.StreamConv(w, b, stride, pre_elu=(name != "conv_in"),
                                       accumulate=(kind == "res1"), max_t_in=cols)
                out_ch = shape[0]
            buf = None if kind == "res1" else torch.empty((out_ch, cols), device="cuda")
            self.layers.append((kind, conv, buf))

    def step(self, x, first=False, stream=None):
        """One frame: x device ``[channels, frame_cols]``; returns the ``[1, samples]`` output."""
        cur = x
        block_in = None
        for kind, conv, buf in self.layers:
            if kind == "res0":
                block_in = cur
                conv.step(cur, buf, first=first, stream=stream)
                cur = buf
            elif kind == "res1":
                conv.step(cur, block_in, first=first, stream=stream)  # block_in += conv(elu(h))
                cur = block_in
            else:
                conv.step(cur, buf, first=first, stream=stream)
                cur = buf
        return cur

    def close(self):
        for _, conv, _ in self.layers:
            conv.close()
