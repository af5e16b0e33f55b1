"""Move workload arrays into device memory for the library (PyTorch as the allocator only)."""
from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_weights(layers, final, device="cuda"):
    """Device copies of every layer's parameters, keyed like ``sdec_layer_weights``.

    A packed ``in_proj`` is uploaded once and ``wq``/``wk``/``wv`` become row-block views of it,
    so the three pointers address one ``[q; k; v]`` matrix."""
    out = []
    for lw in layers:
        d = {}
        for name, arr in lw.items():
            if name in ("wq", "wk", "wv") and "in_proj" in lw:
                continue
            d[name] = to_device(arr, device)
        if "in_proj" in lw:
            qw, kw = lw["wq"].shape[0], lw["wk"].shape[0]
            d["wq"] = d["in_proj"][:qw]
            d["wk"] = d["in_proj"][qw:qw + kw]
            d["wv"] = d["in_proj"][qw + kw:]
        out.append(d)
    fin = {k: to_device(v, device) for k, v in (final or {}).items()}
    return out, fin
