"""CPU oracle of the streaming codec convolutions, computed offline over the whole sequence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[mimi] inferencelayer 0.2.1, ``src/mimi_gpu.rs``: the streaming SEANet pieces -- a causal
``CONV1D`` whose input prefix is carried between frames (``WRITE_XA``, ``CARRY``, ``REPLICATE``
for the first frame), and a transposed conv (``convtr_src``, gather form, optional folded
pre-ELU) whose overlap tail is carried bias-subtracted (``TRP_ADD``, ``TR_OUT``, ``TR_CARRY``);
``ELU_IP``/``ELU_TO``.  Streaming must not change the result: feeding the frames one at a time
gives, concatenated, the offline convolution of the concatenated input.  This module is that
offline result, written from the definitions.

Layouts (channel-major, as the pages' buffers): x ``[C_in, T]``; conv weights
``[C_out, C_in / groups, K]``; transposed-conv weights ``[C_in, C_out / groups, K]``;
groups is 1 or the channel count (channel-wise).
"""
from __future__ import annotations

import numpy as np

from .step import F32


def elu(v: np.ndarray) -> np.ndarray:
    """``v`` if ``v > 0`` else ``exp(v) - 1`` ([mimi] ``ELU_IP``); exp in float64, rounded once."""
    v = np.asarray(v, F32)
    return np.where(v > 0, v, (np.exp(v.astype(np.float64)) - 1.0).astype(F32)).astype(F32)


def _group_matmul(w_k: np.ndarray, x: np.ndarray, groups: int) -> np.ndarray:
    """``out[o] = sum_i w_k[o, i] * x[g(o) * ipg + i]`` for one kernel tap (float64)."""
    c_out, ipg = w_k.shape
    opg = c_out // groups
    out = np.empty((c_out, x.shape[1]), np.float64)
    for g in range(groups):
        out[g * opg:(g + 1) * opg] = w_k[g * opg:(g + 1) * opg] @ x[g * ipg:(g + 1) * ipg]
    return out


def causal_conv1d(x, w, b, stride: int, replicate: bool = False, pre_elu: bool = False,
                  groups: int = 1) -> np.ndarray:
    """Offline causal conv: the input is left-padded by ``K - stride`` columns (zeros, or copies
    of the first sample: [mimi] ``REPLICATE``), then ``y[o, t] = b[o] + sum_{i, k}
    w[o, i, k] * f(xp[i, t*stride + k])`` with f = ELU when ``pre_elu`` (applied to every read
    value, padding included).  ``T`` must be a multiple of ``stride``.  One matrix product per
    kernel tap, in float64, rounded once to float32."""
    x = np.asarray(x, F32)
    w = np.asarray(w, F32)
    c_in, T = x.shape
    c_out, ipg, K = w.shape
    assert T % stride == 0 and c_in == ipg * groups
    pad = K - stride
    first = x[:, :1] if replicate else np.zeros((c_in, 1), F32)
    xp = np.concatenate([np.repeat(first, pad, axis=1), x], axis=1)
    if pre_elu:
        xp = elu(xp)
    xp = xp.astype(np.float64)
    t_out = T // stride
    y = np.repeat(np.asarray(b, np.float64)[:, None], t_out, axis=1)
    for k in range(K):
        cols = xp[:, k:k + (t_out - 1) * stride + 1:stride]  # xp[:, t*stride + k] for every t
        y += _group_matmul(w[:, :, k].astype(np.float64), cols, groups)
    return y.astype(F32)


def conv_transpose1d_full(x, w, b, stride: int, pre_elu: bool = False,
                          groups: int = 1) -> np.ndarray:
    """Offline transposed conv, all ``(T - 1) * stride + K`` output columns:
    ``y[o, t*stride + k] += w[i, o', k] * f(x[i, t])`` over the input channels i of o's group
    (o' = o within the group), plus ``b[o]``.  One matrix product per kernel tap, in float64,
    rounded once."""
    x = np.asarray(x, F32)
    w = np.asarray(w, F32)
    if pre_elu:
        x = elu(x)
    c_in, T = x.shape
    _, opg, K = w.shape
    c_out = opg * groups
    ipg = c_in // groups
    L = (T - 1) * stride + K
    y = np.repeat(np.asarray(b, np.float64)[:, None], L, axis=1)
    x64 = x.astype(np.float64)
    for k in range(K):
        # tap k of input column t lands on output column t*stride + k
        wk = np.empty((c_out, ipg), np.float64)
        for g in range(groups):
            wk[g * opg:(g + 1) * opg] = w[g * ipg:(g + 1) * ipg, :, k].astype(np.float64).T
        y[:, k:k + (T - 1) * stride + 1:stride] += _group_matmul(wk, x64, groups)
    return y.astype(F32)


def streamed_conv_transpose1d(x, w, b, stride: int, pre_elu: bool = False,
                              groups: int = 1) -> np.ndarray:
    """What a frame-by-frame transposed conv emits in total: the first ``T * stride`` columns of
    the full output (the last ``K - stride`` are still waiting for the next frame's overlap)."""
    full = conv_transpose1d_full(x, w, b, stride, pre_elu, groups)
    return full[:, :np.asarray(x).shape[1] * stride]
