"""Shared pieces of the GPU parity tests: metrics, cached workloads, step runners."""
import functools
import sys

import numpy as np

from streaming_ar_transformer_amd import workloads as wl

COS_MIN = 0.99999  # per-position cosine gate of the pages' equality standard
MAX_ABS = 1e-3     # per-position max |delta| bar (the pages report about 2e-4)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cos_maxabs(a, b):
    a64 = np.asarray(a, np.float64).ravel()
    b64 = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a64), np.linalg.norm(b64)
    cos = 1.0 if na == 0 and nb == 0 else float(a64 @ b64 / (na * nb))
    return cos, float(np.max(np.abs(a64 - b64))) if a64.size else 0.0


def assert_close_rows(got, want, what):
    """Every row (one stream's position) must meet the cosine and max|delta| bar."""
    got = np.asarray(got).reshape(-1, np.asarray(got).shape[-1])
    want = np.asarray(want).reshape(got.shape)
    for r in range(got.shape[0]):
        cos, mx = cos_maxabs(got[r], want[r])
        assert cos >= COS_MIN and mx <= MAX_ABS, f"{what} row {r}: cos {cos:.9f} max|d| {mx:.3e}"
    return cos_maxabs(got, want)


def _weight_key(cfg):
    """Configs that draw the same parameters share one cache entry."""
    wid = cfg.cfg_id if cfg.weight_seed is None else cfg.weight_seed
    return cfg.replace(name="", cfg_id=wid, weight_seed=None, m=1, ring=1, window=1, steps=0,
                       start_pos=0)


@functools.lru_cache(maxsize=4)
def _weights(key):
    return wl.make_weights(key)


def weights(cfg):
    return _weights(_weight_key(cfg))


@functools.lru_cache(maxsize=2)
def _device_weights(key):
    from streaming_ar_transformer_amd.device import upload_weights
    layers, final = _weights(key)
    return upload_weights(layers, final)


def device_weights(cfg):
    return _device_weights(_weight_key(cfg))
