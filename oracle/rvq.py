"""CPU oracle of split residual vector quantisation (RVQ encode and decode), plain NumPy float32.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``, ``__graft_entry__`` and
``bench.py``'s CPU leg may use it; the HIP path never does.

[mimi] inferencelayer 0.2.1, ``src/mimi_gpu.rs``: the ``NEAREST``, ``SUB_EMB`` and ``EMB_SUM``
kernels and the encode / decode plans of ``MimiGpu``.  Split RVQ: the latent frame is projected
twice (``rvq_first.in_proj``, ``rvq_rest.in_proj``); the first codebook quantises the first
projection on its own, the remaining codebooks quantise the second one in turn, each subtracting
its chosen code vector from the running residual before the next.  Decoding sums the chosen code
vectors of each group and projects both sums back (``out_proj``), adding the two projections.

A code is an integer decided by float32 arithmetic, so this oracle fixes the arithmetic of that
decision: the squared distance of bin b is ``sum over c in ascending order of (cb[b,c] - r[c])^2``
with the difference and the square each rounded to float32 before the add (no fused
multiply-add), and the smallest distance wins with ties going to the lower bin ([mimi]
``NEAREST``: first-wins argmin, the CPU's in-order strict ``<``).
"""
from __future__ import annotations

import numpy as np

from .step import F32, gemv


def sq_distances(cb: np.ndarray, r: np.ndarray) -> np.ndarray:
    """``d[b] = sum_c (cb[b, c] - r[c])^2`` for every bin b, in float32, summed over c in
    ascending order, each difference and square rounded before the add ([mimi] ``NEAREST``)."""
    cb = np.asarray(cb, F32)
    r = np.asarray(r, F32)
    d = np.zeros(cb.shape[0], F32)
    for c in range(cb.shape[1]):
        df = (cb[:, c] - r[c]).astype(F32)
        d = (d + (df * df).astype(F32)).astype(F32)
    return d


def nearest(cb: np.ndarray, r: np.ndarray) -> int:
    """First-wins argmin of the squared distance: the lowest bin among the minimal ones
    ([mimi] ``NEAREST``; ``numpy.argmin`` returns the first minimal index)."""
    return int(np.argmin(sq_distances(cb, r)))


def emb_sum(cbs: np.ndarray, codes) -> np.ndarray:
    """``acc[c] = sum over l in ascending order of cbs[l, codes[l], c]`` in float32, starting
    from 0 ([mimi] ``EMB_SUM``)."""
    cbs = np.asarray(cbs, F32)
    acc = np.zeros(cbs.shape[2], F32)
    for l, code in enumerate(codes):
        acc = (acc + cbs[l, int(code)]).astype(F32)
    return acc


class OracleRVQ:
    """Split RVQ of one codec: ``in_first``/``in_rest`` ``[vq, dim]``, ``out_first``/``out_rest``
    ``[dim, vq]`` (row-major ``[n_out, k]``), codebooks ``cb_first [1, bins, vq]`` and
    ``cb_rest [nq - 1, bins, vq]``."""

    def __init__(self, in_first, in_rest, out_first, out_rest, cb_first, cb_rest):
        self.in_first = np.asarray(in_first, F32)
        self.in_rest = np.asarray(in_rest, F32)
        self.out_first = np.asarray(out_first, F32)
        self.out_rest = np.asarray(out_rest, F32)
        self.cb_first = np.asarray(cb_first, F32)
        self.cb_rest = np.asarray(cb_rest, F32)
        self.nq = 1 + self.cb_rest.shape[0]

    def project(self, latent: np.ndarray):
        """The two residuals the quantisers start from (the encode plan's two MATVECs)."""
        x = np.asarray(latent, F32).reshape(1, -1)
        return gemv(self.in_first, x)[0], gemv(self.in_rest, x)[0]

    def quantise(self, r_first: np.ndarray, r_rest: np.ndarray):
        """Codes from the two projected residuals, with each level's best and runner-up
        distances (the decision margins).  The last rest level's residual update is skipped, as
        in the encode plan (nothing reads it)."""
        codes = [nearest(self.cb_first[0], r_first)]
        margins = [_margin(sq_distances(self.cb_first[0], r_first))]
        r = np.asarray(r_rest, F32).copy()
        for l in range(self.nq - 1):
            d = sq_distances(self.cb_rest[l], r)
            code = int(np.argmin(d))
            codes.append(code)
            margins.append(_margin(d))
            if l < self.nq - 2:
                r = (r - self.cb_rest[l, code]).astype(F32)
        return np.array(codes, dtype=np.uint32), margins

    def encode(self, latent: np.ndarray) -> np.ndarray:
        return self.quantise(*self.project(latent))[0]

    def decode(self, codes) -> np.ndarray:
        """``out_first . emb_sum(first) + out_rest . emb_sum(rest)`` ([mimi] decode plan: the
        second MATVEC accumulates into the first's output)."""
        acc_f = emb_sum(self.cb_first, [codes[0]]).reshape(1, -1)
        acc_r = emb_sum(self.cb_rest, list(codes[1:])).reshape(1, -1)
        return (gemv(self.out_first, acc_f)[0] + gemv(self.out_rest, acc_r)[0]).astype(F32)


def _margin(d: np.ndarray):
    order = np.argsort(d, kind="stable")
    return float(d[order[0]]), float(d[order[1]]) if d.size > 1 else float("inf")
