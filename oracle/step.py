"""CPU oracle of one streaming autoregressive decode step (plain NumPy, float32).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP path; both take their inputs from
``streaming_ar_transformer_amd.workloads``, which holds no arithmetic of the method.

Precision: the pages compute every step in float32 ("f32 everywhere" in the mimi_gpu.rs module
doc; the talker's self-contained f32 plan in the qwen3tts_gpu.rs module doc), so the oracle does
too.  The rope angle is formed and its cos/sin evaluated in float64 and rounded once to float32.
Softmax denominators and attention value sums run sequentially over keys in ascending position,
the order the qwen3tts_gpu.rs module doc and ``GQA_ATTN_SRC`` describe for the CPU stack.

Page names used in citations:
  [talker]  docs.rs inferencelayer 0.2.8, src/qwen3tts_gpu.rs
  [pocket]  docs.rs inferencelayer 0.2.4, src/pocket_tts_gpu.rs
  [mimi]    docs.rs inferencelayer 0.2.1, src/mimi_gpu.rs
  [parakeet] docs.rs inferencelayer 0.2.10, src/parakeet_gpu.rs
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
INVALID_POS = np.uint32(0xFFFFFFFF)  # [mimi] INVALID_POS: an empty position-ring slot

NORM_RMS, NORM_LAYER = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
FFN_SWIGLU, FFN_GELU = 0, 1


# ------------------------------------------------------------------------------------------------
# elementwise pieces
# ------------------------------------------------------------------------------------------------

def seq_sum(a: np.ndarray) -> np.ndarray:
    """Left-to-right float32 sum over axis 0 (``((a0 + a1) + a2) + ...``).

    [talker] module doc and ``GQA_ATTN_SRC``: the softmax denominator and the value accumulation
    run in the CPU's ascending-j order.  ``np.add.accumulate`` adds row by row."""
    a = np.asarray(a, dtype=F32)
    if a.shape[0] == 0:
        return np.zeros(a.shape[1:], dtype=F32)
    return np.add.accumulate(a, axis=0, dtype=F32)[-1]


def gemv(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """``y[r, n] = sum_k x[r, k] * w[n, k]`` with ``w`` row-major ``[n, k]`` and no bias.

    [talker] ``MATVEC_SRC`` (``y[m,n] = x[m,k] @ W[n,k]^T``); [mimi] ``MATVEC``.  The library
    matmul is the step; its float32 summation order is as good as any other (the pages' gate is a
    cosine, not bitwise equality: [talker] module doc, equality standard)."""
    return np.matmul(np.asarray(x, F32), np.asarray(w, F32).T).astype(F32, copy=False)


def rms_norm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """``v * (1 / sqrt(mean(v^2) + eps)) * g`` over the last axis.

    [talker] ``RMSNORM_SRC`` (whole hidden row) and ``QK_NORM_SRC`` (one head)."""
    v = np.asarray(v, F32)
    ss = np.sum(v * v, axis=-1, dtype=F32, keepdims=True)
    inv = F32(1.0) / np.sqrt(ss / F32(v.shape[-1]) + F32(eps))
    return (v * inv) * np.asarray(g, F32)


def layer_norm(v: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """Affine LayerNorm, two passes: the mean, then the biased variance of the centred row.

    [mimi] ``LN512`` and ``ln_src``: ``(x - mean) * (1 / sqrt(var + eps)) * w + b``."""
    v = np.asarray(v, F32)
    n = F32(v.shape[-1])
    mean = np.sum(v, axis=-1, dtype=F32, keepdims=True) / n
    d = v - mean
    var = np.sum(d * d, axis=-1, dtype=F32, keepdims=True) / n
    inv = F32(1.0) / np.sqrt(var + F32(eps))
    return (d * inv) * np.asarray(w, F32) + np.asarray(b, F32)


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``(g / (1 + exp(-g))) * up``.  [talker] ``SWIGLU_SRC``."""
    g = np.asarray(gate, F32)
    return (g / (F32(1.0) + np.exp(-g))) * np.asarray(up, F32)


def gelu_erf(v: np.ndarray) -> np.ndarray:
    """Exact GELU ``0.5 * v * (1 + erf(v / sqrt(2)))``, evaluated in float64, rounded once.

    [mimi] ``GELU_ERF`` (the codec's FFN activation)."""
    v64 = np.asarray(v, np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return (0.5 * v64 * (1.0 + erf(v64 / math.sqrt(2.0)))).astype(F32)


# ------------------------------------------------------------------------------------------------
# rope
# ------------------------------------------------------------------------------------------------

def rope_cos_sin(pos: int, head_dim: int, theta: float):
    """cos/sin of ``pos * theta^(-2j/head_dim)`` for the ``head_dim/2`` frequency indices ``j``.

    The angle and both trig functions are float64, rounded once to float32.  The frequencies are
    HF's inverse frequencies ([talker] ``TalkerGpu::load``: CPU-built cos/sin tables with
    ``cos[i] == cos[i + half]``; [mimi] ``rope_push_src``: ``exp(-ln(theta) * 2j / hd)``)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * j / float(head_dim))
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope_pairs(head_dim: int, style: int):
    """Index pairs ``(a_j, b_j)`` rotated by frequency ``j``.

    rotate_half ([talker] ``ROPE_SRC``): ``(j, j + hd/2)``; interleaved ([mimi]
    ``rope_push_src``): ``(2j, 2j + 1)``."""
    j = np.arange(head_dim // 2)
    if style == ROPE_HALF:
        return j, j + head_dim // 2
    return 2 * j, 2 * j + 1


def apply_rope(xh: np.ndarray, cos: np.ndarray, sin: np.ndarray, style: int) -> np.ndarray:
    """Rotate each pair: ``(a, b) -> (a cos - b sin, a sin + b cos)`` on the last axis.

    For rotate_half this is ``x*cos + rotate_half(x)*sin`` ([talker] ``ROPE_SRC``); for the
    interleaved form it is [mimi] ``rope_push_src``'s ``(qr*cs - qi*sn, qr*sn + qi*cs)``."""
    xh = np.asarray(xh, F32)
    ia, ib = rope_pairs(xh.shape[-1], style)
    a, b = xh[..., ia], xh[..., ib]
    out = np.empty_like(xh)
    out[..., ia] = a * cos - b * sin
    out[..., ib] = a * sin + b * cos
    return out


# ------------------------------------------------------------------------------------------------
# ring attention
# ------------------------------------------------------------------------------------------------

def valid_slots(P: np.ndarray, pos: int, window: int) -> np.ndarray:
    """Slots a query at ``pos`` may attend, ordered by ascending stored position.

    [mimi] ``attn_src``: slot j is legal iff ``P[j] != INVALID``, ``P[j] <= pos`` and
    ``pos - P[j] < window``."""
    P = np.asarray(P, np.uint32).astype(np.int64)
    ok = (P != int(INVALID_POS)) & (P <= pos) & (pos - P < window)
    slots = np.nonzero(ok)[0]
    return slots[np.argsort(P[slots], kind="stable")]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, P: np.ndarray, pos: int, window: int,
           n_kv_heads: int, normalize_weights_first: bool) -> np.ndarray:
    """Causal GQA attention of the query row ``q[Hq, hd]`` over one stream's ring.

    ``K``, ``V`` are ``[R, Hkv, hd]``.  q-head ``h`` reads kv head ``h // (Hq / Hkv)``
    ([talker] ``GQA_ATTN_SRC``: ``kvh = head / group``).  Scores are ``(q . k) * (1/sqrt(hd))``;
    ``mx`` is their max; ``e_j = exp(s_j - mx)``; ``den`` is the sequential sum of ``e``.  The
    talker form divides first and then sums ``p_j v_j`` ([talker] ``GQA_ATTN_SRC``); the codec
    form sums ``e_j v_j`` and divides once ([mimi] ``attn_src``).  Masked slots contribute
    nothing."""
    n_q, hd = q.shape
    group = n_q // n_kv_heads
    scale = F32(1.0) / np.sqrt(F32(hd))
    slots = valid_slots(P, pos, window)
    out = np.zeros((n_q, hd), dtype=F32)
    if slots.size == 0:
        return out
    for h in range(n_q):
        g = h // group
        k = K[slots, g, :]
        v = V[slots, g, :]
        s = (k @ q[h]).astype(F32) * scale
        mx = np.max(s)
        e = np.exp(s - mx).astype(F32)
        den = seq_sum(e)
        if normalize_weights_first:
            p = e / den
            out[h] = seq_sum(p[:, None] * v)
        else:
            out[h] = seq_sum(e[:, None] * v) / den
    return out


# ------------------------------------------------------------------------------------------------
# the decoder stack
# ------------------------------------------------------------------------------------------------

class OracleDecoder:
    """State and step of one stack: ``m`` independent streams, each with its own K/V rings.

    Per stream: K, V rings ``[n_layers, R, Hkv, hd]`` and ONE position ring ``P[R]`` shared by
    every layer of the stack (each layer stamps the same position into the same slot: [mimi]
    ``Builder::transformer_shaped`` allocates one position ring per stack).  All slots start
    INVALID ([mimi] ``MimiGpu::new``/``reset``; [pocket] ``PocketCodecGpu::new``)."""

    def __init__(self, cfg, layers, final, ring: int | None = None, window: int | None = None,
                 unbounded: bool | None = None):
        self.cfg = cfg
        self.layers = layers
        self.final = final
        self.R = cfg.ring if ring is None else ring
        self.W = cfg.window if window is None else window
        # The talker's cache (and the FlowLM ring) refuses positions past its capacity
        # ([talker] ``TalkerGpu::step``; [pocket] ``PocketBackboneGpu::step``); a codec ring wraps.
        self.unbounded = cfg.is_unbounded if unbounded is None else unbounded
        if self.W > self.R or self.W < 1:
            raise ValueError("window must be in [1, ring]")
        m, L, hkv, hd = cfg.m, cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        self.K = np.zeros((m, L, self.R, hkv, hd), dtype=F32)
        self.V = np.zeros((m, L, self.R, hkv, hd), dtype=F32)
        self.P = np.full((m, self.R), INVALID_POS, dtype=np.uint32)
        self.next_pos = None

    def reset(self):
        """Fresh session: zero the K/V rings, invalidate every position-ring slot."""
        self.K[:] = 0
        self.V[:] = 0
        self.P[:] = INVALID_POS
        self.next_pos = None

    def import_kv(self, stream: int, K: np.ndarray, V: np.ndarray, positions):
        """Write cached, already-roped K/V rows into the rings at ``slot = position mod R`` and
        stamp the position ring ([pocket] ``PocketBackboneGpu::load_voice``: the cache layout
        ``[positions][heads][head_dim]`` is the ring's slot-major layout).  ``K``/``V`` are
        ``[n_layers, len(positions), Hkv, hd]``."""
        positions = np.asarray(positions, dtype=np.int64)
        slots = positions % self.R
        self.K[stream][:, slots] = K
        self.V[stream][:, slots] = V
        self.P[stream][slots] = positions.astype(np.uint32)
        nxt = int(positions.max()) + 1 if positions.size else 0
        self.next_pos = nxt

    def _check(self, pos: int, first: bool):
        if not first and self.next_pos is not None and pos != self.next_pos:
            raise ValueError(f"step pos {pos} != next position {self.next_pos} "
                             "(positions must be contiguous)")
        if self.unbounded and pos >= self.R:
            raise ValueError(f"position {pos} exceeds the {self.R}-slot ring")

    def prefill(self, xs: np.ndarray, pos: int, first: bool = False):
        """A block of ``t`` consecutive positions ``pos .. pos+t-1`` of the single stream in one
        pass; returns every row's output ``[t, d]``.

        [talker] ``TalkerGpu::prefill`` -> ``forward_rows``: the block's rows go through each
        GEMV together, all of the block's K/V rows are appended to the cache before attention,
        and row ``r`` (absolute position ``pos + r``) attends causally: to the cache and to the
        block's rows up to itself.  With a ring this is the legal set at ``pos + r``, provided
        no append evicts a position an earlier row of the block still attends: required here as
        ``pos + t <= R`` (no append evicts anything, the talker's case) or ``R >= W + t - 1``.
        [pocket] ``PocketBackboneGpu``'s doc states the property this must have: feeding the
        block one position at a time gives the same hidden states."""
        cfg = self.cfg
        if cfg.m != 1:
            raise ValueError("prefill runs on a single-stream stack")
        pos = int(pos)
        xs = np.array(xs, dtype=F32).reshape(-1, cfg.d_model)
        t = xs.shape[0]
        if t < 1:
            raise ValueError("empty block")
        if pos + t > self.R and self.R < self.W + t - 1:
            raise ValueError(f"a {t}-row block past the first ring turn needs ring >= window + "
                             f"{t - 1}")
        self._check(pos, first)
        if self.unbounded and pos + t - 1 >= self.R:
            raise ValueError(f"position {pos + t - 1} exceeds the {self.R}-slot ring")
        if first:
            self.P[:] = INVALID_POS
        positions = pos + np.arange(t)
        slots = positions % self.R
        self.P[0, slots] = positions.astype(np.uint32)
        hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        tables = [rope_cos_sin(int(p), hd, cfg.rope_theta) for p in positions]

        def norm(v, w, b):
            if cfg.norm == NORM_RMS:
                return rms_norm(v, w, cfg.norm_eps)
            return layer_norm(v, w, b, cfg.norm_eps)

        def rope_rows(v):  # v [t, heads, hd]: row r rotated by position pos + r
            return np.stack([apply_rope(v[r], tables[r][0], tables[r][1], cfg.rope)
                             for r in range(t)])

        x = xs
        for l, lw in enumerate(self.layers):
            n = norm(x, lw["attn_norm_w"], lw.get("attn_norm_b"))
            q = gemv(lw["wq"], n).reshape(t, hq, hd)
            k = gemv(lw["wk"], n).reshape(t, hkv, hd)
            v = gemv(lw["wv"], n).reshape(t, hkv, hd)
            if cfg.qk_norm:
                q = rms_norm(q, lw["q_norm"], cfg.qk_norm_eps)
                k = rms_norm(k, lw["k_norm"], cfg.qk_norm_eps)
            q, k = rope_rows(q), rope_rows(k)
            self.K[0, l, slots] = k  # the whole block is appended before any row attends
            self.V[0, l, slots] = v
            o = np.stack([
                attend(q[r], self.K[0, l], self.V[0, l], self.P[0], int(positions[r]), self.W,
                       hkv, normalize_weights_first=(cfg.family == "T"))
                for r in range(t)]).reshape(t, hq * hd)
            a_proj = gemv(lw["wo"], o)
            x = x + (lw["ls1"] * a_proj if cfg.layer_scale else a_proj)
            n = norm(x, lw["ffn_norm_w"], lw.get("ffn_norm_b"))
            if cfg.ffn == FFN_SWIGLU:
                act = silu_mul(gemv(lw["w_gate"], n), gemv(lw["w_up"], n))
            else:
                act = gelu_erf(gemv(lw["w_up"], n))
            f_proj = gemv(lw["w_down"], act)
            x = x + (lw["ls2"] * f_proj if cfg.layer_scale else f_proj)
        if cfg.final_norm:
            x = norm(x, self.final["norm_w"], self.final.get("norm_b"))
        self.next_pos = pos + t
        return x

    def step(self, x: np.ndarray, pos: int, first: bool = False, taps: dict | None = None):
        """Advance every stream by one position; returns the output rows ``[m, d]``.

        Talker family, per layer ([talker] ``build_step_plan``): RMSNorm -> q,k,v GEMVs ->
        per-head qk-RMSNorm -> rope -> ring push -> attention -> o GEMV + residual -> RMSNorm ->
        SwiGLU FFN -> down GEMV + residual; a final RMSNorm ends the stack.
        Codec family, per layer ([mimi] ``Builder::transformer_shaped``): LayerNorm -> packed
        qkv GEMV -> rope + ring push -> attention -> out GEMV with LayerScale into the residual ->
        LayerNorm -> lin1 GEMV -> GELU -> lin2 GEMV with LayerScale into the residual.  The
        output is the residual stream.

        ``first`` starts fresh streams: the position rings are invalidated before the step (the
        per-frame ``(pos, first)`` uniform of [mimi]'s module doc).  With ``taps`` a dict,
        per-layer branch values are appended under ``"attn"`` (attention output before the o
        projection), ``"attn_proj"`` and ``"ffn_proj"`` (projection outputs before LayerScale
        and the residual add)."""
        cfg = self.cfg
        pos = int(pos)
        self._check(pos, first)
        x = np.array(x, dtype=F32).reshape(cfg.m, cfg.d_model)
        if first:
            self.P[:] = INVALID_POS
        slot = pos % self.R
        self.P[:, slot] = np.uint32(pos)
        cos, sin = rope_cos_sin(pos, cfg.head_dim, cfg.rope_theta)
        hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        if taps is not None:
            for key in ("attn", "attn_proj", "ffn_proj"):
                taps.setdefault(key, [])

        def norm(v, w, b):
            if cfg.norm == NORM_RMS:
                return rms_norm(v, w, cfg.norm_eps)
            return layer_norm(v, w, b, cfg.norm_eps)

        for l, lw in enumerate(self.layers):
            n = norm(x, lw["attn_norm_w"], lw.get("attn_norm_b"))
            q = gemv(lw["wq"], n).reshape(cfg.m, hq, hd)
            k = gemv(lw["wk"], n).reshape(cfg.m, hkv, hd)
            v = gemv(lw["wv"], n).reshape(cfg.m, hkv, hd)
            if cfg.qk_norm:
                q = rms_norm(q, lw["q_norm"], cfg.qk_norm_eps)
                k = rms_norm(k, lw["k_norm"], cfg.qk_norm_eps)
            q = apply_rope(q, cos, sin, cfg.rope)
            k = apply_rope(k, cos, sin, cfg.rope)
            self.K[:, l, slot] = k
            self.V[:, l, slot] = v
            o = np.stack([
                attend(q[s], self.K[s, l], self.V[s, l], self.P[s], pos, self.W, hkv,
                       normalize_weights_first=(cfg.family == "T"))
                for s in range(cfg.m)]).reshape(cfg.m, hq * hd)
            a_proj = gemv(lw["wo"], o)
            x = x + (lw["ls1"] * a_proj if cfg.layer_scale else a_proj)
            n = norm(x, lw["ffn_norm_w"], lw.get("ffn_norm_b"))
            if cfg.ffn == FFN_SWIGLU:
                act = silu_mul(gemv(lw["w_gate"], n), gemv(lw["w_up"], n))
            else:
                act = gelu_erf(gemv(lw["w_up"], n))
            f_proj = gemv(lw["w_down"], act)
            x = x + (lw["ls2"] * f_proj if cfg.layer_scale else f_proj)
            if taps is not None:
                taps["attn"].append(o.copy())
                taps["attn_proj"].append(a_proj.copy())
                taps["ffn_proj"].append(f_proj.copy())
        if cfg.final_norm:
            x = norm(x, self.final["norm_w"], self.final.get("norm_b"))
        self.next_pos = pos + 1
        return x
