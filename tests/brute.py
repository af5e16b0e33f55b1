"""An independent float64 brute-force decoder for tiny shapes, used to pin the oracle.

It is written from the same definitions but shares no code and no structure with ``oracle/``:
scalar Python loops, ``math.fsum`` sums, complex-number rope, and a plain per-layer history list
(every (position, k, v) ever pushed) with an explicit window test instead of a ring.  A dropped
term, a transposed operand, a wrong head mapping or a wrong rope pairing in the oracle shows up
as a mismatch against it.

Definitions followed (docs.rs inferencelayer pages): the talker layer of qwen3tts_gpu.rs
(``build_step_plan``; ``RMSNORM_SRC``, ``QK_NORM_SRC``, ``ROPE_SRC``, ``GQA_ATTN_SRC``,
``SWIGLU_SRC``) and the codec layer of mimi_gpu.rs (``Builder::transformer_shaped``; ``ln_src``,
``rope_push_src``, ``attn_src``, ``MV_LS``, ``GELU_ERF``).
"""
import cmath
import math


def matvec(w, x):
    return [math.fsum(w[n][k] * x[k] for k in range(len(x))) for n in range(len(w))]


def rms(v, g, eps):
    inv = 1.0 / math.sqrt(math.fsum(t * t for t in v) / len(v) + eps)
    return [v[i] * inv * g[i] for i in range(len(v))]


def lnorm(v, w, b, eps):
    mu = math.fsum(v) / len(v)
    var = math.fsum((t - mu) ** 2 for t in v) / len(v)
    inv = 1.0 / math.sqrt(var + eps)
    return [(v[i] - mu) * inv * w[i] + b[i] for i in range(len(v))]


def rotate(head, pos, theta, half_style):
    """Rope via complex multiplication: pair j holds the complex number a + ib."""
    hd = len(head)
    out = list(head)
    for j in range(hd // 2):
        ia, ib = (j, j + hd // 2) if half_style else (2 * j, 2 * j + 1)
        z = complex(head[ia], head[ib]) * cmath.exp(1j * pos * theta ** (-2.0 * j / hd))
        out[ia], out[ib] = z.real, z.imag
    return out


def softmax_attend(q, keys, vals):
    s = [math.fsum(q[i] * k[i] for i in range(len(q))) / math.sqrt(len(q)) for k in keys]
    mx = max(s)
    e = [math.exp(t - mx) for t in s]
    den = math.fsum(e)
    return [math.fsum(e[j] * vals[j][i] for j in range(len(keys))) / den for i in range(len(q))]


class BruteDecoder:
    def __init__(self, cfg, layers, final, window):
        self.cfg = cfg
        self.layers = [{k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in lw.items()}
                       for lw in layers]
        self.final = {k: v.tolist() for k, v in final.items()}
        self.window = window
        self.hist = [[] for _ in range(cfg.n_layers)]  # per layer: [(pos, k_heads, v_heads)]

    def step(self, x, pos):
        cfg = self.cfg
        x = [float(t) for t in x]
        hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        half = cfg.rope == 0
        rmsn = cfg.norm == 0
        for l, lw in enumerate(self.layers):
            n = rms(x, lw["attn_norm_w"], cfg.norm_eps) if rmsn else \
                lnorm(x, lw["attn_norm_w"], lw["attn_norm_b"], cfg.norm_eps)
            q = matvec(lw["wq"], n)
            k = matvec(lw["wk"], n)
            v = matvec(lw["wv"], n)
            qh = [q[h * hd:(h + 1) * hd] for h in range(hq)]
            kh = [k[h * hd:(h + 1) * hd] for h in range(hkv)]
            vh = [v[h * hd:(h + 1) * hd] for h in range(hkv)]
            if cfg.qk_norm:
                qh = [rms(t, lw["q_norm"], cfg.qk_norm_eps) for t in qh]
                kh = [rms(t, lw["k_norm"], cfg.qk_norm_eps) for t in kh]
            qh = [rotate(t, pos, cfg.rope_theta, half) for t in qh]
            kh = [rotate(t, pos, cfg.rope_theta, half) for t in kh]
            self.hist[l].append((pos, kh, vh))
            live = [(p, kk, vv) for (p, kk, vv) in self.hist[l] if 0 <= pos - p < self.window]
            o = []
            for h in range(hq):
                g = h * hkv // hq  # consecutive q heads share one kv head
                o += softmax_attend(qh[h], [kk[g] for (_, kk, _) in live],
                                    [vv[g] for (_, _, vv) in live])
            a = matvec(lw["wo"], o)
            ls1 = lw.get("ls1") if cfg.layer_scale else None
            x = [x[i] + (ls1[i] * a[i] if ls1 else a[i]) for i in range(len(x))]
            n = rms(x, lw["ffn_norm_w"], cfg.norm_eps) if rmsn else \
                lnorm(x, lw["ffn_norm_w"], lw["ffn_norm_b"], cfg.norm_eps)
            if cfg.ffn == 0:
                gt = matvec(lw["w_gate"], n)
                up = matvec(lw["w_up"], n)
                act = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
            else:
                u = matvec(lw["w_up"], n)
                act = [0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in u]
            f = matvec(lw["w_down"], act)
            ls2 = lw.get("ls2") if cfg.layer_scale else None
            x = [x[i] + (ls2[i] * f[i] if ls2 else f[i]) for i in range(len(x))]
        if cfg.final_norm:
            x = rms(x, self.final["norm_w"], cfg.norm_eps) if rmsn else \
                lnorm(x, self.final["norm_w"], self.final["norm_b"], cfg.norm_eps)
        return x
