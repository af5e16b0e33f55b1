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


def _elu(v):
    return v if v > 0 else math.exp(v) - 1.0


class BruteConv:
    """A causal conv fed one frame at a time: signals are lists of time columns (each a list of
    channel values); the last ``K - stride`` input columns carry over to the next frame."""

    def __init__(self, w, b, stride, pre_elu=False, groups=1):
        self.w, self.b = w.tolist(), b.tolist()
        self.s, self.elu, self.groups = stride, pre_elu, groups
        c_out, ipg, self.K = w.shape
        self.c_in = ipg * groups
        self.prev = [[0.0] * self.c_in for _ in range(self.K - stride)]

    def frame(self, cols):
        buf = self.prev + [list(c) for c in cols]
        c_out, ipg = len(self.w), len(self.w[0])
        opg = c_out // self.groups
        out = []
        for t in range(len(cols) // self.s):
            y = []
            for o in range(c_out):
                g = o // opg
                terms = [self.w[o][i][k] * (_elu(buf[t * self.s + k][g * ipg + i]) if self.elu
                                            else buf[t * self.s + k][g * ipg + i])
                         for i in range(ipg) for k in range(self.K)]
                y.append(self.b[o] + math.fsum(terms))
            out.append(y)
        self.prev = buf[len(buf) - (self.K - self.s):] if self.K > self.s else []
        return out


class BruteConvTr:
    """A transposed conv fed one frame at a time: input column t scatters tap k onto output
    column t * stride + k; the last ``K - stride`` partial sums (no bias yet) wait for the next
    frame, and a column gets its bias when it is emitted."""

    def __init__(self, w, b, stride, pre_elu=False, groups=1):
        self.w, self.b = w.tolist(), b.tolist()
        self.s, self.elu, self.groups = stride, pre_elu, groups
        c_in, opg, self.K = w.shape
        self.c_out = opg * groups
        self.pending = [[0.0] * self.c_out for _ in range(self.K - stride)]

    def frame(self, cols):
        n = len(cols) * self.s
        acc = [list(c) for c in self.pending] + [[0.0] * self.c_out
                                                 for _ in range(n + self.K - self.s - len(self.pending))]
        c_in, opg = len(self.w), len(self.w[0])
        ipg = c_in // self.groups
        for t, col in enumerate(cols):
            for i in range(c_in):
                v = _elu(col[i]) if self.elu else col[i]
                g = i // ipg
                for oo in range(opg):
                    for k in range(self.K):
                        acc[t * self.s + k][g * opg + oo] += self.w[i][oo][k] * v
        out = [[acc[t][o] + self.b[o] for o in range(self.c_out)] for t in range(n)]
        self.pending = acc[n:]
        return out


class BruteSEANet:
    """The SEANet-style decoder of ``seanet_layers`` streamed frame by frame from the brute
    pieces above (the first conv reads its input as is, every other layer through ELU)."""

    def __init__(self, layers, w):
        self.stages = []
        for i, (name, kind, _, stride) in enumerate(layers):
            W, B = w[name + ".w"], w[name + ".b"]
            conv = (BruteConvTr(W, B, stride, pre_elu=True) if kind == "convtr"
                    else BruteConv(W, B, stride, pre_elu=(i != 0)))
            self.stages.append((kind, conv))

    def frame(self, cols):
        h = cols
        block_in = None
        for kind, conv in self.stages:
            if kind == "res0":
                block_in = h
            out = conv.frame(h)
            if kind == "res1":
                out = [[a + c for a, c in zip(ra, rc)] for ra, rc in zip(block_in, out)]
            h = out
        return h


class BrutePocketFrame:
    """The Pocket-style codec frame streamed one latent at a time: 1x1 conv, channel-wise
    transposed conv, the transformer one position at a time (``BruteDecoder``, positions
    ``frame * stride + r``), then the SEANet stack; returns each frame's stages."""

    def __init__(self, cfg, conv, tr_layers, seanet_layers, seanet_w):
        self.quant = BruteConv(conv["quant.w"], conv["quant.b"], 1)
        self.up = BruteConvTr(conv["up.w"], conv["up.b"], cfg.up_stride, groups=cfg.dim)
        self.tr = BruteDecoder(cfg.transformer, tr_layers, {}, cfg.context)
        self.seanet = BruteSEANet(seanet_layers, seanet_w)
        self.pos = 0

    def frame(self, latent):
        z = self.quant.frame([list(latent[:, 0])])
        u = self.up.frame(z)
        tr = []
        for col in u:
            tr.append(self.tr.step(col, self.pos))
            self.pos += 1
        pcm = self.seanet.frame(tr)
        return {"quant": z, "up": u, "tr": tr, "pcm": pcm}
