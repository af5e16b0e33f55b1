"""ctypes binding of ``libsdec.so`` (declared in ``include/sdec.h``).

Argument marshalling only: every step of the decode path runs in the library's HIP kernels.
PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  If the library is missing this module raises on
import of :func:`lib` — there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before libsdec.so binds to it)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdec.so")

OK, E_ARG, E_POS, E_CAPACITY, E_HIP, E_NOMEM = 0, -1, -2, -3, -4, -5
FLAG_EAGER, FLAG_TAPS = 1, 2
PATH_GRAPH, PATH_EAGER = 0, 1
ATTN_LIST, ATTN_SHORT, ATTN_SPLIT = 0, 1, 2
K_NAMES = ["begin", "qkv", "attention", "o_proj", "ffn_up", "ffn_down", "end"]

# Every symbol include/sdec.h declares.
EXPORTS = ["sdec_create", "sdec_step", "sdec_reset", "sdec_destroy", "sdec_last_error",
           "sdec_kv_view", "sdec_set_next_position", "sdec_tap_view", "sdec_step_profile",
           "sdec_gemv", "sdec_ring_attention", "sdec_ring_attention_static", "sdec_status",
           "sdec_prefill", "sdec_rvq_create", "sdec_rvq_encode", "sdec_rvq_quantise", "sdec_rvq_decode",
           "sdec_rvq_destroy", "sdec_conv_create", "sdec_conv_step", "sdec_conv_destroy",
           "sdec_transpose"]


class SdecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sdec error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_uint32), ("d_model", ctypes.c_uint32),
                ("n_q_heads", ctypes.c_uint32), ("n_kv_heads", ctypes.c_uint32),
                ("head_dim", ctypes.c_uint32), ("d_ff", ctypes.c_uint32), ("m", ctypes.c_uint32),
                ("norm", ctypes.c_uint32), ("norm_eps", ctypes.c_float),
                ("qk_norm", ctypes.c_uint32), ("qk_norm_eps", ctypes.c_float),
                ("rope", ctypes.c_uint32), ("rope_theta", ctypes.c_double),
                ("ffn", ctypes.c_uint32), ("layer_scale", ctypes.c_uint32),
                ("final_norm", ctypes.c_uint32), ("window", ctypes.c_uint32),
                ("unbounded", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("max_prefill", ctypes.c_uint32)]


_LAYER_FIELDS = ["attn_norm_w", "attn_norm_b", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "ls1",
                 "ffn_norm_w", "ffn_norm_b", "w_gate", "w_up", "w_down", "ls2"]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


class FinalWeights(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("norm_b", ctypes.c_void_p)]


class RVQConfig(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_uint32), ("vq", ctypes.c_uint32), ("bins", ctypes.c_uint32),
                ("nq", ctypes.c_uint32), ("max_frames", ctypes.c_uint32)]


_RVQ_FIELDS = ["in_first", "in_rest", "out_first", "out_rest", "cb_first", "cb_rest"]


class RVQWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _RVQ_FIELDS]


class ConvConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ("in_ch", "out_ch", "kernel", "stride", "groups",
                                               "transposed", "pre_elu", "replicate_first",
                                               "accumulate", "max_t_in")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
        sig = {
            "sdec_create": (i32, [ctypes.POINTER(Config), ctypes.POINTER(LayerWeights),
                                  ctypes.POINTER(FinalWeights), u32, ctypes.POINTER(vp)]),
            "sdec_step": (i32, [vp, vp, u32, u32, vp]),
            "sdec_prefill": (i32, [vp, vp, u32, u32, u32, vp]),
            "sdec_reset": (i32, [vp, vp]),
            "sdec_destroy": (None, [vp]),
            "sdec_last_error": (ctypes.c_char_p, []),
            "sdec_kv_view": (i32, [vp, u32, u32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(vp)]),
            "sdec_set_next_position": (i32, [vp, u32]),
            "sdec_tap_view": (i32, [vp, u32, u32, ctypes.POINTER(vp)]),
            "sdec_step_profile": (i32, [vp, vp, u32, u32, vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(u32)]),
            "sdec_gemv": (i32, [vp, vp, vp, u32, u32, u32, vp]),
            "sdec_status": (i32, [vp, ctypes.POINTER(u32), ctypes.POINTER(u32)]),
            "sdec_ring_attention": (i32, [vp, vp, vp, vp, vp, u32, u32, u32, u32, u32, u32, u32,
                                          vp]),
            "sdec_ring_attention_static": (i32, [vp, vp, vp, vp, vp, u32, u32, u32, u32, u32, u32,
                                                 u32, vp]),
            "sdec_rvq_create": (i32, [ctypes.POINTER(RVQConfig), ctypes.POINTER(RVQWeights),
                                      ctypes.POINTER(vp)]),
            "sdec_rvq_encode": (i32, [vp, vp, u32, vp, vp]),
            "sdec_rvq_quantise": (i32, [vp, vp, vp, u32, vp, vp]),
            "sdec_rvq_decode": (i32, [vp, vp, u32, vp, vp]),
            "sdec_rvq_destroy": (None, [vp]),
            "sdec_conv_create": (i32, [ctypes.POINTER(ConvConfig), vp, vp, ctypes.POINTER(vp)]),
            "sdec_conv_step": (i32, [vp, vp, u32, vp, u32, vp]),
            "sdec_conv_destroy": (None, [vp]),
            "sdec_transpose": (i32, [vp, u32, u32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int):
    if code != OK:
        raise SdecError(code, lib().sdec_last_error().decode())


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.dtype in (torch.float32, torch.int32) and t.is_contiguous(), \
        "device float32 contiguous tensors only"
    return t.data_ptr()


def make_config(cfg, window=None, unbounded=None, eager=False, taps=False,
                max_prefill=0) -> Config:
    """Fill the C struct from a ``workloads.StepConfig``-like object."""
    c = Config()
    c.n_layers, c.d_model = cfg.n_layers, cfg.d_model
    c.n_q_heads, c.n_kv_heads, c.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    c.d_ff, c.m = cfg.d_ff, cfg.m
    c.norm, c.norm_eps = cfg.norm, cfg.norm_eps
    c.qk_norm, c.qk_norm_eps = int(cfg.qk_norm), cfg.qk_norm_eps
    c.rope, c.rope_theta = cfg.rope, cfg.rope_theta
    c.ffn, c.layer_scale, c.final_norm = cfg.ffn, int(cfg.layer_scale), int(cfg.final_norm)
    c.window = cfg.window if window is None else window
    c.unbounded = int(cfg.is_unbounded if unbounded is None else unbounded)
    c.flags = (FLAG_EAGER if eager else 0) | (FLAG_TAPS if taps else 0)
    c.max_prefill = max_prefill
    return c


class Decoder:
    """One stack behind ``sdec_create`` / ``sdec_step`` / ``sdec_reset``.

    ``layers`` is a list of dicts of device float32 tensors keyed like ``sdec_layer_weights``;
    they are borrowed (this object keeps references so they outlive the handle)."""

    def __init__(self, cfg, layers, final=None, ring=None, window=None, unbounded=None,
                 eager=False, taps=False, max_prefill=0):
        self.cfg = cfg
        self.ring = cfg.ring if ring is None else ring
        self.c = make_config(cfg, window=window, unbounded=unbounded, eager=eager, taps=taps,
                             max_prefill=max_prefill)
        self._keep = (layers, final)
        arr = (LayerWeights * cfg.n_layers)()
        for i, lw in enumerate(layers):
            for name in _LAYER_FIELDS:
                setattr(arr[i], name, _ptr(lw.get(name)))
        fw = FinalWeights()
        if final:
            fw.norm_w, fw.norm_b = _ptr(final.get("norm_w")), _ptr(final.get("norm_b"))
        h = ctypes.c_void_p()
        _check(lib().sdec_create(ctypes.byref(self.c), arr, ctypes.byref(fw), self.ring,
                                 ctypes.byref(h)))
        self.h = h

    def step(self, x, pos: int, first: bool = False, stream=None):
        _check(lib().sdec_step(self.h, _ptr(x), int(pos), int(bool(first)), _stream(stream)))
        return x

    def prefill(self, x, pos: int, first: bool = False, stream=None):
        """Block of ``x.shape[0]`` consecutive positions from ``pos`` (``sdec_prefill``)."""
        _check(lib().sdec_prefill(self.h, _ptr(x), int(pos), int(x.shape[0]), int(bool(first)),
                                  _stream(stream)))
        return x

    def step_profile(self, x, pos: int, first: bool = False, stream=None, into=None):
        """Eager step with a HIP event pair around each launch; returns {kernel: [ms, calls]}."""
        ms = (ctypes.c_double * len(K_NAMES))()
        calls = (ctypes.c_uint32 * len(K_NAMES))()
        _check(lib().sdec_step_profile(self.h, _ptr(x), int(pos), int(bool(first)),
                                       _stream(stream), ms, calls))
        out = into if into is not None else {k: [0.0, 0] for k in K_NAMES}
        for i, k in enumerate(K_NAMES):
            out[k][0] += ms[i]
            out[k][1] += calls[i]
        return out

    @property
    def path(self) -> int:
        """The step path in use: PATH_GRAPH or PATH_EAGER."""
        path = ctypes.c_uint32()
        _check(lib().sdec_status(self.h, ctypes.byref(path), None))
        return path.value

    @property
    def attention_form(self) -> int:
        """How the last step's attention ran: ATTN_LIST, ATTN_SHORT or ATTN_SPLIT."""
        form = ctypes.c_uint32()
        _check(lib().sdec_status(self.h, None, ctypes.byref(form)))
        return form.value

    def reset(self, stream=None):
        _check(lib().sdec_reset(self.h, _stream(stream)))

    def kv_view(self, stream_idx: int, layer: int):
        k, v, p = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().sdec_kv_view(self.h, stream_idx, layer, ctypes.byref(k), ctypes.byref(v),
                                  ctypes.byref(p)))
        return k.value, v.value, p.value

    def set_next_position(self, pos: int):
        _check(lib().sdec_set_next_position(self.h, int(pos)))

    def tap_view(self, layer: int, which: int) -> int:
        p = ctypes.c_void_p()
        _check(lib().sdec_tap_view(self.h, layer, which, ctypes.byref(p)))
        return p.value

    def close(self):
        if getattr(self, "h", None):
            lib().sdec_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemv(w, x, y, stream=None):
    """``y[m, n] = x[m, k] @ w[n, k]^T`` through ``sdec_gemv``."""
    n, k = w.shape
    m = x.shape[0]
    _check(lib().sdec_gemv(_ptr(w), _ptr(x), _ptr(y), n, k, m, _stream(stream)))
    return y


def ring_attention(q, k_ring, v_ring, pos_ring, out, n_q_heads, n_kv_heads, head_dim, ring,
                   window, pos, stream=None):
    m = q.shape[0]
    _check(lib().sdec_ring_attention(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(pos_ring),
                                     _ptr(out), m, n_q_heads, n_kv_heads, head_dim, ring, window,
                                     int(pos), _stream(stream)))
    return out


def ring_attention_static(q, k_ring, v_ring, pos_ring, out, n_q_heads, n_kv_heads, head_dim,
                          ring, window, pos, stream=None):
    """``ring_attention`` through the entry point that allocates nothing (its scratch is a fixed
    array in device memory, shared by every call on the device)."""
    m = q.shape[0]
    _check(lib().sdec_ring_attention_static(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(pos_ring),
                                            _ptr(out), m, n_q_heads, n_kv_heads, head_dim, ring,
                                            window, int(pos), _stream(stream)))
    return out


# --- raw device copies for ring import/export (marshalling through the HIP runtime) ---

def _hip():
    # The runtime torch loaded is already in the process under this soname.
    return ctypes.CDLL("libamdhip64.so.7")


def copy_from_device(ptr: int, nbytes: int, dtype, shape):
    import numpy as np
    out = np.empty(shape, dtype=dtype)
    assert out.nbytes == nbytes
    torch.cuda.synchronize()
    hip = _hip()
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(ptr),
                       ctypes.c_size_t(nbytes), 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise RuntimeError(f"hipMemcpy D2H failed: {rc}")
    return out


def copy_to_device(ptr: int, arr):
    import numpy as np
    arr = np.ascontiguousarray(arr)
    torch.cuda.synchronize()
    hip = _hip()
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(ctypes.c_void_p(ptr), ctypes.c_void_p(arr.ctypes.data),
                       ctypes.c_size_t(arr.nbytes), 1)  # hipMemcpyHostToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy H2D failed: {rc}")


class RVQ:
    """Split RVQ behind ``sdec_rvq_*``.  ``weights`` maps the ``sdec_rvq_weights`` names to
    device float32 tensors (borrowed: this object keeps references); codes are int32 tensors
    ``[frames, nq]`` holding the uint32 codes."""

    def __init__(self, dim, vq, bins, nq, max_frames, weights):
        self.c = RVQConfig(dim, vq, bins, nq, max_frames)
        self._keep = weights
        w = RVQWeights()
        for n in _RVQ_FIELDS:
            setattr(w, n, _ptr(weights[n]))
        h = ctypes.c_void_p()
        _check(lib().sdec_rvq_create(ctypes.byref(self.c), ctypes.byref(w), ctypes.byref(h)))
        self.h = h

    def encode(self, latent, codes, stream=None):
        _check(lib().sdec_rvq_encode(self.h, _ptr(latent), int(latent.shape[0]), _ptr(codes),
                                     _stream(stream)))
        return codes

    def quantise(self, r_first, r_rest, codes, stream=None):
        _check(lib().sdec_rvq_quantise(self.h, _ptr(r_first), _ptr(r_rest),
                                       int(r_first.shape[0]), _ptr(codes), _stream(stream)))
        return codes

    def decode(self, codes, latent, stream=None):
        _check(lib().sdec_rvq_decode(self.h, _ptr(codes), int(codes.shape[0]), _ptr(latent),
                                     _stream(stream)))
        return latent

    def close(self):
        if getattr(self, "h", None):
            lib().sdec_rvq_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def transpose(x, y, stream=None):
    """``y = x.T`` for a device ``[rows, cols]`` float32 tensor into a ``[cols, rows]`` one
    (``sdec_transpose``)."""
    rows, cols = x.shape
    assert tuple(y.shape) == (cols, rows), "y must be [cols, rows]"
    _check(lib().sdec_transpose(_ptr(x), rows, cols, _ptr(y), _stream(stream)))
    return y


class StreamConv:
    """One streaming (transposed) conv behind ``sdec_conv_*``: ``w`` and ``b`` are device float32
    tensors (borrowed); frames are device ``[in_ch, t_in]`` tensors."""

    def __init__(self, w, b, stride, transposed=False, groups=1, pre_elu=False,
                 replicate_first=False, accumulate=False, max_t_in=1024):
        if transposed:
            in_ch, opg, k = w.shape
            out_ch = opg * groups
        else:
            out_ch, ipg, k = w.shape
            in_ch = ipg * groups
        self.c = ConvConfig(in_ch, out_ch, k, stride, groups, int(transposed), int(pre_elu),
                            int(replicate_first), int(accumulate), max_t_in)
        self._keep = (w, b)
        self.stride, self.transposed, self.out_ch = stride, transposed, out_ch
        h = ctypes.c_void_p()
        _check(lib().sdec_conv_create(ctypes.byref(self.c), _ptr(w), _ptr(b), ctypes.byref(h)))
        self.h = h

    def out_cols(self, t_in: int) -> int:
        return t_in * self.stride if self.transposed else t_in // self.stride

    def step(self, x, y, first=False, stream=None):
        _check(lib().sdec_conv_step(self.h, _ptr(x), int(x.shape[1]), _ptr(y), int(bool(first)),
                                    _stream(stream)))
        return y

    def close(self):
        if getattr(self, "h", None):
            lib().sdec_conv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

