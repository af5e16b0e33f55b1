"""CPU oracle of the streaming decode step.

TEST INFRASTRUCTURE ONLY: a plain, slow, float32 NumPy implementation written from the pages'
definitions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the HIP path never does, and this package imports nothing from it.
"""
from .step import (  # noqa: F401
    F32, INVALID_POS, NORM_LAYER, NORM_RMS, ROPE_HALF, ROPE_INTERLEAVED, FFN_GELU, FFN_SWIGLU,
    OracleDecoder, apply_rope, attend, gelu_erf, gemv, layer_norm, rms_norm, rope_cos_sin,
    rope_pairs, seq_sum, silu_mul, valid_slots,
)
from .rvq import OracleRVQ, emb_sum, nearest, sq_distances  # noqa: F401,E402
from .conv import (  # noqa: F401,E402
    causal_conv1d, conv_transpose1d_full, elu, streamed_conv_transpose1d,
)
from .pocket import decode_frames, seanet_decode  # noqa: F401,E402
