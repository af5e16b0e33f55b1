/*
 * sdec — one autoregressive decode step of a streaming transformer on MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; every device pointer is a HIP device address, every
 * stream a hipStream_t passed as void*.  The method these calls implement is the one the
 * docs.rs inferencelayer pages describe:
 *   [talker] inferencelayer 0.2.8, src/qwen3tts_gpu.rs — TalkerGpu::load / new_state / step
 *            and the build_step_plan pass list (RMSNorm, q/k/v GEMVs, per-head qk-RMSNorm,
 *            rotate_half rope, KV append, GQA causal attention, o GEMV + residual, RMSNorm,
 *            SwiGLU FFN, down GEMV + residual, final RMSNorm);
 *   [mimi]   inferencelayer 0.2.1, src/mimi_gpu.rs — TrShape, Builder::transformer_shaped
 *            (LayerNorm, packed qkv GEMV, rope fused with the KV-ring push, windowed ring
 *            attention, GEMVs with LayerScale folded into the residual, GELU), reset;
 *   [pocket] inferencelayer 0.2.4, src/pocket_tts_gpu.rs — PocketBackboneGpu::load_voice
 *            (importing a K/V cache into the rings), step (ring capacity check), reset.
 *
 * Errors: every int-returning call returns SDEC_OK (0) or a negative code; the message of the
 * last failure on the calling thread is in sdec_last_error().  All argument checks run on the
 * host before anything is enqueued; on error no GPU work is enqueued and the handle's state is
 * unchanged.
 */
#ifndef SDEC_H
#define SDEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SDEC_OK = 0,
  SDEC_E_ARG = -1,      /* null pointer, bad configuration, misaligned pointer, bad m */
  SDEC_E_POS = -2,      /* pos is not the next position while first == 0 ([talker] step:
                           positions must be contiguous) */
  SDEC_E_CAPACITY = -3, /* an unbounded stack got a position past its ring ([talker] step:
                           cache length past max_pos; [pocket] PocketBackboneGpu::step) */
  SDEC_E_HIP = -4,      /* a HIP runtime call failed; the message carries hipGetErrorString */
  SDEC_E_NOMEM = -5     /* device allocation failed */
};

enum { SDEC_NORM_RMS = 0, SDEC_NORM_LAYER = 1 };
enum { SDEC_ROPE_HALF = 0, SDEC_ROPE_INTERLEAVED = 1 };
enum { SDEC_FFN_SWIGLU = 0, SDEC_FFN_GELU_ERF = 1 };

/* sdec_config.flags */
#define SDEC_FLAG_EAGER 1u /* launch kernels one by one per step instead of replaying a graph */
#define SDEC_FLAG_TAPS 2u  /* keep per-layer branch outputs readable through sdec_tap_view */

/* Geometry and options of one decoder stack ([talker] Dims; [mimi] TrShape). */
typedef struct sdec_config {
  uint32_t n_layers;
  uint32_t d_model;     /* hidden width; multiple of 4 */
  uint32_t n_q_heads;
  uint32_t n_kv_heads;  /* divides n_q_heads; q-head h reads kv head h / (n_q_heads/n_kv_heads) */
  uint32_t head_dim;    /* 64 or 128 ([talker] load: head_dim <= 128) */
  uint32_t d_ff;        /* FFN width; multiple of 4 */
  uint32_t m;           /* independent streams stepped in lockstep, 1..8 */
  uint32_t norm;        /* SDEC_NORM_RMS (x/sqrt(mean x^2+eps)*g) or SDEC_NORM_LAYER (two-pass) */
  float norm_eps;
  uint32_t qk_norm;     /* nonzero: per-head RMSNorm of q and k before rope ([talker] QK_NORM_SRC) */
  float qk_norm_eps;
  uint32_t rope;        /* SDEC_ROPE_HALF: pairs (j, j+hd/2); SDEC_ROPE_INTERLEAVED: (2j, 2j+1) */
  double rope_theta;    /* angle of pair j at position p: p * theta^(-2j/head_dim) */
  uint32_t ffn;         /* SDEC_FFN_SWIGLU (silu(Wg n) * (Wu n)) or SDEC_FFN_GELU_ERF (gelu(W1 n)) */
  uint32_t layer_scale; /* nonzero: residual adds are x += ls (*) branch ([mimi] MV_LS) */
  uint32_t final_norm;  /* nonzero: the output is norm(x) with the final weights, else x itself */
  uint32_t window;      /* a key at position p is legal for the query at pos iff
                           p <= pos and pos - p < window ([mimi] attn_src); 1 <= window <= ring */
  uint32_t unbounded;   /* nonzero: the stack refuses pos >= ring_slots instead of wrapping
                           (the talker's cache and the FlowLM ring); requires window == ring */
  uint32_t flags;       /* SDEC_FLAG_* */
  uint32_t max_prefill; /* positions one sdec_prefill call may carry: 0 or 1 = none beyond a
                           single step, at most 16; above 1 the stack must have m == 1, and
                           max_prefill (rounded up to a power of two) * d_model floats must fit
                           64 KiB ([talker] TalkerGpu::load: max_m bounds the prefill block
                           width) */
} sdec_config;

/* One layer's parameters: device pointers, float32, borrowed (the caller keeps them alive and
 * unchanged until sdec_destroy; the library never copies or frees them).  Matrices are
 * row-major [n_out, k] ([talker] MATVEC_SRC: W stored [n,k], no transpose), 16-byte aligned.
 * A field the configuration does not use may be NULL. */
typedef struct sdec_layer_weights {
  const float* attn_norm_w; /* [d_model] pre-attention norm gain */
  const float* attn_norm_b; /* [d_model] LayerNorm bias (NORM_LAYER only) */
  const float* wq;          /* [n_q_heads*head_dim, d_model] */
  const float* wk;          /* [n_kv_heads*head_dim, d_model] */
  const float* wv;          /* [n_kv_heads*head_dim, d_model]; a packed in_proj [q;k;v] passes
                               in_proj, in_proj + qw*d, in_proj + (qw+kw)*d ([mimi] rope_push_src) */
  const float* wo;          /* [d_model, n_q_heads*head_dim] */
  const float* q_norm;      /* [head_dim] (qk_norm only) */
  const float* k_norm;      /* [head_dim] (qk_norm only) */
  const float* ls1;         /* [d_model] LayerScale of the attention branch (layer_scale only) */
  const float* ffn_norm_w;  /* [d_model] */
  const float* ffn_norm_b;  /* [d_model] (NORM_LAYER only) */
  const float* w_gate;      /* [d_ff, d_model] (SwiGLU only) */
  const float* w_up;        /* [d_ff, d_model]: SwiGLU up projection, or the GELU FFN's W1 */
  const float* w_down;      /* [d_model, d_ff] */
  const float* ls2;         /* [d_model] LayerScale of the FFN branch (layer_scale only) */
} sdec_layer_weights;

typedef struct sdec_final_weights {
  const float* norm_w; /* [d_model] (final_norm only) */
  const float* norm_b; /* [d_model] (final_norm with NORM_LAYER only) */
} sdec_final_weights;

typedef struct sdec_handle sdec_handle;

/* Build a stack: validate the configuration, allocate the K/V rings ([m][n_layers][ring_slots]
 * [n_kv_heads][head_dim] float32 each, zeroed), one position ring per stream ([m][ring_slots]
 * uint32, every slot 0xFFFFFFFF = empty, [mimi] INVALID_POS), the scratch buffers, and record
 * the per-token launch sequence as a hipGraph.  `layers` points to n_layers structs (host
 * memory, read during the call).  Synchronous; *out is set only on success. */
int sdec_create(const sdec_config* cfg, const sdec_layer_weights* layers,
                const sdec_final_weights* final_weights, uint32_t ring_slots,
                sdec_handle** out);

/* One decode step of every stream at position `pos` ([talker] TalkerGpu::step; [mimi] the
 * per-frame (pos, first) uniform).  x: device [m][d_model] float32, read as the step's input
 * rows and overwritten in place with the output rows (the final-norm hidden state, or the
 * residual stream when the stack has no final norm).  first != 0 starts fresh streams: every
 * position ring is invalidated before the step.  With first == 0, pos must equal the previous
 * step's pos + 1 (or the position set by sdec_set_next_position).  Asynchronous: enqueues on
 * `stream` and returns; x must stay valid until the work completes. */
int sdec_step(sdec_handle* h, float* x, uint32_t pos, uint32_t first, void* stream);

/* Cached prefill of a block of t consecutive positions pos .. pos+t-1 of a single-stream stack
 * ([talker] TalkerGpu::prefill and forward_rows: the block's K/V rows are appended to the cache,
 * every row attends causally to the cache and to the earlier rows of the block, and every row's
 * output is returned).  x: device [t][d_model] float32 input rows, overwritten with the t output
 * rows.  The result equals t sdec_step calls at pos, pos+1, ... (first applies to the first of
 * them).  Requires m == 1 and 1 <= t <= max_prefill (SDEC_E_ARG); that no row's push evicts a
 * position an earlier row of the block attends: pos + t <= ring_slots (nothing is evicted) or
 * ring_slots >= window + t - 1; and for an unbounded stack pos + t <= ring_slots
 * (SDEC_E_CAPACITY).  Launches kernels one by one (no
 * graph); asynchronous on `stream`.  Taps are not written. */
int sdec_prefill(sdec_handle* h, float* x, uint32_t pos, uint32_t t, uint32_t first, void* stream);
/* Fresh session on `stream`: zero the K/V rings, set every position-ring slot to empty and
 * forget the next position ([mimi] MimiGpu::reset; [pocket] PocketCodecGpu::reset). */
int sdec_reset(sdec_handle* h, void* stream);

/* Release every buffer the library owns and the graph.  Synchronizes the device first.
 * NULL is accepted.  (The pages' GPU objects own the device buffers their constructor allocates
 * -- [talker] TalkerGpu::load, [mimi] MimiGpu::new -- and release them when dropped; this is that
 * release, made explicit for a C caller.) */
void sdec_destroy(sdec_handle* h);

/* Which step path the handle runs: 0 = the per-layer launches recorded once as a hipGraph and
 * replayed per step ([talker] StepPlan: the plan is built once and replayed per token), 1 = the
 * same launches enqueued one by one (SDEC_FLAG_EAGER).  attention: how the last step's ring
 * attention ran -- 0 items over chunks of the compacted legal slots, 1 inside the o-projection
 * launch (at most 21 legal slots), 2 several streams (legal slots dealt to a fixed number of
 * items).  Every form computes the masked attention of [talker] StepPlan / [mimi] attn_src; they
 * differ only in how the work is split.  path and attention may be NULL. */
int sdec_status(sdec_handle* h, uint32_t* path, uint32_t* attention);

/* Message of the last failed call on this thread ("" if none).  Valid until the next call.
 * The pages return errors as a Result carrying the text of the failed check ([talker]
 * TalkerGpu::step's ensure! on the embedding length, the position and the cache capacity;
 * [pocket] PocketBackboneGpu::step); here the code is the return value and the text is kept
 * here. */
const char* sdec_last_error(void);

/* Device pointers of stream `stream_idx`'s rings for `layer`: *k and *v are [ring_slots]
 * [n_kv_heads][head_dim] float32 (keys already roped), *pos_ring is [ring_slots] uint32 and is
 * shared by every layer of the stream.  Writing them imports a cache ([pocket] load_voice: the
 * [positions][heads][head_dim] cache layout is the ring's slot-major layout); follow with
 * sdec_set_next_position.  A position may be stamped in at most one slot (the library's own
 * pushes use slot pos mod ring_slots): the step sizes its attention work from the number of
 * distinct positions the window can hold.  Any output pointer may be NULL. */
int sdec_kv_view(sdec_handle* h, uint32_t stream_idx, uint32_t layer, float** k, float** v,
                 uint32_t** pos_ring);

/* Declare the position the next step (with first == 0) must carry, after an import through
 * sdec_kv_view ([pocket] load_voice sets the clock to the imported length). */
int sdec_set_next_position(sdec_handle* h, uint32_t next_pos);

/* Stage taps ([pocket] PocketCodecGpu::debug_read and [mimi] MimiGpu::debug_read read a named
 * intermediate buffer back for stage-level parity).
 * With SDEC_FLAG_TAPS: device pointer of a per-layer branch output of the latest step,
 * [m][width] float32.  which = 0: attention output before the o projection (width
 * n_q_heads*head_dim); 1: o projection output before LayerScale and the residual add;
 * 2: FFN down projection output before LayerScale and the residual add (width d_model). */
int sdec_tap_view(sdec_handle* h, uint32_t layer, uint32_t which, float** ptr);

/* Per-kernel timing of one eager step: runs the step like sdec_step (same checks, same state
 * update) with a hipEvent pair around every launch, waits for it, and adds each launch's
 * milliseconds into ms[kind] and 1 into calls[kind] (kind = SDEC_K_*; arrays of SDEC_K_COUNT). */
enum {
  SDEC_K_BEGIN = 0,     /* input copy, position-ring stamp, this position's rope cos/sin */
  SDEC_K_QKV = 1,       /* pre-attention norm + q/k/v projections */
  SDEC_K_ATTENTION = 2, /* qk-norm + rope + ring push + ring attention */
  SDEC_K_O = 3,         /* o projection + (LayerScale) residual */
  SDEC_K_FFN_UP = 4,    /* pre-FFN norm + gate/up (SwiGLU) or W1 (GELU) projection */
  SDEC_K_FFN_DOWN = 5,  /* down projection + (LayerScale) residual */
  SDEC_K_END = 6,       /* final norm, or copy of the residual stream, into x */
  SDEC_K_COUNT = 7
};
int sdec_step_profile(sdec_handle* h, float* x, uint32_t pos, uint32_t first, void* stream,
                      double* ms, uint32_t* calls);

/* One-shot GEMV, the step's weight-streaming kernel on its own ([talker] MATVEC_SRC):
 * y[r][i] = sum_j x[r][j] * w[i][j] for r < m (1..8), i < n, with w row-major [n][k]
 * (k a multiple of 4, w and x 16-byte aligned), x [m][k], y [m][n]; all device float32. */
int sdec_gemv(const float* w, const float* x, float* y, uint32_t n, uint32_t k, uint32_t m,
              void* stream);

/* One-shot ring attention ([mimi] attn_src with [talker] GQA_ATTN_SRC's head mapping) for m
 * streams at query position pos: q [m][n_q_heads*head_dim]; k_ring, v_ring [m][ring_slots]
 * [n_kv_heads][head_dim]; pos_ring [m][ring_slots]; out [m][n_q_heads*head_dim].  Slot j is
 * legal iff pos_ring[j] != 0xFFFFFFFF, pos_ring[j] <= pos and pos - pos_ring[j] < window; a
 * head with no legal slot gets zeros.  head_dim is 64 or 128; all device memory. */
int sdec_ring_attention(const float* q, const float* k_ring, const float* v_ring,
                        const uint32_t* pos_ring, float* out, uint32_t m, uint32_t n_q_heads,
                        uint32_t n_kv_heads, uint32_t head_dim, uint32_t ring_slots,
                        uint32_t window, uint32_t pos, void* stream);

/* sdec_ring_attention for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, kernels and result, with
 * no allocation at all.  Its scratch (legal-slot lists, per-chunk softmax partials, merge
 * counters) is a fixed 4 MiB array in device memory that each device the library runs on holds
 * until the process ends; a call whose scratch would exceed it (about m * n_q_heads *
 * ceil(ring_slots / 128) * (head_dim + 2) floats of partials plus m * (ring_slots + 1) words
 * of lists) returns SDEC_E_ARG without enqueuing anything.  Every call on a device shares that
 * device's array and keeps the last call's contents (the merge counters are cleared at the start
 * of each call by a fill kernel), so calls that overlap on one device -- on different streams
 * or threads -- race and must be serialised by the caller.  The first call on a device looks up
 * the array's address there (hipGetSymbolAddress, with that device current). */
int sdec_ring_attention_static(const float* q, const float* k_ring, const float* v_ring,
                               const uint32_t* pos_ring, float* out, uint32_t m,
                               uint32_t n_q_heads, uint32_t n_kv_heads, uint32_t head_dim,
                               uint32_t ring_slots, uint32_t window, uint32_t pos,
                               void* stream);

/* Split residual vector quantiser ([mimi] inferencelayer 0.2.1, src/mimi_gpu.rs: the NEAREST,
 * SUB_EMB and EMB_SUM kernels and MimiGpu's encode / decode plans).  A latent frame [dim] is
 * projected twice (in_first, in_rest: [vq][dim]); code 0 is the nearest bin of codebook
 * cb_first to the first projection; codes 1 .. nq-1 quantise the second projection with the
 * nq-1 rest codebooks in turn, each subtracting its chosen code vector from the running residual
 * before the next.  "Nearest" is the smallest squared distance sum_c (cb[b][c] - r[c])^2 summed
 * over c in ascending order in float32 with no fused multiply-add; ties go to the lower bin.
 * Decoding sums each group's chosen code vectors (in level order) and returns
 * out_first . sum_first + out_rest . sum_rest (out_*: [dim][vq]).  Codebooks: cb_first
 * [bins][vq], cb_rest [nq-1][bins][vq].  All weights are borrowed device pointers, 16-byte
 * aligned, unchanged until sdec_rvq_destroy; the library keeps a transposed copy of the
 * codebooks. */
typedef struct sdec_rvq_config {
  uint32_t dim;        /* latent width; multiple of 4 */
  uint32_t vq;         /* quantiser width; multiple of 64, at most 1024 */
  uint32_t bins;       /* bins per codebook; multiple of 64, at least 64 */
  uint32_t nq;         /* codebooks: 1 first + nq-1 rest; at least 2 */
  uint32_t max_frames; /* frames one call may carry; 1 .. 65535 */
} sdec_rvq_config;
typedef struct sdec_rvq_weights {
  const float* in_first;  /* [vq][dim] */
  const float* in_rest;   /* [vq][dim] */
  const float* out_first; /* [dim][vq] */
  const float* out_rest;  /* [dim][vq] */
  const float* cb_first;  /* [bins][vq] */
  const float* cb_rest;   /* [nq-1][bins][vq] */
} sdec_rvq_weights;
typedef struct sdec_rvq sdec_rvq;
/* Validate, allocate the working buffers and the transposed codebooks.  Synchronous. */
int sdec_rvq_create(const sdec_rvq_config* cfg, const sdec_rvq_weights* w, sdec_rvq** out);
/* Encode `frames` latent frames: latent device [frames][dim] float32 -> codes device
 * [frames][nq] uint32.  Asynchronous on `stream`. */
int sdec_rvq_encode(sdec_rvq* q, const float* latent, uint32_t frames, uint32_t* codes,
                    void* stream);
/* The quantiser alone, from given projections r_first, r_rest (device [frames][vq] each). */
int sdec_rvq_quantise(sdec_rvq* q, const float* r_first, const float* r_rest, uint32_t frames,
                      uint32_t* codes, void* stream);
/* Decode codes device [frames][nq] (each < bins; a larger value reads bin bins-1) into latent
 * device [frames][dim] float32.  Asynchronous on `stream`. */
int sdec_rvq_decode(sdec_rvq* q, const uint32_t* codes, uint32_t frames, float* latent,
                    void* stream);
/* Release the buffers the library owns (synchronizes the device first).  NULL is accepted. */
void sdec_rvq_destroy(sdec_rvq* q);

/* Streaming codec convolution ([mimi] inferencelayer 0.2.1, src/mimi_gpu.rs: CONV1D with the
 * input prefix carried between frames by WRITE_XA / CARRY (REPLICATE on the first frame), and
 * the gather-form transposed conv of convtr_src whose overlap tail TRP_ADD / TR_OUT / TR_CARRY
 * carry bias-subtracted; the ELU of ELU_IP can be folded into the input reads).  Frames are fed
 * one at a time; concatenated, the outputs equal the offline convolution of the concatenated
 * input:
 *   conv (transposed == 0): the input is left-padded by kernel - stride columns (zeros, or
 *     copies of the first column when replicate_first), y[o][t] = b[o] + sum_{i,k}
 *     w[o][i][k] * f(xp[i][t*stride + k]) with w [out_ch][in_ch/groups][kernel]; a frame of
 *     t_in columns (a multiple of stride) gives t_in/stride columns; accumulate adds them to y.
 *   transposed conv: w [in_ch][out_ch/groups][kernel]; a frame of t_in columns gives
 *     t_in*stride columns, the first ones of the full transposed convolution not yet emitted
 *     (the last kernel - stride wait for the next frame's overlap).
 * f is ELU (v > 0 ? v : exp(v) - 1) when pre_elu, else the identity.  groups is 1 or
 * in_ch == out_ch (channel-wise).  kernel >= stride >= 1.  Weights are borrowed device pointers.
 * x is device [in_ch][t_in], y device [out_ch][t_out] (channel-major, as the pages' buffers). */
typedef struct sdec_conv_config {
  uint32_t in_ch;
  uint32_t out_ch;
  uint32_t kernel;
  uint32_t stride;
  uint32_t groups;
  uint32_t transposed;
  uint32_t pre_elu;
  uint32_t replicate_first; /* conv only */
  uint32_t accumulate;      /* conv only: y += conv(x) */
  uint32_t max_t_in;        /* largest frame, in input columns */
} sdec_conv_config;
typedef struct sdec_conv sdec_conv;
/* The handle owns two state buffers (the carried prefix or tail, ping-pong) and, for groups == 1
 * with more than 32 input channels, a partial-sum buffer for up to 16 input-channel splits of a
 * max_t_in frame.  Errors: SDEC_E_ARG (null pointers, channels outside [1, 65535], kernel <
 * stride, groups other than 1 or channel-wise, max_t_in == 0, replicate_first / accumulate on a
 * transposed conv), SDEC_E_NOMEM. */
int sdec_conv_create(const sdec_conv_config* cfg, const float* w, const float* b, sdec_conv** out);
/* One frame.  first != 0 starts a fresh stream (the carried state is ignored).  Asynchronous.
 * Errors (checked before anything is enqueued): SDEC_E_ARG for a null x / y, t_in outside
 * [1, max_t_in] or (conv) not a multiple of stride; SDEC_E_POS for a first frame without first;
 * SDEC_E_HIP for a failed launch.  Steps of one handle must not overlap (they share its state). */
int sdec_conv_step(sdec_conv* c, const float* x, uint32_t t_in, float* y, uint32_t first,
                   void* stream);
/* Release the handle's buffers (synchronizes the device first).  NULL is accepted. */
void sdec_conv_destroy(sdec_conv* c);

/* Layout change between the convolutions' channel-major buffers and the transformer's time-major
 * rows ([pocket] PocketCodecGpu::new: a channel-major to time-major pass before the codec
 * transformer and the reverse pass after it).  x is device [rows][cols] float32, y device
 * [cols][rows]: y[c][r] = x[r][c].  The two buffers must not overlap.  Asynchronous on `stream`.
 * Errors (nothing is enqueued): SDEC_E_ARG for a null pointer, rows or cols == 0, cols above
 * 2096640, or overlapping buffers; SDEC_E_HIP for a failed launch. */
int sdec_transpose(const float* x, uint32_t rows, uint32_t cols, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDEC_H */
