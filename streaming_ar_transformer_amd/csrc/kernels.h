// Internal interface between the C-ABI host code (sdec.cpp) and the HIP kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdec {

constexpr uint32_t kInvalidPos = 0xFFFFFFFFu;
constexpr int kMaxM = 8;
// Rows of one prefill block (a single stream's consecutive positions); blocks above kMaxM rows
// take the 16-row GEMV shapes.
constexpr int kMaxPrefill = 16;
constexpr int kWgThreads = 256;  // four wave64s

// Per-step device state written by the step-begin kernel and read by the layer kernels, so a
// recorded graph stays valid for every position.
struct DevState {
  uint32_t pos;
  uint32_t slot;
  float* x_out;  // the caller's output rows of this step
};

// PRO_ATTN: the input row is this step's attention output, combined in the prologue from the
// per-chunk softmax partials the ring-attention launch left (one stream only).
// PRO_ATTN_SHORT: the input row is this step's attention output, computed inside the launch from
// the raw q/k/v and the ring by waves of its own (one stream, at most kShortSlots legal slots).
enum GemvPrologue : int { PRO_NONE = 0, PRO_RMS = 1, PRO_LN = 2, PRO_ATTN = 3, PRO_ATTN_SHORT = 4 };
constexpr uint32_t kShortSlots = 21;         // legal slots (the pushed one included) of PRO_ATTN_SHORT
constexpr uint32_t kAttnMaxChunks = 64;      // chunks a PRO_ATTN prologue combines
constexpr uint32_t kAttnMaxPartials = 1024;  // heads x chunks a PRO_ATTN prologue combines
constexpr uint32_t kAttnMaxHeads = 16;       // query heads a PRO_ATTN prologue combines
enum GemvEpilogue : int { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2, EPI_GELU = 3 };

// PRO_ATTN_SHORT: what the attention needs ([talker] QK_NORM_SRC, ROPE_SRC, APPEND_SRC and
// GQA_ATTN_SRC; [mimi] rope_push_src and attn_src).  The legal-slot list holds the pushed slot
// first; at most kShortSlots entries are read.
struct ShortAttnArgs {
  const float* qkv;          // this step's raw q (Hq*hd), then k (Hkv*hd), then v (Hkv*hd)
  const float* q_norm;       // [hd] or null (no qk-norm)
  const float* k_norm;
  float eps;
  int rope_style;            // 0 rotate_half, 1 interleaved
  const float* cs;           // [hd/2] cos then [hd/2] sin of this position
  float* k_ring;             // this layer's rings [R][Hkv][hd]
  float* v_ring;
  const uint32_t* legal;     // [R]: the slots this step attends, the pushed slot first
  const uint32_t* n_legal;
  const DevState* st;        // slot of this step's push
  uint32_t n_q_heads, n_kv_heads, ring;
  int early_rows;            // GEMV tile rows requested before the ring rows are in (tuning)
};

// y = x . W^T over up to three row segments (q, k, v share one launch).  With EPI_SWIGLU the
// launch covers `n_rows` FFN indices, reading rows of w[0] (gate) and w[1] (up).
struct GemvArgs {
  const float* w[3];
  uint32_t seg_end[3];  // cumulative row counts of the segments
  uint32_t n_rows;
  uint32_t k;
  uint32_t m;            // valid input rows (streams)
  const float* x;        // [m][x_stride]
  uint32_t x_stride;
  const float* norm_w;   // prologue gain
  const float* norm_b;   // prologue bias (LayerNorm)
  float eps;
  float* y;              // EPI_STORE / EPI_SWIGLU / EPI_GELU output, [m][y_stride]
  uint32_t y_stride;
  float* res;            // EPI_RESIDUAL target, [m][res_stride]
  const DevState* res_st;  // non-null (register and generic kernels): the target is res_st->x_out,
                           // the caller's output rows recorded by the step begin
  uint32_t res_stride;
  const float* res_in;   // EPI_RESIDUAL source of the old residual (null: `res`, in place)
  const float* ls;       // LayerScale or null
  float* tap;            // optional copy of the raw branch, [m][tap_stride]
  uint32_t tap_stride;
  // PRO_ATTN: chunk partials -- unnormalised outputs [k / head_dim heads][n_chunks][head_dim], then
  // (chunk max, chunk sum) pairs [heads][n_chunks][2] -- and the legal-slot count that sets how
  // many chunks hold data; with a single chunk the attention output is read from x as usual
  const float* part;
  const uint32_t* n_legal;
  uint32_t chunk, n_chunks, head_dim;
  float* x_tap;          // PRO_ATTN, PRO_ATTN_SHORT: optional copy of the combined input row
  ShortAttnArgs sa;      // PRO_ATTN_SHORT
};

struct GemvLaunch {
  int prologue;
  int epilogue;
  int rows_per_wave;  // R: rows one wave reduces together
  int kb;             // >0: k == 256*kb and the input rows live in registers; 0: generic k
  int ks;             // >0: split-k kernel, k == 1024*ks (each wave takes a quarter of each row)
  int stream;         // 1: row-stream kernel (one row per wave in flight), k == 256*kb
  int waves_per_wg;
  uint32_t grid;      // workgroups; each wave owns a contiguous, balanced range of row tiles
  int attn_hd, attn_g, attn_hpw;  // PRO_ATTN_SHORT: head_dim, GQA group, kv heads per wave
};

hipError_t launch_gemv(const GemvArgs& a, const GemvLaunch& l, hipStream_t s);
// A launch shape for this GEMV on this device (grid sized to the row tiles).
GemvLaunch plan_gemv(int prologue, int epilogue, uint32_t n_rows, uint32_t k, uint32_t m);
// The short-context attention + o projection launch (PRO_ATTN_SHORT, one stream, n_kv_heads a
// multiple of 4); gemv_supported tells whether a kernel exists for it.
GemvLaunch plan_attn_short_o(uint32_t n_rows, uint32_t k, uint32_t head_dim, uint32_t n_q_heads,
                             uint32_t n_kv_heads);
// Whether a kernel exists for this launch shape.
bool gemv_supported(const GemvLaunch& l, uint32_t k, uint32_t m);
// Per-kernel timing: while a pair is set (null to clear), the step-kernel launches of this thread
// (GEMV, attention, begin, end) stamp `start` and `stop` around their own execution.
void set_launch_events(hipEvent_t start, hipEvent_t stop);

// Ring attention of one layer for every stream.  In the step it also finishes the new position:
// qk-RMSNorm and rope of this step's q and k (from the raw q/k/v projection), and the push of the
// roped k and raw v into ring slot st->slot by the workgroup whose slot chunk holds that slot.
struct AttnArgs {
  const float* qkv;      // [m][qkv_stride]: raw q (Hq*hd), then k (Hkv*hd), then v (Hkv*hd)
  uint32_t qkv_stride;
  const float* q_norm;   // [hd] or null (no qk-norm)
  const float* k_norm;
  float eps;
  int rope_style;        // 0 rotate_half, 1 interleaved
  const float* cs;       // [hd/2] cos then [hd/2] sin of this position; null: q used as given
  uint32_t cs_stride;    // floats between the tables of consecutive streams (0: one shared table)
  int push;              // nonzero: push this step's k/v into the rings
  float* k_ring;         // stream 0 of this layer: [R][Hkv][hd]
  float* v_ring;
  uint64_t ring_stream_stride;  // floats between consecutive streams' rings
  const uint32_t* legal;        // [m][R] slots this step may attend (the pushed slot first)
  const uint32_t* n_legal;      // [m]
  float* out;            // [m][Hq*hd]
  float* part;           // [m][Hq][n_chunks][hd + 2] chunk partials
  uint32_t* counters;    // [m][Hkv], zero between launches (the last chunk resets it)
  uint32_t m, n_q_heads, n_kv_heads, head_dim, ring, chunk, n_chunks;
  const DevState* st;    // slot of this step's push; null: no push
  int partials_only;     // nonzero: with more than one item, every item leaves its chunk
                         // partial (plain stores) and the consumer of `out` combines them
  int split;             // nonzero: each stream's legal slots are dealt round-robin to n_chunks
                         // items (chunk unused), at most kAttnSplitList per item
};
// Most legal slots one item of a split attention launch takes (its slot list lives in LDS).
constexpr uint32_t kAttnSplitList = 1024;
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// The legal-slot lists of m streams for a query at `pos` (ascending slot order), for the one-shot
// attention entry point.
hipError_t launch_compact_legal(const uint32_t* pos_rings, uint32_t m, uint32_t ring, uint32_t pos,
                                uint32_t window, uint32_t* legal, uint32_t* n_legal, hipStream_t s);
uint32_t attention_chunk(uint32_t head_dim);

struct BeginArgs {
  const float* x_in;     // caller rows [m][d]
  float* x_out;          // where the step's output rows go (recorded in DevState)
  float* xres;           // residual stream [m][d]
  uint32_t d;
  uint32_t* pos_rings;   // [m][R]
  uint32_t* legal;       // [m][R] out: the slots this step attends, the new slot first
  uint32_t* n_legal;     // [m]
  uint32_t m, ring, window;
  uint32_t pos, first;
  float* cs;             // [hd/2] cos, [hd/2] sin
  uint32_t head_dim;
  double theta;
  DevState* st;
};
hipError_t launch_begin(const BeginArgs& a, hipStream_t s);
// One stream: the first layer's q/k/v projection (row-stream kernel, x = the caller's row) and the
// step begin in one launch.
struct QkvBeginArgs {
  GemvArgs g;
  BeginArgs b;
  uint32_t gemv_wgs;  // the projection's workgroups (the launch plan's grid)
};
bool qkv_begin_supported(const GemvLaunch& l);
hipError_t launch_qkv_begin(const QkvBeginArgs& a, const GemvLaunch& l, hipStream_t s);
// Multi-position begin ([talker] TalkerGpu::prefill / forward_rows): the m rows are positions
// pos .. pos+m-1 of ONE stream whose position ring is pos_rings[0..R).  Stamps every row's slot
// first, then forms row i's legal list (its own slot first) and its rope cos/sin (cs + i*head_dim).
// Needs pos + m <= R or R >= window + m - 1, so no row's push overwrites a slot an earlier row
// still attends.
hipError_t launch_begin_rows(const BeginArgs& a, hipStream_t s);

// Key/value push of m rows at positions pos .. pos+m-1 of one stream ([talker] forward_rows: the
// block's K/V rows are appended before attention): per row and kv head, the raw key gets the
// per-head RMSNorm (if any) and rope with that row's cos/sin, and key and value are written into
// ring slot (pos + row) mod R.
struct PushArgs {
  const float* qkv;      // [m][qkv_stride] raw q, k, v
  uint32_t qkv_stride;
  const float* k_norm;   // [hd] or null
  float eps;
  int rope_style;
  const float* cs;       // [m][hd]: cos then sin per row
  float* k_ring;         // this layer's rings [R][Hkv][hd]
  float* v_ring;
  uint32_t m, n_q_heads, n_kv_heads, head_dim, ring, pos;
};
hipError_t launch_push(const PushArgs& a, hipStream_t s);

struct EndArgs {
  const float* xres;     // [m][d]
  float* x_out;          // [m][d]; null: the rows DevState::x_out names (set by the step begin)
  const DevState* st;
  uint32_t m, d;
  int norm;              // -1: copy, PRO_RMS or PRO_LN
  const float* w;
  const float* b;
  float eps;
};
hipError_t launch_end(const EndArgs& a, hipStream_t s);

// Split RVQ (rvq.hip; [mimi] NEAREST, SUB_EMB, EMB_SUM).  One quantiser level for every frame:
// optionally resolve the previous level's code from its per-wave candidates (and write it), then
// optionally subtract that code's vector from the running residual (prev_cb), then let every
// wave of 64 bins leave its first-wins candidate (distance, bin).
constexpr int kRvqMaxVq = 1024;
struct RvqLevelArgs {
  const float* cbT;            // this level's codebook, transposed [vq][bins]
  const float* r_in;           // [frames][r_stride] residual entering the level
  uint32_t r_stride;
  float* r_out;                // [frames][vq] the residual this level quantises (null: not kept)
  const float* prev_cb;        // previous level's codebook rows [bins][vq]: subtract its code
  const float* prev_cand_d;    // previous level's candidates [frames][groups] (null: none)
  const uint32_t* prev_cand_i;
  uint32_t prev_level;         // code index of the previous level
  float* cand_d;               // this level's candidates [frames][groups]
  uint32_t* cand_i;
  uint32_t* codes;             // [frames][nq]
  uint32_t nq, bins, vq, groups;
};
struct RvqEmbArgs {
  const uint32_t* codes;       // [frames][nq]
  const float* cb_first;       // [bins][vq]
  const float* cb_rest;        // [nq-1][bins][vq]
  float* acc;                  // [frames][2][vq]: first-group sum, rest-group sum
  uint32_t nq, bins, vq;
};
// [levels][bins][vq] -> [levels][vq][bins] (rvq.hip).
hipError_t launch_transpose(const float* src, float* dst, uint32_t levels, uint32_t bins,
                            uint32_t vq, hipStream_t s);
hipError_t launch_rvq_level(const RvqLevelArgs& a, uint32_t frames, hipStream_t s);
hipError_t launch_rvq_final(const RvqLevelArgs& a, uint32_t frames, hipStream_t s);
hipError_t launch_rvq_emb_sum(const RvqEmbArgs& a, uint32_t frames, hipStream_t s);

// Streaming codec convolutions (conv.hip; [mimi] CONV1D, convtr_src, the prefix and tail carries).
struct SConvArgs {
  const float* w;          // [c_out][c_in / groups][k]
  const float* b;          // [c_out]
  const float* x;          // [c_in][t_in] this frame
  const float* prefix;     // [c_in][pad] carried input columns (pad = k - stride)
  float* prefix_out;       // [c_in][pad] the next frame's prefix
  float* y;                // [c_out][t_in / stride]
  uint32_t c_in, c_out, k, stride, groups, t_in, pad;
  int pre_elu, replicate_first, first, accumulate;
  float* part;             // split-k partial sums [splits][c_out][t_in / stride] (groups == 1)
  uint64_t part_cap;       // floats part holds (0: no split)
  uint32_t* counters;      // per output tile: splits finished (zero between launches)
  uint32_t counter_cap;    // tiles the counters cover (0: a separate launch sums the splits)
};
hipError_t launch_sconv(const SConvArgs& a, hipStream_t s);
struct SConvTrArgs {
  const float* w;          // [c_in][c_out / groups][k]
  const float* b;          // [c_out]
  const float* x;          // [c_in][t_in]
  const float* tail;       // [c_out][tl] carried pending columns, bias subtracted (tl = k - stride)
  float* tail_out;         // [c_out][tl]
  float* y;                // [c_out][t_in * stride]
  uint32_t c_in, c_out, k, stride, groups, t_in, tl;
  int pre_elu, first;
  float* part;             // split-k partial sums [splits][c_out][t_in * stride + tl] (groups == 1)
  uint64_t part_cap;       // floats part holds (0: no split)
  uint32_t* counters;      // per output tile: splits finished (zero between launches)
  uint32_t counter_cap;    // tiles the counters cover (0: a separate launch sums the splits)
};
// Most input-channel splits a streaming conv launch uses (its partial-sum scratch is sized for it).
constexpr uint32_t kConvMaxSplits = 16;
hipError_t launch_sconvtr(const SConvTrArgs& a, hipStream_t s);

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, uint64_t n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float value, uint64_t n, hipStream_t s);

}  // namespace sdec
