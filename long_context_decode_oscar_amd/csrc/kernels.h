// Launch interfaces between the host API (oscar_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

// decode ticket counters: one per (sequence, KV head), each on its own 128-byte line
constexpr int kCounterStride = 32;

// Prefix-shared ("cascade") decode: a unit is up to 16 / GQA consecutive
// sequences whose INT2 page tables share their first `shared_pages` logical
// history pages.  One launch of prefix workgroups attends those pages once
// for all the unit's queries (chunk c of the unit's range writes partial slot
// n_bf16_units + own chunks of the member + c of every member); the decode
// launch that follows covers each sequence's own history from page
// shared_pages on and merges the prefix partials in.
constexpr int kMaxCascUnits = 32;
struct CascUnit {
  int32_t first, count;      // member sequences first .. first + count - 1
  int32_t shared_pages;      // shared logical history pages [0, shared_pages)
  int32_t chunks;            // prefix chunks of the unit (per KV head)
  int32_t pages_per_chunk;   // even
  int32_t wg_start;          // first prefix workgroup of the unit
};

// Length-aware ("packed") split-K plans are passed in the kernel arguments
// for batches of up to this many sequences.
constexpr int kMaxPackedSeqs = 128;

struct DecodeParams {
  const uint16_t* q;         // [B][Hq][D] bf16
  const int32_t* seq_lens;   // [B]
  const int32_t* bf16_pt;    // [B][bf16_pt_stride]
  const int32_t* int2_pt;    // [B][int2_pt_stride]
  const uint8_t* bf16_pool;
  const uint8_t* int2_pool;
  const float* r_k;          // [Hkv][D][D]
  const float* r_v;          // [Hkv][D][D], or null when V is absorbed
  uint16_t* out;             // [B][Hq][D] bf16
  uint32_t* counters;        // [B][Hkv], kCounterStride words apart
  float* part_lse;           // [B][Hkv][U][GQA] log2 of the partial's softmax sum
  float* part_o;             // [B][Hkv][U][GQA][D]
  int32_t bf16_pt_stride, bf16_num_pages;
  int32_t int2_pt_stride, int2_num_pages;
  int32_t batch, num_kv_heads, sink, recent;
  int32_t max_len;           // lengths above it are clamped to it
  int32_t n_bf16_units;      // BF16 (sink + recent) units per (sequence, KV head)
  int32_t bf16_pages_per_unit;
  int32_t max_chunks;        // INT2 (or, BF16-only, BF16) chunks per (sequence, KV head)
  int32_t pages_per_chunk;
  int32_t units_per_head;    // workgroups per (sequence, KV head): n_bf16_units + max_chunks
  int32_t slots_per_head;    // partial slots per (sequence, KV head): units_per_head + max prefix chunks
  float sm_log2;             // softmax scale * log2(e)
  int32_t lut;               // 1: four-level codebook
  uint32_t lut_k;            // byte c: 32 L_K[c] (int8 score operand of code c)
  uint32_t lut_v;            // byte c: 64 L_V[c] (mantissa of the fp16 operand 16 + L_V[c])
  int32_t n_casc;            // prefix-shared units (0: plain decode)
  uint64_t* stamps;          // phase timeline of the profiling build (null otherwise)
};

// Profiling build (-DOSCAR_PHASE_STAMPS=1): the plain decode records, per
// wave, kStampSlots real-time counter values (100 MHz) for workgroups below
// kStampWgs, in the last kStampBytes of the caller's workspace.
#ifndef OSCAR_PHASE_STAMPS
#define OSCAR_PHASE_STAMPS 0
#endif
constexpr int kStampSlots = 16;
constexpr int kStampWgs = 2048;
constexpr int kStampWaves = 8;
constexpr size_t kStampBytes = (size_t)kStampWgs * kStampWaves * kStampSlots * sizeof(uint64_t);

// The prefix-shared units of a decode with prefix groups: a separate kernel
// argument of the instantiations that take prefix groups (the plain launch
// keeps its argument block small: each launch copies it).
struct CascArgs {
  CascUnit unit[kMaxCascUnits];
};

// The length-aware plan's tables, a separate kernel argument of the packed
// kernel instantiations only (the plain launch keeps its small argument
// block).  Sequence b owns workgroups [wg_off[b], wg_off[b+1])
// (num_kv_heads x its units, KV head major) and partial slots
// [slot_off[b], slot_off[b+1]) (num_kv_heads x its slots: its units, then its
// prefix chunks).  Without it every (sequence, KV head) has units_per_head
// workgroups and slots_per_head slots.
struct PackedPlanArgs {
  int32_t wg_off[kMaxPackedSeqs + 1];
  int32_t slot_off[kMaxPackedSeqs + 1];
};

// Returns false if the (head_dim, n_groups, gqa) combination has no kernel.
// packed: the length-aware plan's tables (null: the uniform plan).
// casc: the prefix-shared units (p.n_casc of them; null when p.n_casc = 0).
bool launch_decode(const DecodeParams& p, const CascArgs* casc, const PackedPlanArgs* packed, int head_dim,
                   int n_groups, int gqa, bool bf16_only, int grid, hipStream_t stream);
// The prefix workgroups of the units in casc (grid = sum of Hkv * chunks
// over units).
bool launch_decode_prefix(const DecodeParams& p, const CascArgs& casc, const PackedPlanArgs* packed, int head_dim,
                          int n_groups, int gqa, int grid, hipStream_t stream);

struct MergeParams {
  int32_t rows, head_dim;
  const int32_t* row_offsets;
  const float* o;
  const float* lse;
  uint16_t* out;
};
bool launch_merge(const MergeParams& p, hipStream_t stream);

struct WriteParams {
  // append + demote
  const uint16_t* k_new;     // [B][Hkv][D]
  const uint16_t* v_new;
  const int32_t* seq_lens;   // [B], length before the append
  const int32_t* bf16_pt;
  const int32_t* int2_pt;
  uint8_t* bf16_pool;
  uint8_t* int2_pool;
  int32_t bf16_pt_stride, bf16_num_pages, int2_pt_stride, int2_num_pages;
  // bulk
  const uint16_t* k;         // [T][Hkv][D]
  const uint16_t* v;
  const int32_t* page_ids;   // [ceil(T/16)]
  int32_t num_tokens;
  int32_t pages_per_block;
  // common
  const float* r_k;          // [Hkv][D][D]
  const float* r_v;          // [Hkv][D][D], or null when V is absorbed
  const float* tau_k;        // [Hkv]
  const float* tau_v;
  int32_t batch, num_kv_heads, sink, recent;
  int32_t lut;               // 1: four-level codebook, codes by the thresholds below
  float thr_k[3], thr_v[3];  // midpoints of consecutive levels
};
bool launch_append_demote(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream);
bool launch_quantize_pack(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream);
// BF16 page prefill: num_tokens tokens of k / v to positions first_position + t
// through bf16_pt (one sequence)
bool launch_write_bf16(const WriteParams& p, int head_dim, int first_position, hipStream_t stream);

// ---- offline calibration and the rotation error chain (calib.hip) ----

// out[h] = scale * X[h]^T X[h], X[h] row r at x + h*head_stride + r*row_stride
struct GramParams {
  const float* x;
  int64_t head_stride, row_stride;  // elements
  int32_t heads, rows;
  int32_t rows_per_split, splits;   // rows_per_split a multiple of 16
  float scale;
  float* part;                      // [splits][heads][D][D] partial sums
  float* out;                       // [heads][D][D]
};
bool launch_gram(GramParams p, int dim, hipStream_t stream);

struct CalibAttnParams {
  const float* q;                   // [kv_heads][gqa][tokens][D]
  const float* k;                   // element (h, n, c) at h*kv_hs + n*kv_ns + c
  const float* v;
  const float* k_hat;               // error chain: quantized keys / values,
  const float* v_hat;               // same strides
  float* out;                       // attention: [kv_heads][gqa][tokens][D]
  float* lse;                       // attention: [kv_heads][gqa][tokens] or null
  float* stats;                     // error chain: [kv_heads][gqa][tokens][4]
  int64_t kv_hs, kv_ns;
  int32_t kv_heads, gqa, tokens;
  float scale_log2;                 // softmax scale * log2(e)
};
bool launch_calib_attention(const CalibAttnParams& p, int dim, bool err, hipStream_t stream);

// Workgroup h < split takes matrix h of cov / r_out / eigvals, workgroup
// h >= split matrix h - split of cov2 / r_out2 / eigvals2 (two sets of
// matrices in one launch).
struct EigParams {
  const float* cov;                 // [split][D][D] symmetric
  float* r_out;                     // [split][D][D]
  float* eigvals;                   // [split][D] descending, or null
  const float* cov2;                // [heads - split][D][D] (if heads > split)
  float* r_out2;
  float* eigvals2;
  int32_t heads, split, mix;        // mix: R = U H P_br, else R = U
};
bool launch_eigen_rotation(const EigParams& p, int dim, hipStream_t stream);

struct ClipParams {
  const float* x;                   // row r of head h at x + h*head_stride + r*row_stride
  int64_t head_stride, row_stride;
  int32_t heads, rows, dim;
  const float* r;                   // [heads][D][D] or null (no rotation)
  uint32_t* keys;                   // [heads][rows*D] workspace
  uint32_t* hist;                   // [heads][chunks][2][256] workspace
  uint32_t* sel;                    // [heads][2][2] workspace
  float* tau;                       // [heads]
  int32_t chunks;
  uint32_t rank_lo, rank_hi;        // 0-based ranks of the two order statistics
  double frac;                      // interpolation weight between them
};
bool launch_clip(const ClipParams& p, hipStream_t stream);

// Four-level codebook fit: normalized values of x R (clipped to tau, per
// group of group_size channels) into t, then Lloyd iterations.
struct CodebookParams {
  const float* x;                   // row r of head h at x + h*head_stride + r*row_stride
  int64_t head_stride, row_stride;
  int32_t heads, rows, dim, group_size;
  const float* r;                   // [heads][D][D] or null
  const float* tau;                 // [heads] device
  float* t;                         // [heads][rows][D] workspace
  double* partial;                  // [chunks][4] workspace
  double* state;                    // [4] workspace: current levels
  float* levels;                    // [4] result
  int32_t chunks;
};
bool launch_codebook(const CodebookParams& p, int iterations, hipStream_t stream);

struct DequantParams {
  const int32_t* page_ids;          // [ceil(num_tokens / 16)]
  const uint8_t* int2_pool;
  const float* r;                   // [Hkv][D][D] rotation to undo, or null
  float* out;                       // [num_tokens][Hkv][D]
  int32_t num_tokens, int2_num_pages, num_kv_heads;
  int32_t which;                    // 0: keys, 1: values
  float levels[4];                  // code -> level in code units (0, 1, 2, 3 when uniform)
};
bool launch_dequantize(const DequantParams& p, int dim, int n_groups, hipStream_t stream);

}  // namespace oscar
