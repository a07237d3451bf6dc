// Launch interfaces between the host API (oscar_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

// decode ticket counters: one per (sequence, KV head), each on its own 128-byte line
constexpr int kCounterStride = 32;

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
  int32_t units_per_head;    // n_bf16_units + max_chunks
  float sm_log2;             // softmax scale * log2(e)
};

// Returns false if the (head_dim, n_groups, gqa) combination has no kernel.
bool launch_decode(const DecodeParams& p, int head_dim, int n_groups, int gqa, bool bf16_only, int grid,
                   hipStream_t stream);

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
};
bool launch_append_demote(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream);
bool launch_quantize_pack(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream);
// BF16 page prefill: num_tokens tokens of k / v to positions first_position + t
// through bf16_pt (one sequence)
bool launch_write_bf16(const WriteParams& p, int head_dim, int first_position, hipStream_t stream);

}  // namespace oscar
