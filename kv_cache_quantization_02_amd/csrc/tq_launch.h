// tq_launch.h -- argument blocks passed by value to the kernels, and the
// host-side launchers each kernel file exports to the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"

namespace tq {

// Row r in [0, rows) is (s, t, h) with r = (s * n_tok + t) * n_head + h.
struct RowSplit {
  FastDiv div_head;  // divides by n_head
  FastDiv div_tok;   // divides by n_tok
};

struct QuantArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int8_t* signs;
  uint8_t* k_q;
  uint16_t* k_scale;
  uint16_t* k_zero;
  uint8_t* v_q;
  uint16_t* v_scale;
  uint32_t rows;
  RowSplit split;
  RowMap in, out;
  // Append into a cache: when out_pos is set, row (s, t, h) is written to
  // out-row (s, out_pos[s] + t, h), and only when 0 <= out_pos[s] + t < out_cap.
  const int32_t* out_pos;
  int32_t out_cap;
};

struct DequantArgs {
  const uint8_t* k_q;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint8_t* v_q;
  const uint16_t* v_scale;
  const int8_t* signs;
  uint16_t* k;  // may be null: keys skipped
  uint16_t* v;  // may be null: values skipped
  uint32_t rows;
  RowSplit split;
  RowMap in, out;
  // Windowed fetch: when in_len is set, rows (s, t, h) with h >= in_len[s]
  // are not read and are written as +0 (the fetch puts the token index last,
  // so that consecutive rows are consecutive tokens of one kv head).
  const int32_t* in_len;
  // Values left in the rotated domain: centroid * scale16, no transform or signs.
  int32_t rotated;
};

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* k_q;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint8_t* v_q;
  const uint16_t* v_scale;
  const int8_t* signs;
  const int32_t* ctx_lens;
  uint16_t* out;
  float* part;  // [batch, n_q_heads, splits, head_dim + 4]: acc[d], m, l, pad
  int64_t seq_stride, head_stride;
  int32_t batch, n_q_heads, n_kv_heads, max_ctx, splits, tokens_per_split;
  float softmax_scale;
  // Query tokens per sequence: query m of sequence b sits at position
  // ctx_b - n_queries + m and sees the cached tokens t <= that position.
  int32_t n_queries;
};

// Inverse rotation of bf16 rows: out = bf16(signs * FWHT(in) / sqrt(d)).
struct UnrotateArgs {
  const uint16_t* in;
  const int8_t* signs;
  uint16_t* out;
  uint32_t rows;
  RowSplit split;
  RowMap in_map, out_map;
};

hipError_t launch_quantize(const QuantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks);
hipError_t launch_unrotate(const UnrotateArgs& a, int d, hipStream_t st, int max_blocks);
hipError_t launch_dequantize(const DequantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks);
hipError_t launch_decode_attn(const AttnArgs& a, int d, int kb, int vb, hipStream_t st);

// Split-K decode geometry for a given problem (shared by the workspace query).
bool decode_attn_uses_mfma(int d, int kb, int vb);
void decode_attn_geometry(int d, int kb, int vb, int batch, int n_queries, int n_q_heads, int n_kv_heads,
                          int max_ctx, int* splits, int* tokens_per_split);
size_t decode_attn_part_bytes(int d, int batch, int n_queries, int n_q_heads, int splits);

}  // namespace tq
