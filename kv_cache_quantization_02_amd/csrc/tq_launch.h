// tq_launch.h -- argument blocks passed by value to the kernels, and the
// host-side launchers each kernel file exports to the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_check.h"
#include "tq_device.h"

namespace tq {

// Row r in [0, rows) is (s, t, h) with r = (s * n_tok + t) * n_head + h.
struct RowSplit {
  FastDiv div_head;  // divides by n_head
  FastDiv div_tok;   // divides by n_tok
};

// Row r -> (s, t, h), and the buffer row index of (s, t, h) under a map.
__device__ __forceinline__ void split_row(uint32_t r, const RowSplit& rs, uint32_t& s, uint32_t& t,
                                          uint32_t& h) {
  const uint32_t st = fast_div(r, rs.div_head);
  h = r - st * rs.div_head.d;
  s = fast_div(st, rs.div_tok);
  t = st - s * rs.div_tok.d;
}

__device__ __forceinline__ int64_t row_index(const RowMap& m, uint32_t s, uint32_t t, uint32_t h) {
  return (int64_t)s * m.seq_stride + (int64_t)t * m.tok_stride + (int64_t)h * m.head_stride;
}

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
  // rows the in and out maps address (the checked build's bounds; with
  // out_pos, the out map over the capacity)
  int64_t in_ext, out_ext;
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
  // Windowed fetch: when in_len is set, rows (s, t, h) with
  // h >= min(in_len[s], in_cap) are not read and are written as +0 (the fetch
  // puts the token index last, so that consecutive rows are consecutive
  // tokens of one kv head).
  const int32_t* in_len;
  int32_t in_cap;
  // Values left in the rotated domain: centroid * scale16, no transform or signs.
  int32_t rotated;
  // rows the in map (over the capacity in a fetch) and the out map address
  int64_t in_ext, out_ext;
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
  // Set by the launcher when every 16-byte copy of the matrix-core kernel's
  // wide layout is 16-byte aligned (value and key scale/zero planes at
  // 16-byte boundaries, even row strides).
  int32_t wide;
  // cache rows the strides address over max_ctx tokens (checked build)
  int64_t cache_ext;
};

// Inverse rotation of bf16 rows: out = bf16(signs * FWHT(in) / sqrt(d)).
struct UnrotateArgs {
  const uint16_t* in;
  const int8_t* signs;
  uint16_t* out;
  uint32_t rows;
  RowSplit split;
  RowMap in_map, out_map;
  int64_t in_ext, out_ext;  // rows each map addresses (checked build)
};

// Paper variant (dense rotation, one norm per row, optional QJL residual).
// Quantize reads bf16 rows x through x_map and writes the planes through
// plane_map; dequantize reads the planes and writes bf16 rows to x_out.
struct DenseArgs {
  const uint16_t* x;
  uint16_t* x_out;
  const uint16_t* rot;   // [d][d] bf16, row-major
  const uint16_t* proj;  // [d][d] bf16, row-major (QJL only)
  uint8_t* idx;          // d*bits/8 bytes per row
  float* norm;
  uint8_t* qjl;          // d/8 bytes per row (QJL only)
  float* gamma;          // (QJL only)
  uint32_t rows;
  RowSplit split;
  RowMap x_map, plane_map;
  int64_t x_ext, plane_ext;  // rows each map addresses (checked build)
};

// Re-laying a cache at another capacity.  Each plane is a set of
// segments, one per (sequence, kv head), of consecutive rows: the first
// `copy` bytes of a destination segment come from the source segment, the
// rest up to `dst_bytes` are zero.  Offsets are in bytes.
struct GrowPlane {
  const uint8_t* src;
  uint8_t* dst;
  int64_t src_seq, src_head, dst_seq, dst_head;
  int64_t copy, dst_bytes;
  uint32_t chunks;  // blocks per segment
  uint32_t vec16;   // every segment start 16-byte aligned on both sides
  int64_t src_ext, dst_ext;  // bytes the segments span on each side (checked build)
};

struct GrowArgs {
  GrowPlane plane[5];
  uint32_t first[5];  // first block of each plane; plane p owns [first[p], first[p+1])
  uint32_t total;     // blocks over all planes
  uint32_t n_kv_heads;
};

hipError_t launch_quantize(const QuantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks);
hipError_t launch_unrotate(const UnrotateArgs& a, int d, hipStream_t st, int max_blocks);
hipError_t launch_dequantize(const DequantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks);
hipError_t launch_decode_attn(const AttnArgs& a, int d, int kb, int vb, hipStream_t st);
hipError_t launch_grow(const GrowArgs& a, hipStream_t st, int max_blocks);
// Bytes of one destination segment that one block covers.
constexpr int64_t kGrowChunkBytes = 256 * 16 * 4;

hipError_t launch_dense_quantize(const DenseArgs& a, int d, int bits, bool qjl, hipStream_t st);
hipError_t launch_dense_dequantize(const DenseArgs& a, int d, int bits, bool qjl, hipStream_t st);

// Split-K decode geometry for a given problem (shared by the workspace query).
bool decode_attn_uses_mfma(int d, int kb, int vb);
void decode_attn_geometry(int d, int kb, int vb, int batch, int n_queries, int n_q_heads, int n_kv_heads,
                          int max_ctx, int* splits, int* tokens_per_split);
size_t decode_attn_part_bytes(int d, int batch, int n_queries, int n_q_heads, int splits);

}  // namespace tq
