// tq_check.h -- bounds tests of the checked build (compiled with -DTQ_CHECK
// into libtq_check.so; the library built without it is unchanged by them).
//
// Every kernel tests the global rows, records and byte offsets it derives
// against the extents the host computed for those buffers from the call's
// own arguments (row maps, capacities, counts).  A failed test ORs its bit
// into the flag word of the kernel's source file -- a vector atomic, never a
// trap -- and the access stays in range: a store is dropped, a load reads
// the buffer's first row instead.  tq_check_flags() returns the OR of every
// file's word on the current device and clears them.  Without TQ_CHECK the
// tests compile to nothing and the extents are ignored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

enum CheckBit : uint32_t {
  kChkQuantIn = 1u << 0,     // quantize / append: bf16 input rows
  kChkQuantOut = 1u << 1,    // quantize / append: plane rows written
  kChkDequantIn = 1u << 2,   // dequantize / fetch: plane rows read
  kChkDequantOut = 1u << 3,  // dequantize / fetch: bf16 rows written
  kChkUnrotIn = 1u << 4,     // un-rotate: rows read
  kChkUnrotOut = 1u << 5,    // un-rotate: rows written
  kChkAttnQ = 1u << 6,       // attention: query rows
  kChkAttnLen = 1u << 7,     // attention: context-length entries
  kChkAttnCache = 1u << 8,   // attention: cache rows
  kChkAttnPart = 1u << 9,    // attention: split-partial records
  kChkAttnOut = 1u << 10,    // attention: output rows
  kChkGrowSrc = 1u << 11,    // growth: source bytes
  kChkGrowDst = 1u << 12,    // growth: destination bytes
  kChkDenseIn = 1u << 13,    // paper variant: rows read
  kChkDenseOut = 1u << 14,   // paper variant: rows written
};

#ifdef TQ_CHECK
constexpr bool kChecked = true;
// One word per source file (each file that includes this header has its own).
static __device__ uint32_t g_check_word;

__device__ __forceinline__ bool check_ok(bool ok, uint32_t bit) {
  if (!ok) atomicOr(&g_check_word, bit);
  return ok;
}
// i when 0 <= i < n; otherwise the failure is recorded and 0 comes back
__device__ __forceinline__ int64_t check_row(int64_t i, int64_t n, uint32_t bit) {
  return check_ok(i >= 0 && i < n, bit) ? i : 0;
}
// This file's word, then cleared (host side; the caller synchronises first).
static inline uint32_t check_read_clear_file() {
  uint32_t v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_word), sizeof(v)) != hipSuccess) return 0x80000000u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &z, sizeof(z)) != hipSuccess) return 0x80000000u;
  return v;
}
#else
constexpr bool kChecked = false;
__device__ __forceinline__ bool check_ok(bool, uint32_t) { return true; }
__device__ __forceinline__ int64_t check_row(int64_t i, int64_t, uint32_t) { return i; }
static inline uint32_t check_read_clear_file() { return 0; }
#endif

// Each kernel file's word (host; declared here, defined in the file).
uint32_t check_read_clear_codec();
uint32_t check_read_clear_attn();
uint32_t check_read_clear_cache();
uint32_t check_read_clear_dense();

// Rows a map addresses: (n_seq - 1) * seq_stride + (n_tok - 1) * tok_stride
// + (n_head - 1) * head_stride + 1 (strides are non-negative), 0 for none,
// saturated at INT64_MAX.
inline int64_t map_extent(int64_t n_seq, int64_t n_tok, int64_t n_head, int64_t ss, int64_t ts, int64_t hs) {
  if (n_seq <= 0 || n_tok <= 0 || n_head <= 0) return 0;
  const __int128 e = (__int128)(n_seq - 1) * ss + (__int128)(n_tok - 1) * ts + (__int128)(n_head - 1) * hs + 1;
  return e > (__int128)INT64_MAX ? INT64_MAX : (int64_t)e;
}

}  // namespace tq
