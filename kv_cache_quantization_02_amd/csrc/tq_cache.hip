// tq_cache.hip -- re-laying a quantized cache at another capacity.
//
// A cache that runs out of room grows in 256-token steps: storage of the
// new capacity is allocated, the old rows go to its front and the rest is
// zero padding (campaign execution-log page, the KV append dispatch probe:
// at a growth boundary the cache allocates padding and concatenates the old
// storage with it).  On the GPU that is a strided copy bound by HBM: each
// kept byte is read once and each byte of the new storage written once.
//
// Work split: each plane is B*Hkv segments (one per sequence and kv head)
// of consecutive rows; a block covers kGrowChunkBytes of one destination
// segment, 16 bytes per lane and 4 units per lane, so a wave moves 1 KB per
// instruction.  Blocks of one segment are consecutive, and a grid-stride
// loop keeps the grid within the launch cap for caches of any size.
#include "tq_launch.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
typedef uint32_t grow_u32x4 __attribute__((ext_vector_type(4)));
static_assert(kGrowChunkBytes == (int64_t)kThreads * 16 * kUnroll, "a chunk is one block's 16-byte units");

// Plane p's descriptor by uniform selects (no dynamic index into the
// argument block, which would send it through private memory).
__device__ __forceinline__ GrowPlane pick(const GrowArgs& a, int p, uint32_t& first) {
  GrowPlane pl = a.plane[0];
  first = a.first[0];
#pragma unroll
  for (int i = 1; i < 5; ++i)
    if (p == i) {
      pl = a.plane[i];
      first = a.first[i];
    }
  return pl;
}

// One 16-byte unit that straddles the end of the kept bytes or of the
// segment, word by word (row lengths are whole words).
__device__ __forceinline__ void copy_words(const uint8_t* src, uint8_t* dst, int64_t x, int64_t copy,
                                           int64_t end) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int64_t xw = x + 4 * w;
    if (xw < end) *(uint32_t*)(dst + xw) = xw < copy ? *(const uint32_t*)(src + xw) : 0u;
  }
}

__global__ __launch_bounds__(kThreads) void grow_kernel(GrowArgs a) {
  const int tid = threadIdx.x;
  for (uint32_t blk = blockIdx.x; blk < a.total; blk += gridDim.x) {
    int p = 0;
#pragma unroll
    for (int i = 1; i < 5; ++i) p += blk >= a.first[i] ? 1 : 0;
    uint32_t first;
    const GrowPlane pl = pick(a, p, first);
    const uint32_t r = blk - first;
    const uint32_t seg = r / pl.chunks;
    const uint32_t chunk = r - seg * pl.chunks;
    const uint32_t b = seg / a.n_kv_heads;
    const uint32_t g = seg - b * a.n_kv_heads;
    int64_t so = (int64_t)b * pl.src_seq + (int64_t)g * pl.src_head;
    int64_t dof = (int64_t)b * pl.dst_seq + (int64_t)g * pl.dst_head;
    if (kChecked) {
      // the segment's kept bytes and its whole destination inside the
      // extents (a failed bound reads from and writes to nothing outside:
      // the chunk is skipped); both tests run, so both bits can be set
      const bool src_ok = check_ok(so + pl.copy <= pl.src_ext, kChkGrowSrc);
      const bool dst_ok = check_ok(dof + pl.dst_bytes <= pl.dst_ext, kChkGrowDst);
      if (!(src_ok && dst_ok)) continue;
    }
    const uint8_t* src = pl.src + so;
    uint8_t* dst = pl.dst + dof;
    const int64_t x0 = (int64_t)chunk * kGrowChunkBytes;
    if (pl.vec16 && x0 + kGrowChunkBytes <= pl.copy) {
      // a chunk of kept rows: every load of the block issues before its
      // first store.  Loads and stores are non-temporal: each byte is read
      // and written once, and keeping the copy out of the caches took the
      // growth of the 16 x 8 x 32768 k8v3 cache from 330-336 to 273-276 us.
      grow_u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_nontemporal_load((const grow_u32x4*)(src + x0 + (u * kThreads + tid) * 16));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        __builtin_nontemporal_store(v[u], (grow_u32x4*)(dst + x0 + (u * kThreads + tid) * 16));
    } else if (pl.vec16 && x0 >= pl.copy && x0 + kGrowChunkBytes <= pl.dst_bytes) {
      // a chunk of padding
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        __builtin_nontemporal_store(grow_u32x4{0u, 0u, 0u, 0u}, (grow_u32x4*)(dst + x0 + (u * kThreads + tid) * 16));
    } else if (pl.vec16) {
      // the chunk where the kept rows end or the segment ends
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t x = x0 + (int64_t)(u * kThreads + tid) * 16;
        if (x + 16 <= pl.copy)
          *(uint4*)(dst + x) = *(const uint4*)(src + x);
        else if (x >= pl.copy && x + 16 <= pl.dst_bytes)
          *(uint4*)(dst + x) = make_uint4(0u, 0u, 0u, 0u);
        else if (x < pl.dst_bytes)
          copy_words(src, dst, x, pl.copy, pl.dst_bytes);
      }
    } else {
      // 2-byte aligned planes: half-words
      for (int u = 0; u < (int)(kGrowChunkBytes / 2 / kThreads); ++u) {
        const int64_t x = x0 + (int64_t)(u * kThreads + tid) * 2;
        if (x < pl.dst_bytes) *(uint16_t*)(dst + x) = x < pl.copy ? *(const uint16_t*)(src + x) : (uint16_t)0;
      }
    }
  }
}

}  // namespace

uint32_t check_read_clear_cache() { return check_read_clear_file(); }

hipError_t launch_grow(const GrowArgs& a, hipStream_t st, int max_blocks) {
  if (a.total == 0) return hipSuccess;
  const uint32_t grid = a.total < (uint32_t)max_blocks ? a.total : (uint32_t)max_blocks;
  hipLaunchKernelGGL(grow_kernel, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace tq
