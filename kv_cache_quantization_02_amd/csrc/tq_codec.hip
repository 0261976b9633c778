// tq_codec.hip -- quantize / dequantize kernels for gfx950.
//
// TurboQuant page, "Algorithm (vllm-metal reference semantics, exact)":
//   keys   : asymmetric affine per 32-group, fp32 arithmetic, fp16 scale/zero;
//   values : y = FWHT(x * signs) / sqrt(d); RMS per 32-group; Lloyd-Max index
//            of y / (scale + 1e-8); little-endian packed bitstream.
//
// These kernels are bound by VALU issue, not by HBM, so the layout is chosen
// to minimise vector instructions per row:
//   * one lane owns one whole 32-element group (64 contiguous bf16 bytes), so
//     group min/max, the mean square and every per-group scalar (divisions,
//     square root, fp16 conversion) are computed once, inside the lane;
//   * the row's groups sit on lanes whose xor partners are DPP-reachable
//     (g bit 0 -> lane xor 1, bit 1 -> xor 2, bit 2 -> xor 8, bit 3 -> xor 4),
//     so each cross-lane transform stage is one v_fmac_f32_dpp per element;
//   * divisions by the group scale are exact via one correctly rounded
//     reciprocal and Markstein's correction, 3 operations per element.
// Quantize and dequantize are one launch each: even blocks stream key rows,
// odd blocks value rows.
#include "tq_codebooks.h"
#include "tq_device.h"
#include "tq_launch.h"

#include <utility>

namespace tq {

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 with I a
// compile-time constant, so per-batch arrays are indexed statically and stay
// in registers (a runtime loop index would move them to scratch memory).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__constant__ uint32_t c_bnd_2[3] = {TQ_BOUNDARIES_2BIT};
__constant__ uint32_t c_bnd_3[7] = {TQ_BOUNDARIES_3BIT};
__constant__ uint32_t c_bnd_4[15] = {TQ_BOUNDARIES_4BIT};
__constant__ uint32_t c_bnd_5[31] = {TQ_BOUNDARIES_5BIT};
__constant__ uint32_t c_bnd_8[255] = {TQ_BOUNDARIES_8BIT};
__constant__ uint32_t c_cen_2[4] = {TQ_CENTROIDS_2BIT};
__constant__ uint32_t c_cen_3[8] = {TQ_CENTROIDS_3BIT};
__constant__ uint32_t c_cen_4[16] = {TQ_CENTROIDS_4BIT};
__constant__ uint32_t c_cen_5[32] = {TQ_CENTROIDS_5BIT};
__constant__ uint32_t c_cen_8[256] = {TQ_CENTROIDS_8BIT};

template <int B>
__device__ __forceinline__ const uint32_t* boundaries() {
  if constexpr (B == 2) return c_bnd_2;
  else if constexpr (B == 3) return c_bnd_3;
  else if constexpr (B == 4) return c_bnd_4;
  else if constexpr (B == 5) return c_bnd_5;
  else return c_bnd_8;
}

template <int B>
__device__ __forceinline__ const uint32_t* centroids() {
  if constexpr (B == 2) return c_cen_2;
  else if constexpr (B == 3) return c_cen_3;
  else if constexpr (B == 4) return c_cen_4;
  else if constexpr (B == 5) return c_cen_5;
  else return c_cen_8;
}

// ------------------------------------------------------------ lane layout
// D/32 lanes per row, 64/(D/32) rows per wave; lane -> (group g, row rw).
template <int D>
struct GroupLanes {
  static constexpr int LPR = D / kGroup;
  static constexpr int RPW = 64 / LPR;
  static constexpr int NSTAGE = (D == 64) ? 1 : (D == 128) ? 2 : (D == 256) ? 3 : 4;
  __device__ static int group(int lane) {
    if constexpr (D == 64) return lane & 1;
    else if constexpr (D == 128) return lane & 3;
    else if constexpr (D == 256) return (lane & 3) | (((lane >> 3) & 1) << 2);
    else return (lane & 3) | (((lane >> 3) & 1) << 2) | (((lane >> 2) & 1) << 3);
  }
  __device__ static int row(int lane) {
    if constexpr (D == 64) return lane >> 1;
    else if constexpr (D == 128) return lane >> 2;
    else if constexpr (D == 256) return ((lane >> 2) & 1) | ((lane >> 4) << 1);
    else return lane >> 4;
  }
};

// The lane mask that pairs groups g and g ^ (1 << k).
template <int K>
constexpr int stage_mask() { return K == 0 ? 1 : K == 1 ? 2 : K == 2 ? 8 : 4; }

// w += c * w(lane ^ M) for all 32 elements: one DPP-fused fmac per element
// for M in {1, 2, 8}; a swizzle plus an fma for M = 4.
template <int M>
__device__ __forceinline__ void cross_stage(float (&w)[32], float c) {
  if constexpr (M == 4) {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = __builtin_fmaf(lane_xor<4>(w[i]), c, w[i]);
  } else {
#define TQ_FMAC_DPP8(CTRL)                                                                      \
  asm volatile("s_nop 1\n\t"                                                                    \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL "\n\t"                                        \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL                                               \
               : "+v"(w[j]), "+v"(w[j + 1]), "+v"(w[j + 2]), "+v"(w[j + 3]), "+v"(w[j + 4]),   \
                 "+v"(w[j + 5]), "+v"(w[j + 6]), "+v"(w[j + 7])                                \
               : "v"(c))
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
      if constexpr (M == 1)
        TQ_FMAC_DPP8("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1");
      else if constexpr (M == 2)
        TQ_FMAC_DPP8("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1");
      else
        TQ_FMAC_DPP8("row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1");
    }
#undef TQ_FMAC_DPP8
  }
}

// Unnormalised Walsh-Hadamard transform of the row, stages h = 1 .. D/2 in
// ascending order.  Stages below 32 run inside the lane; stage h = 32 * 2^k
// pairs this lane with lane ^ stage_mask<k>.  The lane holding the upper
// element of a cross pair computes self - partner, the negative of the true
// value, so the result is sigma * FWHT with sigma = +-1 per lane; the sign is
// returned so the caller folds it into its final multiply.
template <int D>
__device__ __forceinline__ float fwht_group(float (&w)[32], int lane) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = w[i], b = w[i + h];
        w[i] = a + b;
        w[i + h] = a - b;
      }
    }
  }
  float sigma = 1.f;
  constexpr int NS = GroupLanes<D>::NSTAGE;
  if constexpr (NS >= 1) { const float c = (lane & stage_mask<0>()) ? -1.f : 1.f; cross_stage<stage_mask<0>()>(w, c); sigma *= c; }
  if constexpr (NS >= 2) { const float c = (lane & stage_mask<1>()) ? -1.f : 1.f; cross_stage<stage_mask<1>()>(w, c); sigma *= c; }
  if constexpr (NS >= 3) { const float c = (lane & stage_mask<2>()) ? -1.f : 1.f; cross_stage<stage_mask<2>()>(w, c); sigma *= c; }
  if constexpr (NS >= 4) { const float c = (lane & stage_mask<3>()) ? -1.f : 1.f; cross_stage<stage_mask<3>()>(w, c); sigma *= c; }
  return sigma;
}

// 32 bf16 (64 bytes) -> 16 raw words.
__device__ __forceinline__ void load_group(const uint16_t* p, uint32_t (&u)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = q[j];
    u[4 * j] = v.x; u[4 * j + 1] = v.y; u[4 * j + 2] = v.z; u[4 * j + 3] = v.w;
  }
}

// ------------------------------------------------------------ input tiles
// A wave's rows for one iteration form one 4 KB tile: 64 lanes x one
// 32-element group (64 bytes).  Loading it group by group leaves every load
// instruction scattered over the tile (64 bytes apart per lane), which costs a
// quarter of the achievable HBM rate; instead the tile is copied HBM -> LDS
// by four global_load_lds_dwordx4 of 64 x 16 bytes, one iteration ahead of
// its use, and each lane then reads its own group back from LDS.  Copy slot p
// holds quarter q of reader lane L's group with p = 4L + ((q + L/2) mod 4):
// every eight consecutive readers of a quarter hit distinct 16-byte bank
// groups.  The copies are inline assembly so the compiler does not wait for
// them before unrelated LDS reads; M0 (their LDS base) is reserved by the
// compiler and read by no other instruction of these kernels.
//
// The input copies and the plane stores are non-temporal (nt): the bf16 rows
// are read once and the planes are read by a later call, and with the decode's
// cache copies also non-temporal this pair measured best inside the bench step
// (quantize 561-566 against 566-569 us, the dequantize that follows 544-545
// against 554-556 us, three alternating runs).  Either alone moves cost
// between the kernels: non-temporal copies alone took quantize to 545 us but
// the dequantize after it to 602 us.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t tq_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tq_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) tq_u32x4 lds_u32x4;
constexpr int kTile = 4096;

__device__ __forceinline__ int tile_slot(int reader, int q) { return 4 * reader + ((q + (reader >> 1)) & 3); }

__device__ __forceinline__ void tile_copy16(const void* src, const lds_u8* dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"((uint32_t)(uintptr_t)dst)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Rows r of a tensor are memory rows r (no head, token or sequence gaps).
__device__ __forceinline__ bool rows_contiguous(const RowMap& m, const RowSplit& sp) {
  return m.head_stride == 1 && m.tok_stride == (int64_t)sp.div_head.d &&
         m.seq_stride == (int64_t)sp.div_tok.d * sp.div_head.d;
}

// One int32 from global memory, waited for inside the same asm block.  The
// append path reads its sequence positions through this: a plain load there
// sits in a branch of the row loop, and the compiler then waits for every
// outstanding memory operation (the next tile's copies included) at the top
// of every iteration, append or not.
__device__ __forceinline__ int32_t load_i32_now(const int32_t* p) {
  int32_t v;
  asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Output row of input row r for the quantize kernels, or -1 when the row is
// past the end or falls outside the cache window of an append.
__device__ __forceinline__ int64_t quant_out_row(const QuantArgs& a, uint32_t r, bool contig_out) {
  if (r >= a.rows) return -1;
  int64_t o = r;
  if (!contig_out) {
    uint32_t s, t, h;
    split_row(r, a.split, s, t, h);
    o = row_index(a.out, s, t, h);
    if (a.out_pos) {
      const int64_t p = load_i32_now(a.out_pos + s);
      if (p + t < 0 || p + t >= a.out_cap) return -1;
      o += p * a.out.tok_stride;
    }
  }
  // a row outside the out map's extent is not written (checked build)
  return check_ok(o < a.out_ext, kChkQuantOut) ? o : -1;
}

// Byte offset, within a contiguous tile, of copy slot 64j + lane.
template <int D>
__device__ __forceinline__ uint32_t tile_src_offset(int j, int lane) {
  using L = GroupLanes<D>;
  const int p = 64 * j + lane, reader = p >> 2, q = ((p & 3) - (reader >> 1)) & 3;
  return (uint32_t)(2 * (L::row(reader) * D + kGroup * L::group(reader) + 8 * q));
}

// Copies of a whole tile of contiguous rows: scalar base, lane offsets fixed.
__device__ __forceinline__ void tile_issue_contig(const uint16_t* src, uint32_t base_row, int d,
                                                  const uint32_t (&off)[4], const lds_u8* stage) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(src) + (uint64_t)base_row * (uint64_t)(2 * d);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off[j]), "s"(b),
                 "s"((uint32_t)(uintptr_t)(stage + 1024 * j))
                 : "memory", "m0");
}

// Issue the four copies of the tile of rows base .. base + RPW - 1 (rows past
// the end re-read the last row; their results are never stored).
template <int D>
__device__ __forceinline__ void tile_issue(const uint16_t* src, const QuantArgs& a, uint32_t base, bool contig,
                                           const uint32_t (&off)[4], const lds_u8* stage, int lane) {
  using L = GroupLanes<D>;
  if (contig && base + L::RPW <= a.rows) {
    // (a failed bound reads the first rows instead; the contiguous path
    // implies at least RPW rows)
    tile_issue_contig(src, check_ok(base + L::RPW <= a.in_ext, kChkQuantIn) ? base : 0u, D, off, stage);
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 64 * j + lane, reader = p >> 2, q = ((p & 3) - (reader >> 1)) & 3;
    uint32_t r = base + (uint32_t)L::row(reader);
    if (r >= a.rows) r = a.rows - 1;
    int64_t irow = r;
    if (!contig) {
      uint32_t s, t, h;
      split_row(r, a.split, s, t, h);
      irow = row_index(a.in, s, t, h);
    }
    irow = check_row(irow, a.in_ext, kChkQuantIn);
    tile_copy16(src + irow * D + kGroup * L::group(reader) + 8 * q, stage + 1024 * j);
  }
}

__device__ __forceinline__ void tile_read(const lds_u8* stage, int lane, uint32_t (&u)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const tq_u32x4 w = *(const lds_u32x4*)(stage + 16 * tile_slot(lane, q));
    u[4 * q] = w.x; u[4 * q + 1] = w.y; u[4 * q + 2] = w.z; u[4 * q + 3] = w.w;
  }
}

// Wait until the tile of this iteration has landed.  Issued after it: the
// previous iteration's stores (at least one instruction per output array,
// `min_stores`) and, with `next`, the next tile's four copies.  vmcnt retires
// in issue order, so allowing that many to remain outstanding is exact or
// conservative.
template <int MinStores>
__device__ __forceinline__ void tile_wait(bool first, bool next) {
  if (next) {
    if (first) wait_vmcnt<4>();
    else wait_vmcnt<4 + MinStores>();
  } else {
    wait_vmcnt<0>();
  }
}

// Exact division of every element by a per-group divisor s: with r = RN(1/s),
// q0 = RN(y r), e = y - q0 s (exact by fma), q = RN(q0 + e r) equals RN(y/s)
// (Markstein 1990) while s is a normal number and no step overflows.
__device__ __forceinline__ float div_markstein(float y, float s, float r) {
  const float q0 = y * r;
  const float e = __builtin_fmaf(-q0, s, y);
  return __builtin_fmaf(e, r, q0);
}

__device__ __forceinline__ bool normal_divisor(float s) {
  // 2^-100 <= |s| < 2^100 keeps every Markstein step away from the
  // subnormal and overflow ranges; other divisors take the exact '/'.
  const float a = __builtin_fabsf(s);
  return a >= 7.88860905e-31f && a < 1.26765060e+30f;
}

// Lloyd-Max index #{boundaries < yn}, yn = RN(y / den) exact.  Odd widths
// with symmetric tables are searched on the magnitude: key = bits(yn)
// rotated left by one (the sign lands in bit 0), so for a non-negative
// boundary b with key-threshold 2*bits(b), key > 2*bits(b) holds exactly when
// b < yn for yn >= 0 and when b <= |yn| for yn < 0 -- the two cases the count
// needs -- and the index is then c ^ (yn > 0 ? H+1 : H) with H the number of
// negative boundaries.  NaN yn gives 0.
template <int B>
__device__ __forceinline__ uint32_t lloyd_max_index(float yn, const float* lds_bnd) {
  if constexpr (B <= 4) {
    constexpr int H = (1 << (B - 1)) - 1;  // negative boundaries; boundary H is 0
    const uint32_t* bnd = boundaries<B>();
    const uint32_t key = __builtin_amdgcn_alignbit(__float_as_uint(yn), __float_as_uint(yn), 31);
    uint32_t c = 0;
#pragma unroll
    for (int j = 1; j <= H; ++j) c += (key > (bnd[H + j] << 1)) ? 1u : 0u;
    const uint32_t base = (yn > 0.f) ? (uint32_t)(H + 1) : (uint32_t)H;
    return c ^ base;
  } else {
    uint32_t idx = 0;
#pragma unroll
    for (int step = 1 << (B - 1); step >= 1; step >>= 1)
      idx += (lds_bnd[idx + step - 1] < yn) ? (uint32_t)step : 0u;
    return idx;
  }
}

// ------------------------------------------------------------------ keys
template <int D, int KB>
__device__ __forceinline__ void quantize_keys_rows(const QuantArgs& a, uint32_t blk, uint32_t nblk, uint8_t* tile_lds) {
  using L = GroupLanes<D>;
  constexpr int G = D / kGroup;
  const int lane = threadIdx.x & 63, g = L::group(lane), rw = L::row(lane);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wave = blk * 4u + (uint32_t)wv;
  const uint32_t nwave = nblk * 4u, stride = nwave * L::RPW;
  const float lo = KB == 8 ? -127.f : 0.f;
  const float hi = KB == 8 ? 127.f : (float)((1 << KB) - 1);
  const lds_u8* const tiles = (const lds_u8*)(tile_lds + wv * 2 * kTile);
  const bool contig = rows_contiguous(a.in, a.split);
  const bool contig_out = rows_contiguous(a.out, a.split) && !a.out_pos;
  const uint32_t off[4] = {tile_src_offset<D>(0, lane), tile_src_offset<D>(1, lane), tile_src_offset<D>(2, lane),
                           tile_src_offset<D>(3, lane)};
  uint32_t base = wave * L::RPW;
  if (base < a.rows) tile_issue<D>(a.k, a, base, contig, off, tiles, lane);
  for (int it = 0; base < a.rows; base += stride, ++it) {
    const bool next = base + stride < a.rows;
    if (next) tile_issue<D>(a.k, a, base + stride, contig, off, tiles + ((it + 1) & 1) * kTile, lane);
    tile_wait<3>(it == 0, next);  // k_q, k_scale, k_zero stores
    uint32_t u[16];
    tile_read(tiles + (it & 1) * kTile, lane, u);
    const int64_t orow = quant_out_row(a, base + rw, contig_out);
    const bool wr = orow >= 0;
    float x[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[2 * i] = bf16_lo(u[i]);
      x[2 * i + 1] = bf16_hi(u[i]);
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      mn = __builtin_elementwise_minimum(mn, x[i]);
      mx = __builtin_elementwise_maximum(mx, x[i]);
    }
    float scale, zero;
    if constexpr (KB == 8) {
      scale = (mx - mn) / 254.0f;
      zero = __builtin_rintf((mx + mn) / (2.0f * scale));
    } else {
      scale = (mx - mn) / (float)((1 << KB) - 1);
      zero = __builtin_rintf(mn / scale);
    }
    const bool fast = normal_divisor(scale);
    const float rcp = 1.0f / scale;
    float q[32];
    if (fast) {
#pragma unroll
      for (int i = 0; i < 32; ++i) q[i] = div_markstein(x[i], scale, rcp);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) q[i] = x[i] / scale;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = __builtin_fminf(__builtin_fmaxf(q[i] - zero, lo), hi);
    if constexpr (KB == 8) {
      // round half-to-even into the low byte by adding 1.5 * 2^23, then gather
      // the four low bytes of each quad of floats
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b0 = __float_as_uint(q[4 * i] + 12582912.0f);
        const uint32_t b1 = __float_as_uint(q[4 * i + 1] + 12582912.0f);
        const uint32_t b2 = __float_as_uint(q[4 * i + 2] + 12582912.0f);
        const uint32_t b3 = __float_as_uint(q[4 * i + 3] + 12582912.0f);
        const uint32_t lo2 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
        const uint32_t hi2 = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
        o[i] = lo2 | hi2;
      }
      // the key plane is only 8-byte aligned: 8-byte stores
      if constexpr (D == 128) {
        // Whole rows per store instruction.  Each lane's four 8-byte stores
        // of its group (8 bytes at a 32-byte stride per instruction) reach
        // memory as partial lines when they bypass the caches (7% more bytes
        // written per launch).  The wave's 16 code rows (2 KB, row
        // r at 128 r, group g at 32 g) and their plane rows are staged in this
        // iteration's input tile, already read into registers, and store j
        // writes rows 4 j .. 4 j + 3 whole: lane L takes bytes 8 (L mod 16) of
        // row 4 j + L / 16.  The slot is next written by the copies issued at
        // the top of the following iteration, after these reads are consumed.
        lds_u8* const stage = (lds_u8*)(tile_lds + wv * 2 * kTile + (it & 1) * kTile);
        *(lds_u32x4*)(stage + 32 * lane) = tq_u32x4{o[0], o[1], o[2], o[3]};
        *(lds_u32x4*)(stage + 32 * lane + 16) = tq_u32x4{o[4], o[5], o[6], o[7]};
        if (g == 0) *(__attribute__((address_space(3))) int64_t*)(stage + 2048 + 8 * rw) = orow;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t ro = *(const __attribute__((address_space(3))) int64_t*)(stage + 2048 + 8 * (4 * j + (lane >> 4)));
          const tq_u32x2 v = *(const __attribute__((address_space(3))) tq_u32x2*)(stage + 512 * j + 8 * lane);
          if (ro >= 0) __builtin_nontemporal_store(v, reinterpret_cast<tq_u32x2*>(a.k_q + ro * D) + (lane & 15));
        }
        __builtin_amdgcn_wave_barrier();
      } else if (wr) {
        tq_u32x2* dst = reinterpret_cast<tq_u32x2*>(a.k_q + orow * D + kGroup * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(tq_u32x2{o[2 * i], o[2 * i + 1]}, dst + i);
      }
    } else if constexpr (KB == 2 || KB == 4) {
      // v_cvt_pk_u8_f32 rounds to nearest even into one byte of a word: bytes
      // of the elements 8/KB apart, then one shift-or per byte word merges
      // them into the packed word (element i at bits KB*i)
      constexpr int EPW = 32 / KB, PER = 8 / KB;
      uint32_t o[KB];
#pragma unroll
      for (int w = 0; w < KB; ++w) {
        uint32_t acc = 0;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
          uint32_t bw = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) bw = __builtin_amdgcn_cvt_pk_u8_f32(q[EPW * w + PER * k + m], k, bw);
          acc |= bw << (KB * m);
        }
        o[w] = acc;
      }
      if (wr) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.k_q + orow * (D * KB / 8) + 4 * KB * g);
#pragma unroll
        for (int i = 0; i < KB; ++i) __builtin_nontemporal_store(o[i], dst + i);
      }
    } else {
      uint32_t o[KB] = {};
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(q[i], 0, 0);  // RNE into byte 0
        const int bit = KB * i, wd = bit >> 5, off = bit & 31;
        o[wd] |= v << off;
        if (off + KB > 32) o[wd + 1] |= v >> (32 - off);
      }
      if (wr) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.k_q + orow * (D * KB / 8) + 4 * KB * g);
#pragma unroll
        for (int i = 0; i < KB; ++i) __builtin_nontemporal_store(o[i], dst + i);
      }
    }
    if (wr) {
      __builtin_nontemporal_store((uint16_t)f16_bits(scale), a.k_scale + orow * G + g);
      __builtin_nontemporal_store((uint16_t)f16_bits(zero), a.k_zero + orow * G + g);
    }
  }
}

// Lloyd-Max indices of a group's 32 elements y for a 2- or 3-bit table,
// packed into the group's VB words, without dividing: |y| is compared with
// the group's thresholds RN(b * den) for the positive boundaries b.  The index
// can then differ from that of RN(y / den) only where y / den lies within a
// few ulps (< 5e-7) of a boundary -- exact equality included -- inside the
// tie window the format allows.  With c = #{thresholds below |y|}, the index
// is H + 1 + c above zero and H - c otherwise; bit by bit, the top bit is
// s = [y > 0] and bit k below it is bit k of c XOR !s.  Each bit is a lane
// mask (index_pair), and it enters the packed words by o = 2 o + bit, stream
// positions taken from the highest down, so no bit is ever materialised,
// shifted or or-ed into place.  Requires a normal den and finite y.
template <int VB>
__device__ __forceinline__ void threshold_index(const float (&y)[32], float den, uint32_t (&o)[VB]) {
  constexpr int H = (1 << (VB - 1)) - 1;
  const uint32_t* bnd = boundaries<VB>();
  float thr[H];
#pragma unroll
  for (int j = 1; j <= H; ++j) thr[j - 1] = __uint_as_float(bnd[H + j]) * den;
  static_for<16>([&](auto P) {
    constexpr int i = 31 - 2 * (int)P;              // the pair (i, i - 1)
    constexpr int top = VB * i + VB - 1;            // its highest stream position
    constexpr int hi = top >> 5, lo = (VB * (i - 1)) >> 5;
    constexpr int nh = hi == lo ? 2 * VB : top - 32 * hi + 1;
    index_pair<VB, nh>(y[i], y[i - 1], thr, o[hi], o[lo]);
  });
}

// Lloyd-Max indices of a group's 32 elements y for the 4-bit table, through a
// cell table held across the wave's lanes: 5 vector operations per element,
// where the threshold search takes 12.  With zk = y * RN(4/den) the scaled
// boundaries 4b lie at least 1.03 apart (the table's narrowest gap is 0.258).
// Rounding y * RN(4/den) to a multiple of 1/4 (one fma with 1.5 * 2^21, whose
// float bits then end in 4 * that multiple) and dropping the two fractional
// bits gives the cell c; every zk in cell c lies in the closed interval
// [c - 1/8, c + 7/8], which holds at most one scaled boundary.  Lane (c mod 64)
// of the table holds that boundary (+1e30 where there is none) and the number
// of boundaries below the cell, so the index #{b : 4b < zk} is
// count + [zk > boundary], two wave permutes away; the fma's float bits serve
// as the permute's byte address as they are (it reads lane (address / 4) mod
// 64).  A normal den bounds |y / den| by sqrt(32) (1 + 4 ulp) -- no element
// exceeds the root of the group's sum of squares -- so |zk| < 23 and the
// cells -23 .. 22 fall on distinct lanes.  The index then differs from that of
// RN(y / den) only where y / den lies within 3 ulps of a boundary (< 5e-7),
// inside the tie window the format allows.
struct CellTable {
  int t;  // float bits of the cell's scaled boundary
  int j;  // boundaries below the cell
};

template <int VB>
__device__ __forceinline__ CellTable cell_table(int lane) {
  const int c = lane < 32 ? lane : lane - 64;
  const float lo = (float)c - 0.125f, hi = (float)c + 0.875f;
  const uint32_t* bnd = boundaries<VB>();
  float t = 1e30f;
  int j = 0;
  for (int k = 0; k < (1 << VB) - 1; ++k) {
    const float b = 4.0f * __uint_as_float(bnd[k]);
    if (b < lo) ++j;
    else if (b <= hi) t = __builtin_fminf(t, b);
  }
  return {__float_as_int(t), j};
}

// Elements go from the highest down in pairs: the permutes of one pair are
// issued before the previous pair's results are used (four pairs in flight
// measured the same and hold 9 more registers), and each index enters its
// word by o = (o << VB) | idx (an element that straddles two words opens the
// lower one).
template <int VB>
__device__ __forceinline__ void table_index(const float (&y)[32], float rcp, const CellTable& tab,
                                            uint32_t (&o)[VB]) {
  constexpr int NB = 2, NBATCH = 32 / NB;
  const float rk = 4.0f * rcp;
  float t[2][NB];
  int j[2][NB];
  auto issue = [&](auto B) {
    constexpr int b = (int)B;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int cell = __float_as_int(__builtin_fmaf(y[31 - NB * b - k], rk, 3145728.0f));
      t[b & 1][k] = __int_as_float(__builtin_amdgcn_ds_bpermute(cell, tab.t));
      j[b & 1][k] = __builtin_amdgcn_ds_bpermute(cell, tab.j);
    }
  };
  auto consume = [&](auto B) {
    constexpr int b = (int)B;
    static_for<NB>([&](auto K) {
      constexpr int i = 31 - NB * b - (int)K;
      const uint32_t idx = (uint32_t)j[b & 1][K] + (y[i] * rk > t[b & 1][K] ? 1u : 0u);
      constexpr int lw = (VB * i) >> 5, hw = (VB * i + VB - 1) >> 5;
      if constexpr (lw == hw) {
        o[lw] = (o[lw] << VB) | idx;
      } else {
        constexpr int nh = VB * i + VB - 32 * hw;  // bits in the higher word
        o[hw] = (o[hw] << nh) | (idx >> (VB - nh));
        o[lw] = idx & ((1u << (VB - nh)) - 1u);
      }
    });
  };
  static_for<NBATCH>([&](auto B) {
    issue(B);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr ((int)B > 0) consume(std::integral_constant<int, (int)B - 1>{});
    __builtin_amdgcn_sched_barrier(0);
  });
  consume(std::integral_constant<int, NBATCH - 1>{});
}

// ---------------------------------------------------------------- values
template <int D, int VB>
__device__ __forceinline__ void quantize_values_rows(const QuantArgs& a, uint32_t blk, uint32_t nblk,
                                                     uint8_t* tile_lds) {
  using L = GroupLanes<D>;
  constexpr int G = D / kGroup;
  __shared__ float bnd_lds[VB >= 5 ? (1 << VB) : 1];
  if constexpr (VB >= 5) {
    for (int i = threadIdx.x; i < (1 << VB) - 1; i += blockDim.x)
      bnd_lds[i] = __uint_as_float(boundaries<VB>()[i]);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, g = L::group(lane), rw = L::row(lane);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wave = blk * 4u + (uint32_t)wv;
  const uint32_t nwave = nblk * 4u, stride = nwave * L::RPW;
  // sign masks of this lane's 32 elements, two per bf16 pair (bits 15 and 31)
  uint32_t smask[16];
  {
    const uint4* sp = reinterpret_cast<const uint4*>(a.signs + kGroup * g);
    const uint4 s0 = sp[0], s1 = sp[1];
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = sw[i >> 1] >> (16 * (i & 1));
      smask[i] = ((word & 0x80u) << 8) | ((word & 0x8000u) << 16);
    }
  }
  const float rd = inv_sqrt_d<D>();
  [[maybe_unused]] CellTable tab{};
  if constexpr (VB == 4) tab = cell_table<VB>(lane);
  const lds_u8* const tiles = (const lds_u8*)(tile_lds + wv * 2 * kTile);
  const bool contig = rows_contiguous(a.in, a.split);
  const bool contig_out = rows_contiguous(a.out, a.split) && !a.out_pos;
  const uint32_t off[4] = {tile_src_offset<D>(0, lane), tile_src_offset<D>(1, lane), tile_src_offset<D>(2, lane),
                           tile_src_offset<D>(3, lane)};
  uint32_t base = wave * L::RPW;
  if (base < a.rows) tile_issue<D>(a.v, a, base, contig, off, tiles, lane);
  for (int it = 0; base < a.rows; base += stride, ++it) {
    const bool next = base + stride < a.rows;
    if (next) tile_issue<D>(a.v, a, base + stride, contig, off, tiles + ((it + 1) & 1) * kTile, lane);
    tile_wait<2>(it == 0, next);  // v_q, v_scale stores
    const int64_t orow = quant_out_row(a, base + rw, contig_out);
    const bool active = orow >= 0;
    uint32_t u[16];
    tile_read(tiles + (it & 1) * kTile, lane, u);
    float w[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t x = u[i] ^ smask[i];
      w[2 * i] = bf16_lo(x);
      w[2 * i + 1] = bf16_hi(x);
    }
    const float m = fwht_group<D>(w, lane) * rd;
    float y[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = w[i] * m;
    // mean square: adjacent pairs, then pairs of pairs, ... (fixed tree)
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = y[2 * i] * y[2 * i] + y[2 * i + 1] * y[2 * i + 1];
#pragma unroll
    for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
      for (int i = 0; i < n; ++i) e[i] = e[2 * i] + e[2 * i + 1];
    const float scale = __builtin_sqrtf(e[0] * 0.03125f);
    const float den = scale + 1e-8f;
    const bool fast = normal_divisor(den);
    uint32_t o[VB] = {};
    auto put = [&](int i, uint32_t idx) {
      const int bit = VB * i, wd = bit >> 5, off = bit & 31;
      o[wd] |= idx << off;
      if (off + VB > 32) o[wd + 1] |= idx >> (32 - off);
    };
    // Index by division: y / den exactly, then the table search.
    auto divided = [&]() {
      const float rcp = 1.0f / den;
      if (fast) {
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = div_markstein(y[i], den, rcp);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] = y[i] / den;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) put(i, lloyd_max_index<VB>(y[i], bnd_lds));
    };
    if constexpr (VB == 4) {
      // the permutes need every lane: the table runs wave-wide, and groups
      // without a normal den (whose words it leaves meaningless) divide
      table_index<VB>(y, 1.0f / den, tab, o);
      if (!fast) {
#pragma unroll
        for (int i = 0; i < VB; ++i) o[i] = 0;
        divided();
      }
    } else if constexpr (VB <= 4) {
      if (fast) threshold_index<VB>(y, den, o);
      else divided();
    } else {
      divided();
    }
    if (active) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.v_q + orow * (D * VB / 8) + 4 * VB * g);
#pragma unroll
      for (int i = 0; i < VB; ++i) __builtin_nontemporal_store(o[i], dst + i);
      __builtin_nontemporal_store((uint16_t)f16_bits(scale), a.v_scale + orow * G + g);
    }
  }
}

// ------------------------------------------------------------- dequantize
// Output staging for the dequantize kernels.  A wave's 64 lanes hold
// 64 x 64 bytes = one 4 KB tile of RPW consecutive bf16 rows (lane (rw, g)
// holds bytes 64g .. 64g+63 of row rw).  Storing that straight from the
// group layout writes partial cache lines and costs ~1.6x the bytes at HBM,
// so the tile goes through LDS (every 64 bytes padded by 16 so the writes are
// bank-conflict free) and is stored back as chunk c = lane + 64j (j = 0..3)
// of the row-major tile: each store instruction then covers whole rows.
// Row offsets travel through LDS too; a negative offset marks a row past the end.
constexpr int kTileBytes = 64 * 80;  // 64 lanes x (64 + 16 pad) bytes

// Both halves of a bf16 pair with every NaN rewritten as 0x7FC0.
__device__ __forceinline__ uint32_t canon_bf16x2(uint32_t p) {
  const uint32_t lo = p & 0xFFFFu, hi = p >> 16;
  return (((lo & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : lo) | ((((hi & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : hi) << 16);
}

__device__ __forceinline__ int tile_offset(int chunk) { return 16 * chunk + 16 * (chunk >> 2); }

template <int D>
__device__ __forceinline__ void store_tile(const uint32_t (&o)[16], uint16_t* base, int64_t my_off,
                                           uint8_t* tile, int64_t* offs, int lane, int g, int rw) {
  constexpr int CPR = D / 8;  // 16-byte chunks per bf16 row
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(tile + tile_offset(rw * CPR + 4 * g + j)) =
        make_uint4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
  if (g == 0) offs[rw] = my_off;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane + 64 * j;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + tile_offset(c));
    const int64_t off = offs[c / CPR];
    // streaming store at device scope (nt sc1): the bf16 output is not re-read
    // by this kernel, so it should not displace other data from the caches.
    // The compiler's own non-temporal store (nt alone) measured 0.7% slower
    // (557 against 552-554 us at d128, three alternating runs).  The compiler
    // does not count this store in its memory waits, which only makes the
    // waits of later loads stricter.
    if (off >= 0) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(base + off + 8 * (c % CPR)),
                   "v"(u32x4{v.x, v.y, v.z, v.w})
                   : "memory");
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Dequantize loops take kBatch rows per lane per pass and issue all their
// loads before any arithmetic: a lane reads only 12-36 packed bytes per row,
// so this keeps enough bytes in flight to cover HBM latency.
constexpr int kBatch = 4;

// Zero bytes that a dequantize lane reads in place of a row it must not read
// (past the end, or past a fetch window: such rows are not stored, or are
// stored as +0).  Every lane then issues the same loads whatever its rows, so
// the compiler can wait for each row's loads alone; with the loads in per-lane
// branches, the number of loads issued after a row's is not known, and its
// first use waits for every outstanding memory operation.  32 bytes cover the
// largest per-lane read (one group's int8 keys).
__device__ __attribute__((aligned(16))) uint32_t kZeroRow[8] = {};

// Row indices of one dequantize pass (kBatch rows per lane, `step` apart) and
// which of them are read: rows past the end are not, nor, in a windowed fetch,
// tokens at or past min(lens[s], capacity) (they come out as +0).  A fetch's
// lengths are all loaded before any is used, so one wait covers them.
template <int D>
__device__ __forceinline__ void pass_rows(const DequantArgs& a, uint32_t base, uint32_t step, int rw,
                                          int64_t (&irow)[kBatch], int64_t (&orow)[kBatch], bool (&act)[kBatch],
                                          bool (&live)[kBatch]) {
  uint32_t seq[kBatch], tok[kBatch];
  static_for<kBatch>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const uint32_t r = base + u * step + rw;
    act[u] = r < a.rows;
    uint32_t s, t, h;
    split_row(act[u] ? r : 0u, a.split, s, t, h);
    irow[u] = row_index(a.in, s, t, h);
    orow[u] = row_index(a.out, s, t, h);
    if (kChecked && act[u]) {
      // rows outside the extents: nothing is written, the first row is read
      act[u] = check_ok(orow[u] < a.out_ext, kChkDequantOut);
      if (!a.in_len) irow[u] = check_row(irow[u], a.in_ext, kChkDequantIn);
    }
    // computed here, before the pass's loads: left to the compiler, this
    // arithmetic sinks below them, and its 64-bit temporaries then share
    // registers with loaded values, which makes the first use of any row
    // wait for the loads of all rows
    asm volatile("" : "+v"(orow[u]));
    seq[u] = s;
    tok[u] = h;
    live[u] = act[u];
  });
  if (a.in_len) {
    int32_t len[kBatch];
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      len[u] = a.in_len[seq[u]];  // rows past the end use sequence 0's (not read)
    });
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      live[u] = act[u] && (int64_t)tok[u] < min((int64_t)len[u], (int64_t)a.in_cap);
      if (kChecked && live[u]) irow[u] = check_row(irow[u], a.in_ext, kChkDequantIn);
    });
  }
}

template <int D, int KB>
__device__ __forceinline__ void dequantize_keys_rows(const DequantArgs& a, uint32_t blk, uint32_t nblk,
                                                     uint8_t* tile, int64_t* offs) {
  using L = GroupLanes<D>;
  constexpr int G = D / kGroup;
  constexpr int KW = KB == 8 ? 8 : KB;  // packed words per lane
  const int lane = threadIdx.x & 63, g = L::group(lane), rw = L::row(lane);
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t step = nblk * 4u * L::RPW;
  for (uint32_t base = wave * L::RPW; base < a.rows; base += kBatch * step) {
    uint32_t wv[kBatch][KW];
    uint32_t sbits[kBatch], zbits[kBatch];  // raw fp16: converted only when used, so
                                            // every load of the pass is in flight first
    int64_t irow[kBatch], orow[kBatch];
    bool act[kBatch], live[kBatch];
    pass_rows<D>(a, base, step, rw, irow, orow, act, live);
    const uint8_t* const zrow = reinterpret_cast<const uint8_t*>(kZeroRow);
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const uint8_t* const q = live[u] ? a.k_q + irow[u] * (D * KB / 8) + 4 * KW * g : zrow;
      const uint16_t* const sp = live[u] ? a.k_scale + irow[u] * G + g : reinterpret_cast<const uint16_t*>(zrow);
      const uint16_t* const zp = live[u] ? a.k_zero + irow[u] * G + g : reinterpret_cast<const uint16_t*>(zrow);
      if constexpr (KB == 8) {
        const uint2* src = reinterpret_cast<const uint2*>(q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 v = src[i];
          wv[u][2 * i] = v.x;
          wv[u][2 * i + 1] = v.y;
        }
      } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(q);
#pragma unroll
        for (int i = 0; i < KB; ++i) wv[u][i] = src[i];
      }
      sbits[u] = *sp;
      zbits[u] = *zp;
    });
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      // every lane takes part in the tile exchange; rows that are not read
      // compute on zeros (+0 bits) and are stored as +0 or not at all
      const float s16 = canon_nan(f16_value(sbits[u])), z16 = canon_nan(f16_value(zbits[u]));
      float k[32];
      if constexpr (KB == 8) {
        if (__all(z16 == __builtin_rintf(z16))) {
          // Every zero point of the wave is an integer (or infinite), as the
          // quantizer writes them: idx + zero == (idx + 128) + (zero - 128)
          // exactly, both terms being integers far below 2^24, and the biased
          // byte converts in one instruction.
          const float zb = z16 - 128.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t b = wv[u][i] ^ 0x80808080u;
            k[4 * i] = ((float)(b & 0xFFu) + zb) * s16;
            k[4 * i + 1] = ((float)((b >> 8) & 0xFFu) + zb) * s16;
            k[4 * i + 2] = ((float)((b >> 16) & 0xFFu) + zb) * s16;
            k[4 * i + 3] = ((float)((b >> 24) & 0xFFu) + zb) * s16;
          }
        } else {
          // Any other fp16 zero point (a fraction, a subnormal, NaN): the
          // signed index is converted exactly and added in one rounding.
#pragma unroll
          for (int i = 0; i < 32; ++i)
            k[i] = ((float)(int32_t)(int8_t)(wv[u][i >> 2] >> (8 * (i & 3))) + z16) * s16;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int bit = KB * i, wd = bit >> 5, off = bit & 31;
          uint32_t v = wv[u][wd] >> off;
          if (off + KB > 32) v |= wv[u][wd + 1] << (32 - off);
          k[i] = ((float)(v & ((1u << KB) - 1)) + z16) * s16;
        }
      }
      uint32_t o[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = pack_bf16x2(k[2 * i], k[2 * i + 1]);
      // finite scale and zero give finite keys; a non-finite one can give a
      // NaN of any sign or payload (0 * Inf, Inf - Inf), written as 0x7FC0
      if (__any(!(__builtin_isfinite(s16) && __builtin_isfinite(z16)))) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = canon_bf16x2(o[i]);
      }
      store_tile<D>(o, a.k, act[u] ? orow[u] * D : -1, tile, offs, lane, g, rw);
    });
  }
}

// One value group back to bf16: centroid lookup, scale, transform,
// 1/sqrt(d), signs (applied to the rounded bf16 pair: an exact sign flip).
// CANON rewrites NaN halves to 0x7FC0 after the sign flip.
// With `rotated` the row stays in the rotated domain (centroid * scale, no
// transform, no signs); rows with `zero` are written as +0.
template <int D, int VB, bool CANON>
__device__ __forceinline__ void dequant_value_group(const uint32_t (&wv)[VB], float sc, const float* cen,
                                                    const uint32_t (&smask)[16], float rd, int lane,
                                                    int g, int rw, uint16_t* base, int64_t off,
                                                    uint8_t* tile, int64_t* offs, bool rotated, bool zero) {
  float z[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int bit = VB * i, wd = bit >> 5, off = bit & 31;
    uint32_t v;
    if (off + VB <= 32)
      v = __builtin_amdgcn_ubfe(wv[wd], off, VB);
    else
      v = (wv[wd] >> off) | ((wv[wd + 1] << (32 - off)) & ((1u << VB) - 1));
    z[i] = cen[v] * sc;
  }
  uint32_t o[16];
  if (rotated) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = pack_bf16x2(z[2 * i], z[2 * i + 1]);
  } else {
    const float m = fwht_group<D>(z, lane) * rd;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = pack_bf16x2(z[2 * i] * m, z[2 * i + 1] * m) ^ smask[i];
  }
  if (__any(zero)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = zero ? 0u : o[i];
  }
  if constexpr (CANON) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = canon_bf16x2(o[i]);
  }
  store_tile<D>(o, base, off, tile, offs, lane, g, rw);
}

template <int D, int VB>
__device__ __forceinline__ void dequantize_values_rows(const DequantArgs& a, uint32_t blk, uint32_t nblk,
                                                       uint8_t* tile, int64_t* offs) {
  using L = GroupLanes<D>;
  constexpr int G = D / kGroup;
  __shared__ float cen_lds[1 << VB];
  for (int i = threadIdx.x; i < (1 << VB); i += blockDim.x)
    cen_lds[i] = __uint_as_float(centroids<VB>()[i]);
  __syncthreads();
  const int lane = threadIdx.x & 63, g = L::group(lane), rw = L::row(lane);
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t step = nblk * 4u * L::RPW;
  uint32_t smask[16];
  {
    const uint4* sp = reinterpret_cast<const uint4*>(a.signs + kGroup * g);
    const uint4 s0 = sp[0], s1 = sp[1];
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = sw[i >> 1] >> (16 * (i & 1));
      smask[i] = ((word & 0x80u) << 8) | ((word & 0x8000u) << 16);
    }
  }
  const float rd = inv_sqrt_d<D>();
  for (uint32_t base = wave * L::RPW; base < a.rows; base += kBatch * step) {
    uint32_t wv[kBatch][VB];
    uint32_t sbits[kBatch];  // raw fp16, converted only when used
    int64_t irow[kBatch], orow[kBatch];
    bool act[kBatch], live[kBatch];
    pass_rows<D>(a, base, step, rw, irow, orow, act, live);
    const uint8_t* const zrow = reinterpret_cast<const uint8_t*>(kZeroRow);
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const uint32_t* const src = reinterpret_cast<const uint32_t*>(
          live[u] ? a.v_q + irow[u] * (D * VB / 8) + 4 * VB * g : zrow);
      const uint16_t* const sp = live[u] ? a.v_scale + irow[u] * G + g : reinterpret_cast<const uint16_t*>(zrow);
#pragma unroll
      for (int i = 0; i < VB; ++i) wv[u][i] = src[i];
      sbits[u] = *sp;
    });
    static_for<kBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      // the transform needs every lane of the row: inactive rows compute on
      // zeros and skip the store.  Only a non-finite scale can produce NaN;
      // such rows take the variant that keeps every NaN at 0x7FC0.
      const float sc = canon_nan(f16_value(sbits[u]));
      const bool rot = a.rotated != 0, zero = act[u] && !live[u];
      if (__any(!__builtin_isfinite(sc)))
        dequant_value_group<D, VB, true>(wv[u], sc, cen_lds, smask, rd, lane, g, rw, a.v,
                                         act[u] ? orow[u] * D : -1, tile, offs, rot, zero);
      else
        dequant_value_group<D, VB, false>(wv[u], sc, cen_lds, smask, rd, lane, g, rw, a.v,
                                          act[u] ? orow[u] * D : -1, tile, offs, rot, zero);
    });
  }
}

// One launch per call: even blocks stream key rows, odd blocks value rows,
// so both halves progress side by side over the whole grid.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  // two input tiles per wave (the current one and the next one in flight)
  __shared__ __attribute__((aligned(16))) uint8_t tile_lds[4 * 2 * kTile];
  const uint32_t blk = blockIdx.x >> 1, nblk = gridDim.x >> 1;
  if (blockIdx.x & 1)
    quantize_values_rows<D, VB>(a, blk, nblk, tile_lds);
  else
    quantize_keys_rows<D, KB>(a, blk, nblk, tile_lds);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  // output staging, one tile per wave, shared by the key and value halves
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][kTileBytes];
  __shared__ int64_t row_offs[4][GroupLanes<D>::RPW];
  uint8_t* const tile = tiles[threadIdx.x >> 6];
  int64_t* const offs = row_offs[threadIdx.x >> 6];
  // with one output skipped every block works on the other
  const bool both = a.k && a.v;
  const uint32_t blk = both ? blockIdx.x >> 1 : blockIdx.x;
  const uint32_t nblk = both ? gridDim.x >> 1 : gridDim.x;
  const bool values = both ? (blockIdx.x & 1) : (a.v != nullptr);
  if (values)
    dequantize_values_rows<D, VB>(a, blk, nblk, tile, offs);
  else
    dequantize_keys_rows<D, KB>(a, blk, nblk, tile, offs);
}

// ------------------------------------------------------------- dispatch
// Blocks per half: enough to cover the rows (4 waves of 64*32/d rows each,
// one chunk), capped so a block loops over several chunks on large inputs.
// Past 1,024 blocks, each block also gets at least `per_block` chunks: the
// dequantize loops take kBatch chunks per pass, and a block with fewer pays
// its set-up for little work (d = 512, 196,608 rows: 251 -> 109 us).
static unsigned blocks_per_half(uint32_t rows, int d, int max_blocks, uint32_t per_block) {
  const uint32_t rows_per_block = 4u * (64u * 32u / (uint32_t)d);
  const uint32_t need = (rows + rows_per_block - 1) / rows_per_block;
  uint32_t blocks = (need + per_block - 1) / per_block;
  if (blocks < 1024u) blocks = need < 1024u ? need : 1024u;
  if (blocks > (uint32_t)max_blocks) blocks = (uint32_t)max_blocks;
  return blocks < 1 ? 1u : blocks;
}

template <int D, int KB>
static void quant_vb(const QuantArgs& a, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 2: quantize_kernel<D, KB, 2><<<grid, 256, 0, st>>>(a); break;
    case 3: quantize_kernel<D, KB, 3><<<grid, 256, 0, st>>>(a); break;
    case 4: quantize_kernel<D, KB, 4><<<grid, 256, 0, st>>>(a); break;
    case 5: quantize_kernel<D, KB, 5><<<grid, 256, 0, st>>>(a); break;
    default: quantize_kernel<D, KB, 8><<<grid, 256, 0, st>>>(a); break;
  }
}

template <int D, int KB>
static void dequant_vb(const DequantArgs& a, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 2: dequantize_kernel<D, KB, 2><<<grid, 256, 0, st>>>(a); break;
    case 3: dequantize_kernel<D, KB, 3><<<grid, 256, 0, st>>>(a); break;
    case 4: dequantize_kernel<D, KB, 4><<<grid, 256, 0, st>>>(a); break;
    case 5: dequantize_kernel<D, KB, 5><<<grid, 256, 0, st>>>(a); break;
    default: dequantize_kernel<D, KB, 8><<<grid, 256, 0, st>>>(a); break;
  }
}

template <int D>
static hipError_t launch_quant_d(const QuantArgs& a, int kb, int vb, hipStream_t st, int max_blocks) {
  const dim3 grid(2 * blocks_per_half(a.rows, D, max_blocks, 1));
  switch (kb) {
    case 2: quant_vb<D, 2>(a, vb, grid, st); break;
    case 4: quant_vb<D, 4>(a, vb, grid, st); break;
    case 5: quant_vb<D, 5>(a, vb, grid, st); break;
    default: quant_vb<D, 8>(a, vb, grid, st); break;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dequant_d(const DequantArgs& a, int kb, int vb, hipStream_t st, int max_blocks) {
  const unsigned half = blocks_per_half(a.rows, D, max_blocks, kBatch);
  const dim3 grid((a.k && a.v) ? 2 * half : half);
  switch (kb) {
    case 2: dequant_vb<D, 2>(a, vb, grid, st); break;
    case 4: dequant_vb<D, 4>(a, vb, grid, st); break;
    case 5: dequant_vb<D, 5>(a, vb, grid, st); break;
    default: dequant_vb<D, 8>(a, vb, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks) {
  switch (d) {
    case 64: return launch_quant_d<64>(a, kb, vb, st, max_blocks);
    case 128: return launch_quant_d<128>(a, kb, vb, st, max_blocks);
    case 256: return launch_quant_d<256>(a, kb, vb, st, max_blocks);
    default: return launch_quant_d<512>(a, kb, vb, st, max_blocks);
  }
}

// ------------------------------------------------------ inverse rotation
// bf16 rows in the rotated domain back to the original one:
// out = signs * FWHT(in) / sqrt(d), the transform first and the signs last
// (TurboQuant page, "Deferred inverse FWHT": the attention output is
// un-rotated once per query row).  Same lane layout and tile stores as the
// value dequantizer; every row is read before its tile is written, so the
// call may work in place.
template <int D>
__global__ __launch_bounds__(256) void unrotate_kernel(UnrotateArgs a) {
  using L = GroupLanes<D>;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][kTileBytes];
  __shared__ int64_t row_offs[4][L::RPW];
  const int lane = threadIdx.x & 63, g = L::group(lane), rw = L::row(lane);
  uint8_t* tile = tiles[threadIdx.x >> 6];
  int64_t* offs = row_offs[threadIdx.x >> 6];
  const uint32_t wave = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t step = gridDim.x * 4u * L::RPW;
  uint32_t smask[16];
  {
    const uint4* sp = reinterpret_cast<const uint4*>(a.signs + kGroup * g);
    const uint4 s0 = sp[0], s1 = sp[1];
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = sw[i >> 1] >> (16 * (i & 1));
      smask[i] = ((word & 0x80u) << 8) | ((word & 0x8000u) << 16);
    }
  }
  const float rd = inv_sqrt_d<D>();
  for (uint32_t base = wave * L::RPW; base < a.rows; base += step) {
    const uint32_t r = base + rw;
    const bool act = r < a.rows;
    uint32_t s, t, h;
    split_row(act ? r : 0u, a.split, s, t, h);
    const int64_t irow = check_row(row_index(a.in_map, s, t, h), a.in_ext, kChkUnrotIn);
    const int64_t orow = row_index(a.out_map, s, t, h);
    const bool put = act && check_ok(orow < a.out_ext, kChkUnrotOut);
    uint32_t u[16];
    if (act) {
      load_group(a.in + irow * D + kGroup * g, u);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = 0;
    }
    float w[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[2 * i] = bf16_lo(u[i]);
      w[2 * i + 1] = bf16_hi(u[i]);
    }
    const float m = fwht_group<D>(w, lane) * rd;
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[i] = canon_bf16x2(pack_bf16x2(w[2 * i] * m, w[2 * i + 1] * m) ^ smask[i]);
    }
    store_tile<D>(o, a.out, put ? orow * D : -1, tile, offs, lane, g, rw);
  }
}

hipError_t launch_unrotate(const UnrotateArgs& a, int d, hipStream_t st, int max_blocks) {
  const int rows_per_block = 4 * (64 / (d / kGroup));
  long long blocks = ((long long)a.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > max_blocks) blocks = max_blocks;
  const dim3 grid((unsigned)blocks);
  switch (d) {
    case 64: unrotate_kernel<64><<<grid, 256, 0, st>>>(a); break;
    case 128: unrotate_kernel<128><<<grid, 256, 0, st>>>(a); break;
    case 256: unrotate_kernel<256><<<grid, 256, 0, st>>>(a); break;
    default: unrotate_kernel<512><<<grid, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

uint32_t check_read_clear_codec() { return check_read_clear_file(); }

hipError_t launch_dequantize(const DequantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks) {
  switch (d) {
    case 64: return launch_dequant_d<64>(a, kb, vb, st, max_blocks);
    case 128: return launch_dequant_d<128>(a, kb, vb, st, max_blocks);
    case 256: return launch_dequant_d<256>(a, kb, vb, st, max_blocks);
    default: return launch_dequant_d<512>(a, kb, vb, st, max_blocks);
  }
}

}  // namespace tq
