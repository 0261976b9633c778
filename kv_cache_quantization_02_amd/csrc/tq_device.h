// tq_device.h -- gfx950 device helpers shared by the codec and attention kernels.
//
// Lane layout of the row helpers below (used by the split attention kernel):
// a (token, kv-head) row of d elements is spread over d/8 consecutive lanes of
// a wave64, lane `sub` of the row holding elements 8*sub .. 8*sub+7 (one
// 16-byte bf16 load).  A
// 32-element group therefore lives in 4 consecutive lanes, and the
// Walsh-Hadamard stages h = 1, 2, 4 run inside a lane while h = 8 << k pairs
// lanes sub and sub ^ (1 << k).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kGroup = 32;

struct RowMap {
  int64_t seq_stride, tok_stride, head_stride;
};

// Exact unsigned division n / d for n < 2^31 by a multiply and a shift
// (Granlund & Montgomery 1994, Thm 4.2 with N = 31): m = ceil(2^(31+l) / d),
// l = ceil(log2 d), q = (m * n) >> (31 + l).
struct FastDiv {
  uint32_t mul;
  uint32_t shift;  // 31 + l
  uint32_t d;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)f.mul * n) >> f.shift);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
typedef float tq_float2 __attribute__((ext_vector_type(2)));
typedef __bf16 tq_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const tq_float2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, tq_bf16x2));
}

// fp16 pattern of a float, round to nearest even; every NaN -> 0x7E00.
__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = (_Float16)x;
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  return (x != x) ? 0x7E00u : b;
}

__device__ __forceinline__ float f16_value(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Replace any NaN by the default quiet NaN so that every NaN an output
// inherits from it rounds to the canonical bf16 NaN.
__device__ __forceinline__ float canon_nan(float x) {
  return (x != x) ? __uint_as_float(0x7FC00000u) : x;
}

// The value `x` held by lane (lane ^ M), for M a power of two below 64.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  int v = __float_as_int(x);
  if constexpr (M == 1) {
    v = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 8) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (M == 4 || M == 16) {
    v = __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1F);  // bit mode, xor M
  } else {
    static_assert(M == 32, "lane_xor: unsupported mask");
    v = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32u) << 2), v);
  }
  return __int_as_float(v);
}

// Walsh-Hadamard stages h = 1, 2, 4 on the 8 elements held by this lane:
// (u_i, u_{i+h}) <- (u_i + u_{i+h}, u_i - u_{i+h}).
__device__ __forceinline__ void fwht_in_lane(float (&y)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
  }
}

// Stage h = 8*M across lanes: the lane with bit M clear holds u_i and forms
// u_i + u_{i+h}; its partner holds u_{i+h} and forms u_i - u_{i+h}.  Both are
// one rounding of sgn*self + partner with sgn = +1 / -1 (fma is exact here).
template <int M>
__device__ __forceinline__ void fwht_cross(float (&y)[8], float sgn) {
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = __builtin_fmaf(sgn, y[i], lane_xor<M>(y[i]));
}

// All stages h = 1 .. D/2 in ascending order, for the layout above.
template <int D>
__device__ __forceinline__ void fwht_row(float (&y)[8], int sub) {
  fwht_in_lane(y);
  if constexpr (D >= 16) fwht_cross<1>(y, (sub & 1) ? -1.f : 1.f);
  if constexpr (D >= 32) fwht_cross<2>(y, (sub & 2) ? -1.f : 1.f);
  if constexpr (D >= 64) fwht_cross<4>(y, (sub & 4) ? -1.f : 1.f);
  if constexpr (D >= 128) fwht_cross<8>(y, (sub & 8) ? -1.f : 1.f);
  if constexpr (D >= 256) fwht_cross<16>(y, (sub & 16) ? -1.f : 1.f);
  if constexpr (D >= 512) fwht_cross<32>(y, (sub & 32) ? -1.f : 1.f);
}

// Float32 1/sqrt(d) for the supported head dims.
template <int D>
__device__ __forceinline__ float inv_sqrt_d() {
  if constexpr (D == 64) return __uint_as_float(0x3E000000u);
  else if constexpr (D == 128) return __uint_as_float(0x3DB504F3u);
  else if constexpr (D == 256) return __uint_as_float(0x3D800000u);
  else return __uint_as_float(0x3D3504F3u);
}

// The B*8 bits of this lane's 8 packed elements (stream bytes B*sub ..
// B*sub+B-1 of the row), loaded with naturally aligned accesses that never
// leave the row (row lengths are multiples of 8 bytes).
template <int B>
__device__ __forceinline__ uint64_t load_lane_bits(const uint8_t* row, int sub) {
  if constexpr (B == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * sub);
    return (uint64_t)w.x | ((uint64_t)w.y << 32);
  } else if constexpr (B == 4) {
    return *reinterpret_cast<const uint32_t*>(row + 4 * sub);
  } else if constexpr (B == 2) {
    return *reinterpret_cast<const uint16_t*>(row + 2 * sub);
  } else {
    const int off = B * sub;
    const int a = off & ~3;
    const int sh = (off & 3) * 8;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(row + a);
    uint32_t w1 = 0;
    if ((off & 3) + B > 4) w1 = *reinterpret_cast<const uint32_t*>(row + a + 4);
    return (((uint64_t)w1 << 32) | w0) >> sh;
  }
}

// Store the low B bytes of `bits` at stream bytes B*sub .. of the row.
template <int B>
__device__ __forceinline__ void store_lane_bits(uint8_t* row, int sub, uint64_t bits) {
  if constexpr (B == 8) {
    *reinterpret_cast<uint2*>(row + 8 * sub) = make_uint2((uint32_t)bits, (uint32_t)(bits >> 32));
  } else if constexpr (B == 4) {
    *reinterpret_cast<uint32_t*>(row + 4 * sub) = (uint32_t)bits;
  } else if constexpr (B == 2) {
    *reinterpret_cast<uint16_t*>(row + 2 * sub) = (uint16_t)bits;
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) row[B * sub + i] = (uint8_t)(bits >> (8 * i));
  }
}

// ------------------------------------------------------------ index bits
// Lloyd-Max index bits of two elements ya, yb of a 1-, 2-, 3- or 4-bit table,
// pushed into packed words.  Thresholds t[0] < ... < t[H-1] on |y|
// (H = 2^(VB-1) - 1) give c = #{t < |y|} by binary search; the index is then
// H + 1 + c for y > 0 and H - c otherwise, so its top bit is s = [y > 0] and
// bit k below it is (bit k of c) XNOR s.  Each bit is a lane mask, and it
// enters a word by w = 2 w + bit: one v_addc_co_u32 whose carry-in is the
// mask.  Bits are pushed from the highest stream position down, ya's
// (the higher element) first, so no bit is materialised, shifted or or-ed.
// The first NH pushes go to word wh, the rest to wl (a pair of 3-bit
// elements can straddle two words).
//
// Inline assembly because the compiler turns the plain-C form back into
// select + shift + or.  Every vector read of a mask written by a vector
// compare sits at least two instructions after it (the required wait
// states), and all masks are internal to the block.  The compiler does not
// add wait states in front of the block for its operands: ya and yb must not
// come straight from a matrix-core result (pass them through a vector
// operation first).
#define TQ_PUSH(W, M) "v_addc_co_u32 %[" #W "], vcc, %[" #W "], %[" #W "], %[" #M "]\n\t"

#define TQ_IDX1_BODY(W0, W1)                           \
  "v_cmp_lt_f32_e64 %[rsa], 0, %[ya]\n\t"              \
  "v_cmp_lt_f32_e64 %[rsb], 0, %[yb]\n\t"              \
  "s_nop 1\n\t"                                        \
  TQ_PUSH(W0, rsa) TQ_PUSH(W1, rsb)

#define TQ_IDX2_BODY(W0, W1, W2, W3)                   \
  "v_cmp_lt_f32_e64 %[rsa], 0, %[ya]\n\t"              \
  "v_cmp_lt_f32_e64 %[rsb], 0, %[yb]\n\t"              \
  "v_cmp_gt_f32_e64 %[r0a], |%[ya]|, %[t0]\n\t"        \
  "v_cmp_gt_f32_e64 %[r0b], |%[yb]|, %[t0]\n\t"        \
  "s_xnor_b64 %[r0a], %[r0a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r0b], %[r0b], %[rsb]\n\t"              \
  TQ_PUSH(W0, rsa) TQ_PUSH(W1, r0a) TQ_PUSH(W2, rsb) TQ_PUSH(W3, r0b)

#define TQ_IDX3_BODY(W0, W1, W2, W3, W4, W5)           \
  "v_cmp_gt_f32_e64 %[r1a], |%[ya]|, %[t1]\n\t"        \
  "v_cmp_gt_f32_e64 %[r1b], |%[yb]|, %[t1]\n\t"        \
  "v_cmp_lt_f32_e64 %[rsa], 0, %[ya]\n\t"              \
  "v_cndmask_b32_e64 %[ta], %[t0], %[t2], %[r1a]\n\t"  \
  "v_cmp_lt_f32_e64 %[rsb], 0, %[yb]\n\t"              \
  "v_cndmask_b32_e64 %[tb], %[t0], %[t2], %[r1b]\n\t"  \
  "v_cmp_gt_f32_e64 %[r0a], |%[ya]|, %[ta]\n\t"        \
  "v_cmp_gt_f32_e64 %[r0b], |%[yb]|, %[tb]\n\t"        \
  "s_xnor_b64 %[r1a], %[r1a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r0a], %[r0a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r1b], %[r1b], %[rsb]\n\t"              \
  "s_xnor_b64 %[r0b], %[r0b], %[rsb]\n\t"              \
  TQ_PUSH(W0, rsa) TQ_PUSH(W1, r1a) TQ_PUSH(W2, r0a)   \
  TQ_PUSH(W3, rsb) TQ_PUSH(W4, r1b) TQ_PUSH(W5, r0b)

#define TQ_IDX4_BODY                                    \
  "v_cmp_gt_f32_e64 %[r2a], |%[ya]|, %[t3]\n\t"        \
  "v_cmp_gt_f32_e64 %[r2b], |%[yb]|, %[t3]\n\t"        \
  "v_cmp_lt_f32_e64 %[rsa], 0, %[ya]\n\t"              \
  "v_cndmask_b32_e64 %[ta], %[t1], %[t5], %[r2a]\n\t"  \
  "v_cndmask_b32_e64 %[tb], %[t1], %[t5], %[r2b]\n\t"  \
  "v_cndmask_b32_e64 %[ua], %[t0], %[t4], %[r2a]\n\t"  \
  "v_cndmask_b32_e64 %[va], %[t2], %[t6], %[r2a]\n\t"  \
  "v_cmp_gt_f32_e64 %[r1a], |%[ya]|, %[ta]\n\t"        \
  "v_cndmask_b32_e64 %[ub], %[t0], %[t4], %[r2b]\n\t"  \
  "v_cndmask_b32_e64 %[vb], %[t2], %[t6], %[r2b]\n\t"  \
  "v_cmp_gt_f32_e64 %[r1b], |%[yb]|, %[tb]\n\t"        \
  "v_cmp_lt_f32_e64 %[rsb], 0, %[yb]\n\t"              \
  "v_cndmask_b32_e64 %[ta], %[ua], %[va], %[r1a]\n\t"  \
  "v_cndmask_b32_e64 %[tb], %[ub], %[vb], %[r1b]\n\t"  \
  "v_cmp_gt_f32_e64 %[r0a], |%[ya]|, %[ta]\n\t"        \
  "v_cmp_gt_f32_e64 %[r0b], |%[yb]|, %[tb]\n\t"        \
  "s_xnor_b64 %[r2a], %[r2a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r1a], %[r1a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r0a], %[r0a], %[rsa]\n\t"              \
  "s_xnor_b64 %[r2b], %[r2b], %[rsb]\n\t"              \
  "s_xnor_b64 %[r1b], %[r1b], %[rsb]\n\t"              \
  "s_xnor_b64 %[r0b], %[r0b], %[rsb]\n\t"              \
  TQ_PUSH(w, rsa) TQ_PUSH(w, r2a) TQ_PUSH(w, r1a) TQ_PUSH(w, r0a) \
  TQ_PUSH(w, rsb) TQ_PUSH(w, r2b) TQ_PUSH(w, r1b) TQ_PUSH(w, r0b)

template <int VB, int NH>
__device__ __forceinline__ void index_pair(float ya, float yb, const float* t, uint32_t& wh, uint32_t& wl) {
  uint64_t rsa, rsb, r0a, r0b;
  if constexpr (VB == 1) {
    static_assert(NH == 2, "1-bit pairs fill one word");
    asm(TQ_IDX1_BODY(w, w) : [w] "+v"(wh), [rsa] "=&s"(rsa), [rsb] "=&s"(rsb) : [ya] "v"(ya), [yb] "v"(yb) : "vcc");
    (void)t;
    (void)r0a;
    (void)r0b;
  } else if constexpr (VB == 2) {
    static_assert(NH == 4, "2-bit pairs fill one word");
    asm(TQ_IDX2_BODY(w, w, w, w)
        : [w] "+v"(wh), [rsa] "=&s"(rsa), [rsb] "=&s"(rsb), [r0a] "=&s"(r0a), [r0b] "=&s"(r0b)
        : [ya] "v"(ya), [yb] "v"(yb), [t0] "v"(t[0])
        : "vcc");
  } else if constexpr (VB == 3) {
    uint64_t r1a, r1b;
    float ta, tb;
#define TQ_IDX3_OPERANDS                                                                                   \
  [rsa] "=&s"(rsa), [rsb] "=&s"(rsb), [r0a] "=&s"(r0a), [r0b] "=&s"(r0b), [r1a] "=&s"(r1a), [r1b] "=&s"(r1b), \
      [ta] "=&v"(ta), [tb] "=&v"(tb)                                                                       \
      : [ya] "v"(ya), [yb] "v"(yb), [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2])                        \
      : "vcc"
    if constexpr (NH == 6)
      asm(TQ_IDX3_BODY(w, w, w, w, w, w) : [w] "+v"(wh), TQ_IDX3_OPERANDS);
    else if constexpr (NH == 4)
      asm(TQ_IDX3_BODY(wh, wh, wh, wh, wl, wl) : [wh] "+v"(wh), [wl] "+v"(wl), TQ_IDX3_OPERANDS);
    else if constexpr (NH == 2)
      asm(TQ_IDX3_BODY(wh, wh, wl, wl, wl, wl) : [wh] "+v"(wh), [wl] "+v"(wl), TQ_IDX3_OPERANDS);
    else
      static_assert(NH == 6, "3-bit pairs split 6, 4 + 2 or 2 + 4");
#undef TQ_IDX3_OPERANDS
  } else {
    static_assert(VB == 4 && NH == 8, "4-bit pairs fill one word");
    uint64_t r1a, r1b, r2a, r2b;
    float ta, tb, ua, ub, va, vb;
    asm(TQ_IDX4_BODY
        : [w] "+v"(wh), [rsa] "=&s"(rsa), [rsb] "=&s"(rsb), [r0a] "=&s"(r0a), [r0b] "=&s"(r0b), [r1a] "=&s"(r1a),
          [r1b] "=&s"(r1b), [r2a] "=&s"(r2a), [r2b] "=&s"(r2b), [ta] "=&v"(ta), [tb] "=&v"(tb), [ua] "=&v"(ua),
          [ub] "=&v"(ub), [va] "=&v"(va), [vb] "=&v"(vb)
        : [ya] "v"(ya), [yb] "v"(yb), [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]),
          [t4] "v"(t[4]), [t5] "v"(t[5]), [t6] "v"(t[6])
        : "vcc");
  }
}
#undef TQ_IDX1_BODY
#undef TQ_IDX2_BODY
#undef TQ_IDX3_BODY
#undef TQ_IDX4_BODY
#undef TQ_PUSH

}  // namespace tq
