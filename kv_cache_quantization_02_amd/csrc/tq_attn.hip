// tq_attn.hip -- fused dequant-on-fetch GQA decode attention over the
// quantized cache, split over the context ("split-K") plus a combine kernel.
//
// TurboQuant page, "Deferred inverse FWHT": attention is linear in V, so the
// values are accumulated in the rotated domain, z = centroid[idx] * scale16,
// and the output is un-rotated once per (sequence, query head):
//   out = signs * FWHT(sum_t p_t z_t / sum_t p_t) / sqrt(d).
// Keys are dequantized on the fly, k_hat = (idx + zero16) * scale16.
//
// Split kernel: one 256-thread block per (sequence, kv head, head tile,
// split).  Inside a wave, lane-group c (d/8 lanes) owns cache rows
// t = t0 + k*TPW + c; lane `sub` of the group holds elements 8*sub..8*sub+7 of
// the row, the matching slice of up to four query heads, and their
// rotated-domain accumulators.  Scores are kept in the log2 domain (the
// query is pre-multiplied by softmax_scale * log2(e)).  Each block writes
// one (m, l, acc[d]) partial per query head; the combine kernel merges the
// splits, applies the transform, the normalisation and the signs.
#include "tq_codebooks.h"
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

__constant__ uint32_t a_cen_2[4] = {TQ_CENTROIDS_2BIT};
__constant__ uint32_t a_cen_3[8] = {TQ_CENTROIDS_3BIT};
__constant__ uint32_t a_cen_4[16] = {TQ_CENTROIDS_4BIT};
__constant__ uint32_t a_cen_5[32] = {TQ_CENTROIDS_5BIT};
__constant__ uint32_t a_cen_8[256] = {TQ_CENTROIDS_8BIT};

template <int B>
__device__ __forceinline__ const uint32_t* attn_centroids() {
  if constexpr (B == 2) return a_cen_2;
  else if constexpr (B == 3) return a_cen_3;
  else if constexpr (B == 4) return a_cen_4;
  else if constexpr (B == 5) return a_cen_5;
  else return a_cen_8;
}

constexpr int kHeadTile = 4;   // query heads per block
// Rows per lane-group between softmax rescales (VALU kernel).  Two rows and
// 1024 blocks beat four rows and 2048 blocks by 12-30% (d = 512 k5v2 and k8v3
// over a 16 x 8 x 4096 cache 316 / 395 -> 277 / 277 us; d = 64 k5v3 over
// 16 x 8 x 16384 183 -> 145 us): fewer registers per wave and shorter chains.
constexpr int kChunk = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // log2 slack of the matrix-core kernel's running maximum

// One split partial per (sequence, query head): acc[d], m, l, two pad words
// (keeps every record 16-byte aligned).
template <int D>
constexpr int part_stride() { return D + 4; }

// x of another lane of the row, chosen by the DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over the D/8 lanes of a row, in every one of them.  The xor-4, -16 and
// -32 steps go through the LDS crossbar (swizzle, bpermute): the VALU kernel
// that uses this is bound by its VALU issue, and an all-VALU version (DPP
// mirrors, permlane swaps) was 2-6% slower at d = 512.
template <int D>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (D >= 16) v += lane_xor<1>(v);
  if constexpr (D >= 32) v += lane_xor<2>(v);
  if constexpr (D >= 64) v += lane_xor<4>(v);
  if constexpr (D >= 128) v += lane_xor<8>(v);
  if constexpr (D >= 256) v += lane_xor<16>(v);
  if constexpr (D >= 512) v += lane_xor<32>(v);
  return v;
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void decode_attn_split_kernel(AttnArgs a) {
  constexpr int LPR = D / 8, TPW = 64 / LPR, G = D / kGroup;
  constexpr int KROW = D * KB / 8, VROW = D * VB / 8;
  __shared__ float cen_lds[1 << VB];
  __shared__ float red[4][TPW][kHeadTile][D + 2];

  const int split = blockIdx.x % a.splits;
  int rest = blockIdx.x / a.splits;
  const int rep = a.n_q_heads / a.n_kv_heads, nrow = a.n_queries * rep;
  const int tiles = (nrow + kHeadTile - 1) / kHeadTile;
  const int tile = rest % tiles;
  rest /= tiles;
  const int g = rest % a.n_kv_heads;
  const int b = rest / a.n_kv_heads;

  for (int i = threadIdx.x; i < (1 << VB); i += blockDim.x)
    cen_lds[i] = __uint_as_float(attn_centroids<VB>()[i]);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, c = lane / LPR;

  int ctx = a.ctx_lens[check_row(b, a.batch, kChkAttnLen)];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t_begin = split * a.tokens_per_split;
  int t_end = t_begin + a.tokens_per_split;
  if (t_end > ctx) t_end = ctx;

  // query slice (pre-scaled into the log2 domain); tile row j is query
  // jr / rep, head jr % rep of this kv head, with jr = tile * kHeadTile + j
  const float qscale = a.softmax_scale * kLog2e;
  float q[kHeadTile][8];
  bool hv[kHeadTile];
  int lim[kHeadTile];  // tokens t < lim[j] are visible to row j
#pragma unroll
  for (int j = 0; j < kHeadTile; ++j) {
    const int jr = tile * kHeadTile + j;
    hv[j] = jr < nrow;
    const int mq = hv[j] ? jr / rep : 0, hq = g * rep + (hv[j] ? jr % rep : 0);
    lim[j] = ctx - a.n_queries + 1 + mq;
    const int64_t qr = check_row(((int64_t)b * a.n_queries + mq) * a.n_q_heads + hq,
                                 (int64_t)a.batch * a.n_queries * a.n_q_heads, kChkAttnQ);
    const uint4 w = *reinterpret_cast<const uint4*>(a.q + qr * D + 8 * sub);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[j][2 * i] = hv[j] ? bf16_lo(ws[i]) * qscale : 0.f;
      q[j][2 * i + 1] = hv[j] ? bf16_hi(ws[i]) * qscale : 0.f;
    }
  }
  __syncthreads();
  // per head, the sum of this lane's query elements: a lane's 8 key elements
  // share one group's scale and zero, so its partial score is
  // scale * (sum q * idx + zero * sum q)
  float qs[kHeadTile];
#pragma unroll
  for (int j = 0; j < kHeadTile; ++j) {
    qs[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) qs[j] += q[j][i];
  }

  float m[kHeadTile], l[kHeadTile], acc[kHeadTile][8];
#pragma unroll
  for (int j = 0; j < kHeadTile; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
  }

  const int64_t row0 = (int64_t)b * a.seq_stride + (int64_t)g * a.head_stride;
  constexpr int STEP = TPW * kChunk;  // rows per wave per chunk
  for (int t0 = t_begin + wave * STEP; t0 < t_end; t0 += 4 * STEP) {
    float sc[kChunk][kHeadTile];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const int t = t0 + k * TPW + c;
      const bool valid = t < t_end;
      float kx[8], s16 = 0.f, z16 = 0.f;  // indices, the group's scale and zero
      if (valid) {
        const int64_t row = check_row(row0 + t, a.cache_ext, kChkAttnCache);
        const uint64_t bits = load_lane_bits<KB>(a.k_q + row * KROW, sub);
        s16 = f16_value(a.k_scale[row * G + (sub >> 2)]);
        z16 = f16_value(a.k_zero[row * G + (sub >> 2)]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (KB == 8)
            kx[i] = (float)(int8_t)(bits >> (8 * i));
          else
            kx[i] = (float)(uint32_t)((bits >> (KB * i)) & ((1u << KB) - 1));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kx[i] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < kHeadTile; ++j) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = __builtin_fmaf(q[j][i], kx[i], d);
        d = row_sum<D>(s16 * __builtin_fmaf(z16, qs[j], d));
        sc[k][j] = (valid && t < lim[j]) ? d : -INFINITY;
      }
    }
    // softmax statistics for the chunk, then the rotated-domain accumulation
    float p[kChunk][kHeadTile];
#pragma unroll
    for (int j = 0; j < kHeadTile; ++j) {
      float cm = sc[0][j];
#pragma unroll
      for (int k = 1; k < kChunk; ++k) cm = fmaxf(cm, sc[k][j]);
      const float mn = fmaxf(m[j], cm);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m[j] - mn);
      float ps = 0.f;
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        p[k][j] = (sc[k][j] == -INFINITY) ? 0.f : exp2f(sc[k][j] - mn);
        ps += p[k][j];
      }
      l[j] = l[j] * alpha + ps;
      m[j] = mn;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j][i] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const int t = t0 + k * TPW + c;
      if (t < t_end) {
        const int64_t row = check_row(row0 + t, a.cache_ext, kChkAttnCache);
        const uint64_t bits = load_lane_bits<VB>(a.v_q + row * VROW, sub);
        const float vs = f16_value(a.v_scale[row * G + (sub >> 2)]);
        // the group's scale rides on the weights: p * scale, times the centroids
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = cen_lds[(bits >> (VB * i)) & ((1u << VB) - 1)];
#pragma unroll
        for (int j = 0; j < kHeadTile; ++j) {
          const float pv = p[k][j] * vs;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] = __builtin_fmaf(pv, z[i], acc[j][i]);
        }
      }
    }
  }

  // merge the TPW lane-groups of each wave and the four waves
#pragma unroll
  for (int j = 0; j < kHeadTile; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][c][j][8 * sub + i] = acc[j][i];
    if (sub == 0) {
      red[wave][c][j][D] = m[j];
      red[wave][c][j][D + 1] = l[j];
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < kHeadTile * D; o += blockDim.x) {
    const int j = o / D, e = o % D;
    const int jr = tile * kHeadTile + j;
    if (jr >= nrow) continue;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w)
      for (int cc = 0; cc < TPW; ++cc) mm = fmaxf(mm, red[w][cc][j][D]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < 4; ++w)
        for (int cc = 0; cc < TPW; ++cc) {
          const float f = exp2f(red[w][cc][j][D] - mm);
          ll += red[w][cc][j][D + 1] * f;
          aa += red[w][cc][j][e] * f;
        }
    }
    const int64_t orow = ((int64_t)b * a.n_queries + jr / rep) * a.n_q_heads + g * rep + jr % rep;
    const int64_t rec = orow * a.splits + split;
    if (!check_ok(rec < (int64_t)a.batch * a.n_queries * a.n_q_heads * a.splits, kChkAttnPart)) continue;
    float* part = a.part + rec * part_stride<D>();
    part[e] = aa;
    if (e == 0) {
      part[D] = mm;
      part[D + 1] = ll;
    }
  }
}

// ----------------------------------------------------------------------------
// Matrix-core split kernel (int8 keys, value widths 2..5, head_dim 64..256).
//
// Both contractions run on v_mfma_f32_16x16x32_f16 (gfx950 operand layout:
// A[l%16][8(l/16)+i], B[8(l/16)+i][l%16], D[4(l/16)+i][l%16] for lane l).
// A block of four waves serves one (sequence, kv head, tile of four query
// heads, context split); each wave takes 32 cached tokens per step.
//
// Memory: every byte a step reads (key rows, packed value rows, the three
// fp16 planes of its 32 tokens) is copied HBM -> LDS by global_load_lds DMA
// into per-wave stage buffers, S-1 steps ahead of use.  The copies hold no
// registers, so each wave keeps S-1 steps of loads in flight while it
// computes.  Stage layouts are chosen per DMA lane (the LDS side of a DMA is
// fixed at base + 4 * size * lane), so every lane's global offset depends on
// the lane only, except in the final partial step, whose rows beyond the
// context are clamped to its last row (their scores are masked and their
// value scales zeroed).
//  * QK^T: a key byte b (two's complement index) becomes the exact fp16
//    1024 + (b ^ 0x80); a group's contraction gives sum_j q_j (1152 + idx_j),
//    and scale * (idx + zero) . q follows with the group sums of q.  A is
//    block-diagonal over four groups (row 4 (g mod 4) + h); a lane's 16-byte
//    key chunk feeds two MFMAs, and A routes each element to its group's row.
//    Three permlane swaps sum the lane-groups' partials per head.
//  * The query is scaled by softmax_scale * log2 e and by a per-head power of
//    two that puts its largest element in [1/2, 1) before the fp16
//    conversion; the scores are scaled back exactly.
//  * Online softmax per head in the log2 domain, exact rescaling whenever
//    the running maximum moves.
//  * PV: A = p * value scale, B = fp16 centroids, accumulated in the rotated
//    domain.  The value scales of group g are multiplied by 2^-E_g, E_g the
//    least power of two above every scale of that group the wave has seen,
//    so the fp16 product never overflows and only terms below 2^-24 of the
//    largest lose bits; the group's accumulators are rescaled exactly when
//    E_g grows.  Column n of group g's two output tiles holds dims
//    32g + 2n and 32g + 2n + 1, so a lane's two indices per token are
//    adjacent bits of the packed row and one lookup yields both centroids.
//    Contraction index k = 8c + i stands for token c + 4i of the step, which
//    puts the four lane-groups' reads of the packed rows on distinct banks.
// The per-split (m, l, acc) partials are what the combine kernel expects.
typedef _Float16 tq_half8 __attribute__((ext_vector_type(8)));
typedef float tq_float4 __attribute__((ext_vector_type(4)));
typedef _Float16 tq_half2 __attribute__((ext_vector_type(2)));
typedef unsigned short tq_ushort2 __attribute__((ext_vector_type(2)));
typedef int tq_i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) float lds_f32;
typedef uint32_t tq_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tq_u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) tq_i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) tq_float4 lds_f32x4;
typedef __attribute__((address_space(3))) void lds_void;

// all-reduce over the 16 lanes of a row (quad xor 1, xor 2, rotate 4, rotate 8)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x128>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x128>(v);
  return v;
}

__device__ __forceinline__ uint32_t half2_bits(float lo, float hi) {
  const tq_float2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, tq_half2));
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(tq_half2, a) * __builtin_bit_cast(tq_half2, b));
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(tq_ushort2, a),
                                                                __builtin_bit_cast(tq_ushort2, b)));
}

// max over the lanes that share lane % M0 (M0 a power of two below 64)
template <int M>
__device__ __forceinline__ uint32_t xor_max_from(uint32_t v) {
  if constexpr (M < 64) {
    v = pk_max_u16(v, __float_as_uint(lane_xor<M>(__uint_as_float(v))));
    return xor_max_from<2 * M>(v);
  } else {
    return v;
  }
}

// fp16 pattern of 2^-e for e in [-13, 17] (the last three are subnormal)
__device__ __forceinline__ uint32_t f16_pow2_neg(int e) {
  return e <= 14 ? (uint32_t)(15 - e) << 10 : 1u << (24 - e);
}

template <int D, int KB, int VB>
struct MfmaCfg {
  static constexpr int G = D / kGroup, GW = G / 2, NSET = (G + 3) / 4, NT = D / 16, CH = 32;
  static constexpr int KRB = KB == 8 ? D : D * KB / 8;       // key row bytes
  // key chunks per row, and the span of their XOR swizzle (none for the
  // 5-chunk rows of 5-bit keys, which are read as unaligned fields)
  static constexpr int CPR = KRB / 16, SW = (CPR & (CPR - 1)) ? 1 : (CPR < 8 ? CPR : 8);
  static constexpr int W = D * VB / 32;                      // packed value dwords per row
  static constexpr int RB = 4 * W;                           // packed value bytes per row
  static constexpr int NK = (CH * KRB + 1023) / 1024;        // 16-byte DMAs of key rows
  static constexpr int NV = CH * W / 64;                     // 4-byte DMAs of value rows
  // value rows that fill whole 16-byte copies go 16 bytes per lane in every step
  static constexpr bool VX4 = (CH * RB) % 1024 == 0;
  static constexpr int NVX = CH * RB / 1024;
  static constexpr int SC_DW = CH * GW, NSP = (SC_DW + 63) / 64;  // per fp16 plane
  static constexpr int NI_TAIL = NK + (VX4 ? NVX : NV) + 3 * NSP;  // DMA instructions of a partial step
  // A full step can copy its value rows 16 bytes per lane.  When they leave
  // half an instruction over and the key scale and zero planes of the step
  // fill exactly that half (d = 128: 2 x 256 bytes), the last instruction's
  // upper 32 lanes copy those planes, which follow the value rows in the stage.
  static constexpr bool WIDE = (CH * RB) % 1024 == 512 && 2 * CH * 2 * G == 512;
  static constexpr int NVW = (CH * RB + 1023) / 1024;        // 16-byte DMAs of values (+ key planes)
  static constexpr int NI_FULL = WIDE ? NK + NVW + NSP : NI_TAIL;
  static constexpr int NI = NI_FULL < NI_TAIL ? NI_FULL : NI_TAIL;  // fewest per step (the waits count these)
  static constexpr int OFF_V = NK * 1024;  // key rows (5-bit keys: padded to whole copies)
  static constexpr int OFF_KS = OFF_V + CH * RB;
  static constexpr int OFF_KZ = OFF_KS + NSP * 256;
  static constexpr int OFF_VS = OFF_KZ + NSP * 256;
  static constexpr int STAGE = OFF_VS + NSP * 256;
  static constexpr int PB = 4 * CH;   // p[head][slot], then 32 zeros
  // centroid table: fp16 pairs for two indices of up to 5 bits, single fp16
  // entries for 8-bit indices
  static constexpr int LUT = VB == 8 ? 256 : 1 << (2 * VB);
  static constexpr int LUT_BYTES = VB == 8 ? 2 * LUT : 4 * LUT;
  static constexpr int OFF_PB = LUT_BYTES > 256 ? LUT_BYTES : 256;
  static constexpr int OFF_STATS = OFF_PB + 4 * (PB + 32) * 4;
  static constexpr int OFF_BUF = OFF_STATS + 4 * 4 * 2 * 4;
  static constexpr int EXTRA = OFF_BUF + 1024;
  // three stages when two blocks still fit a CU, else two
  static constexpr int S = (4 * 3 * STAGE + EXTRA <= 81920 && 2 * NI_TAIL <= 63) ? 3 : 2;
  static constexpr int ACC_BYTES = 4 * NT * 4 * 64 * 4;
  static constexpr int BUF = (4 * S * STAGE > ACC_BYTES) ? 4 * S * STAGE : ACC_BYTES;
  static_assert(G % 2 == 0 && (CH * W) % 64 == 0 && KRB % 16 == 0, "step layout");
  static_assert((S - 1) * NI_TAIL <= 63, "vmcnt range");
};

// One DMA instruction: each lane copies `size` bytes from base + voff to LDS
// byte lds + size * lane.  Written as inline assembly so that the compiler
// neither tracks these LDS writes (it would wait for every outstanding copy
// before each LDS read) nor moves them; completion is awaited explicitly with
// s_waitcnt vmcnt before a stage is read.  M0 (the LDS base of the copy) is
// reserved by the compiler and read by no other instruction of this kernel;
// each statement sets it immediately before its own copy.  The copies are
// non-temporal (nt): every cached byte is read once per call, and keeping it
// out of the caches took the 16 x 8 x 32768 decode from 166-167 to 155-156 us
// (three alternating runs of the bench step, same box) without slowing the
// codec kernels around it.
__device__ __forceinline__ void dma_x4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_x1(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
// 16 bytes per lane from a per-lane 64-bit address.
__device__ __forceinline__ void dma_x4_addr(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(addr), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// Key indices as MFMA operand bytes.  int8 keys are the stored bytes; packed
// unsigned 4- and 2-bit keys are spread into bytes in an order of their own
// (no shuffling), and the query operand is built in the same order
// (key_elem*: the element held at operand byte i), which leaves the
// contraction unchanged.  The fields of a little-endian stream sit at bit
// KB * e of its words.
template <int KB>
constexpr int key_elem16(int i) {
  return (KB == 8 || KB == 5) ? i : KB == 4 ? ((i >> 3) << 3) + 2 * (i & 3) + ((i >> 2) & 1) : 4 * (i & 3) + (i >> 2);
}
template <int KB>
constexpr int key_elem8(int i) {
  return KB == 8 ? i : 2 * (i & 3) + (i >> 2);
}
// 16 indices from the bytes at p (16, 8 or 4 of them)
template <int KB>
__device__ __forceinline__ tq_i32x4 keys16(const lds_u8* p) {
  if constexpr (KB == 8) {
    return *(const lds_i32x4*)p;
  } else if constexpr (KB == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)p;
    const uint32_t m = 0x0F0F0F0Fu;
    return tq_i32x4{(int)(w.x & m), (int)((w.x >> 4) & m), (int)(w.y & m), (int)((w.y >> 4) & m)};
  } else {
    static_assert(KB == 2, "packed keys of 4 or 2 bits");
    const uint32_t w = *(const lds_u32*)p, m = 0x03030303u;
    return tq_i32x4{(int)(w & m), (int)((w >> 2) & m), (int)((w >> 4) & m), (int)((w >> 6) & m)};
  }
}
// 16 five-bit indices: the 10 bytes at byte bo of a key row (bo even).  The
// operand's dword k holds elements 4k .. 4k + 3 in its bytes.
__device__ __forceinline__ tq_i32x4 keys16_5(const lds_u8* row, int bo) {
  const lds_u32* w = (const lds_u32*)(row + (bo & ~3));
  const uint32_t sh = (uint32_t)(bo & 3) * 8u;  // 0 or 16
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  const uint32_t x = __builtin_amdgcn_alignbit(w1, w0, sh);  // field bits 0 .. 31
  const uint32_t y = __builtin_amdgcn_alignbit(w2, w1, sh);  // 32 .. 63
  const uint32_t z = w2 >> sh;                                // 64 .. 79 (low half)
  uint32_t e[16];
#pragma unroll
  for (int j = 0; j < 6; ++j) e[j] = (x >> (5 * j)) & 31u;
  e[6] = __builtin_amdgcn_alignbit(y, x, 30) & 31u;
#pragma unroll
  for (int j = 7; j < 12; ++j) e[j] = (y >> (5 * j - 32)) & 31u;
  e[12] = __builtin_amdgcn_alignbit(z, y, 28) & 31u;
#pragma unroll
  for (int j = 13; j < 16; ++j) e[j] = (z >> (5 * j - 64)) & 31u;
  tq_i32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = (int)(e[4 * k] | (e[4 * k + 1] << 8) | (e[4 * k + 2] << 16) | (e[4 * k + 3] << 24));
  return r;
}

// 8 indices from the bytes at p (8 or 4 of them)
template <int KB>
__device__ __forceinline__ long keys8(const lds_u8* p) {
  if constexpr (KB == 8) {
    return *(const __attribute__((address_space(3))) long*)p;
  } else {
    static_assert(KB == 4, "the sixteen-row kernel takes 8- and 4-bit keys");
    const uint32_t w = *(const lds_u32*)p, m = 0x0F0F0F0Fu;
    return (long)(((uint64_t)((w >> 4) & m) << 32) | (w & m));
  }
}

// The block's centroid table in LDS: for value widths up to 5 bits the fp16
// pair (centroid[i & (2^VB - 1)], centroid[i >> VB]) at word i, so that one
// lookup of two adjacent indices yields both; for 8-bit values the fp16
// centroid[i] at half-word i.
template <int VB>
__device__ __forceinline__ void fill_centroid_lut(uint8_t* lds) {
  const uint32_t* cen = attn_centroids<VB>();
  if constexpr (VB == 8) {
    uint16_t* t = reinterpret_cast<uint16_t*>(lds);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) t[i] = (uint16_t)half2_bits(__uint_as_float(cen[i]), 0.f);
  } else {
    uint32_t* t = reinterpret_cast<uint32_t*>(lds);
    for (int i = threadIdx.x; i < (1 << (2 * VB)); i += blockDim.x)
      t[i] = half2_bits(__uint_as_float(cen[i & ((1 << VB) - 1)]), __uint_as_float(cen[i >> VB]));
  }
}

// PV B operands of one group: the fp16 centroids at this lane's two dims for
// the 8 tokens of its contraction slots (f[i]: the first value dword of
// token i's group at the lane's field; fsh: the field's bit offset).  b0
// feeds tile 2g (dim 2n), b1 tile 2g+1 (dim 2n+1).
template <int VB, int LUT>
__device__ __forceinline__ void centroid_operands(const lds_u32* const (&f)[8], uint32_t fsh, const lds_u8* lut,
                                                  uint32_t (&b0)[4], uint32_t (&b1)[4]) {
  if constexpr (VB == 8) {
    // two byte indices side by side: one table read each
    uint32_t L0[8], L1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t x = f[i][0] >> fsh;
      L0[i] = *(const __attribute__((address_space(3))) uint16_t*)(lut + ((x << 1) & 0x1FEu));
      L1[i] = *(const __attribute__((address_space(3))) uint16_t*)(lut + ((x >> 7) & 0x1FEu));
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      b0[m] = __builtin_amdgcn_perm(L0[2 * m + 1], L0[2 * m], 0x05040100u);
      b1[m] = __builtin_amdgcn_perm(L1[2 * m + 1], L1[2 * m], 0x05040100u);
    }
  } else {
    uint32_t L[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t x = __builtin_amdgcn_alignbit(f[i][1], f[i][0], fsh);
      L[i] = *(const lds_u32*)(lut + (x & ((uint32_t)(LUT - 1) << 2)));
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      b0[m] = __builtin_amdgcn_perm(L[2 * m + 1], L[2 * m], 0x05040100u);
      b1[m] = __builtin_amdgcn_perm(L[2 * m + 1], L[2 * m], 0x07060302u);
    }
  }
}

// Issue the DMAs of the step whose first row is r0 into `stage`.  TAIL: only
// the first tl rows are inside the context; later rows re-read row tl - 1.
template <int D, int KB, int VB, bool TAIL>
__device__ __forceinline__ void attn_dma(const AttnArgs& a, lds_u8* stage, int64_t r0, int tl, int lane) {
  using C = MfmaCfg<D, KB, VB>;
  // the step's rows r0 .. r0 + (TAIL ? tl : CH) - 1 (checked build: a step
  // past the cache's extent copies its first rows instead)
  if (!check_ok(r0 + (TAIL ? tl : C::CH) <= a.cache_ext, kChkAttnCache)) r0 = 0;
  const uint8_t* kb = a.k_q + r0 * C::KRB;
#pragma unroll
  for (int j = 0; j < C::NK; ++j) {
    // lanes past the step's key chunks (5-bit keys) re-read the last one into the padding
    const int s = min(64 * j + lane, C::CH * C::CPR - 1);
    int t = s / C::CPR;
    const int ch = (s % C::CPR) ^ (t & (C::SW - 1));
    if (TAIL) t = min(t, tl - 1);
    dma_x4(kb, (uint32_t)(t * C::KRB + 16 * ch), lds_addr(stage + 1024 * j));
  }
  if (C::WIDE && !TAIL && a.wide) {
    // value rows, then (upper lanes of the last copy) the key scale and zero planes
    const uint8_t* const vb = a.v_q + r0 * C::RB;
#pragma unroll
    for (int j = 0; j < C::NVW; ++j) {
      const int s = 64 * j + lane;
      const void* src = vb + 16 * s;
      if (j == C::NVW - 1 && lane >= 32) {
        const uint16_t* const pl = lane < 48 ? a.k_scale : a.k_zero;
        src = reinterpret_cast<const uint8_t*>(pl + r0 * C::G) + 16 * (lane & 15);
      }
      dma_x4_addr(src, lds_addr(stage + C::OFF_V + 1024 * j));
    }
    const uint16_t* const vs = a.v_scale + r0 * C::G;
#pragma unroll
    for (int j = 0; j < C::NSP; ++j) {
      int s = 64 * j + lane;
      if (s >= C::SC_DW) s = C::SC_DW - 1;
      dma_x1(vs, (uint32_t)(4 * s), lds_addr(stage + C::OFF_VS + 256 * j));
    }
    return;
  }
  const uint8_t* vb = a.v_q + r0 * C::RB;
  if constexpr (C::VX4) {
#pragma unroll
    for (int j = 0; j < C::NVX; ++j) {
      const int s = 64 * j + lane;
      int off = 16 * s;
      if (TAIL) {
        const int t = off / C::RB;
        off = min(t, tl - 1) * C::RB + (off - t * C::RB);
      }
      dma_x4(vb, (uint32_t)off, lds_addr(stage + C::OFF_V + 1024 * j));
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::NV; ++j) {
      const int s = 64 * j + lane;
      int off = 4 * s;
      if (TAIL) {
        const int t = s / C::W;
        off = 4 * (min(t, tl - 1) * C::W + (s - t * C::W));
      }
      dma_x1(vb, (uint32_t)off, lds_addr(stage + C::OFF_V + 256 * j));
    }
  }
  const uint16_t* planes[3] = {a.k_scale, a.k_zero, a.v_scale};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const uint16_t* pbase = planes[p] + r0 * C::G;
#pragma unroll
    for (int j = 0; j < C::NSP; ++j) {
      int s = 64 * j + lane;
      if (s >= C::SC_DW) s = C::SC_DW - 1;
      int t = s / C::GW;
      const int w = s - t * C::GW;
      if (TAIL) t = min(t, tl - 1);
      dma_x1(pbase, (uint32_t)(4 * (t * C::GW + w)), lds_addr(stage + C::OFF_KS + p * C::NSP * 256 + 256 * j));
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Value scales of one step, in the stage: rows past the context are zeroed;
// E_g (the least power of two above every scale of group g the wave has
// seen) is raised where a scale needs it, rescaling the group's accumulators
// exactly; the scales are rewritten in place as fp16 pairs of consecutive
// contraction slots (dword (slot / 2) * G + g holds slots 2k, 2k + 1 of
// group g), multiplied by 2^-E_g, so that the PV A operand reads them as they
// are.  slot_of(t) is token t's contraction slot.
template <int D, int KB, int VB, typename SlotOf>
__device__ __forceinline__ void stage_value_scales(lds_u8* sp, bool full, int tl, int lane, int (&E)[D / kGroup],
                                                   tq_float4 (&acc)[D / 16], SlotOf slot_of) {
  using C = MfmaCfg<D, KB, VB>;
  constexpr int G = C::G, GW = C::GW;
  lds_u32* const vs = (lds_u32*)(sp + C::OFF_VS);
  constexpr int PER = (C::SC_DW + 63) / 64;
  uint32_t x[PER], mx = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    x[k] = d < C::SC_DW ? vs[d] : 0u;
    if (!full && d / GW >= tl) x[k] = 0u;
    mx = pk_max_u16(mx, x[k] & 0x7FFF7FFFu);
  }
  // E_g only grows when a scale of group g has an exponent field of at
  // least E_g + 15, i.e. |bits| > ((E_g + 15) << 10) - 1: after the first
  // steps that is rare, so the exact cross-lane maximum is taken only
  // when some lane sees such a scale
  uint32_t lim[GW];
#pragma unroll
  for (int w = 0; w < GW; ++w)
    lim[w] = (uint32_t)(((E[2 * w] + 15) << 10) - 1) | ((uint32_t)(((E[2 * w + 1] + 15) << 10) - 1) << 16);
  bool over = false;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int w = (lane + 64 * k) % GW;
    uint32_t l = lim[0];
#pragma unroll
    for (int i = 1; i < GW; ++i)
      if (w == i) l = lim[i];
    over = over || pk_max_u16(x[k] & 0x7FFF7FFFu, l) != l;
  }
  if (__any(over)) {
    mx = xor_max_from<GW>(mx);
#pragma unroll
    for (int w = 0; w < GW; ++w) {
      const uint32_t mw = __builtin_amdgcn_readlane(mx, w);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int g = 2 * w + hf;
        const int ex = (int)((mw >> (16 * hf + 10)) & 31u);
        const int en = (ex > 1 ? ex : 1) - 14;
        if (en > E[g]) {
          const float f = ldexpf(1.f, E[g] - en);
          acc[2 * g] *= f;
          acc[2 * g + 1] *= f;
          E[g] = en;
        }
      }
    }
  }
  uint32_t rp[GW];
#pragma unroll
  for (int w = 0; w < GW; ++w) rp[w] = f16_pow2_neg(E[2 * w]) | (f16_pow2_neg(E[2 * w + 1]) << 16);
  lds_u16* const vs16 = (lds_u16*)vs;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    const int t = d / GW, w = d % GW;
    uint32_t rpl = rp[0];
#pragma unroll
    for (int i = 1; i < GW; ++i)
      if (w == i) rpl = rp[i];
    const uint32_t y = pk_mul_f16(x[k], rpl);
    const int u = slot_of(t);
    const int o = 2 * ((u >> 1) * G + 2 * w) + (u & 1);
    if (d < C::SC_DW) {
      vs16[o] = (uint16_t)y;
      vs16[o + 2] = (uint16_t)(y >> 16);
    }
  }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_attn_mfma_kernel(AttnArgs a) {
  using C = MfmaCfg<D, KB, VB>;
  constexpr int G = C::G, NSET = C::NSET, NT = C::NT, CH = C::CH, W = C::W, S = C::S;
  // one LDS block: the centroid-pair table first (its byte offsets are the
  // masked index bits themselves), then p, the merge statistics, the stages
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[C::OFF_BUF + C::BUF];
  float(*const stats)[4][2] = reinterpret_cast<float(*)[4][2]>(lds_all + C::OFF_STATS);
  uint8_t* const smem = lds_all + C::OFF_BUF;

  const int rep = a.n_q_heads / a.n_kv_heads, nrow = a.n_queries * rep;
  const int tiles = (nrow + kHeadTile - 1) / kHeadTile;
  // The tiles of one (sequence, kv head, split) stream the same cache rows.
  // Blocks are dealt to the 8 XCDs round robin (block i to XCD i mod 8), so
  // when the grid allows, the tiles of a group take blocks 8 apart: they run
  // on one XCD, together, and the later tiles find the rows in its L2.
  int group, tile;
  if (tiles > 1 && gridDim.x % (8u * tiles) == 0) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    tile = j % tiles;
    group = (j / tiles) * 8 + xcd;
  } else {
    tile = (blockIdx.x / a.splits) % tiles;
    group = (blockIdx.x / a.splits / tiles) * a.splits + blockIdx.x % a.splits;
  }
  const int split = group % a.splits;
  int rest = group / a.splits;
  const int gkv = rest % a.n_kv_heads;
  const int b = rest / a.n_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int c = lane >> 4, n = lane & 15, r = n >> 2, hh = n & 3;
  lds_u8* const wbuf = (lds_u8*)smem + wave * S * C::STAGE;
  lds_f32* const pb = (lds_f32*)(lds_all + C::OFF_PB) + wave * (C::PB + 32);
  lds_u8* const lut = (lds_u8*)lds_all;

  fill_centroid_lut<VB>(lds_all);
  if (lane < 32) pb[C::PB + lane] = 0.f;

  int ctx = a.ctx_lens[check_row(b, a.batch, kChkAttnLen)];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t_begin = split * a.tokens_per_split;
  int t_end = t_begin + a.tokens_per_split;
  if (t_end > ctx) t_end = ctx;
  const int64_t row0 = (int64_t)b * a.seq_stride + (int64_t)gkv * a.head_stride;

  // start the first S-1 steps' copies before the query set-up
  const int first = t_begin + wave * CH;
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    const int cb = first + 4 * CH * k;
    if (cb + CH <= t_end)
      attn_dma<D, KB, VB, false>(a, wbuf + k * C::STAGE, row0 + cb, CH, lane);
    else if (cb < t_end)
      attn_dma<D, KB, VB, true>(a, wbuf + k * C::STAGE, row0 + cb, t_end - cb, lane);
  }

  // ---- query
  const float qscale = a.softmax_scale * kLog2e;
  // tile row h is query jr / rep, head jr % rep of this kv head (jr = tile * 4 + h)
  auto qhead = [&](int h) -> const uint16_t* {
    const int jr = tile * kHeadTile + h;
    const int mq = jr < nrow ? jr / rep : 0, hq = gkv * rep + (jr < nrow ? jr % rep : 0);
    return a.q + check_row(((int64_t)b * a.n_queries + mq) * a.n_q_heads + hq,
                           (int64_t)a.batch * a.n_queries * a.n_q_heads, kChkAttnQ) * D;
  };
  auto hvalid = [&](int h) { return tile * kHeadTile + h < nrow; };
  // per-head power of two (lane-group c measures head c)
  float qmax = 0.f;
  if (hvalid(c)) {
    const uint16_t* qp = qhead(c) + n * (D / 16);
#pragma unroll
    for (int i = 0; i < D / 16; i += 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(qp + i);
      qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w))));
    }
  }
  qmax = row16_max(qmax) * fabsf(qscale);
  int qe = 0;
  (void)frexpf(qmax, &qe);
  qe = qe < -100 ? -100 : (qe > 100 ? 100 : qe);
  // The query enters the int8 MFMA as the exact pair hi * 256 + lo of the
  // fixed-point value q * softmax_scale * log2 e * 2^(14 - qe), |.| <= 2^14,
  // hi in [-64, 64], lo in [-128, 127]; the key bytes are the B operand as
  // stored.  Scores come back to scale through 2^(qe - 14).
  const float smul = ldexpf(1.f, qe - 14);
  // tokens visible to this lane-group's row (lane-group c holds row c's scores)
  int lim_c;
  {
    const int jr = tile * kHeadTile + c;
    lim_c = ctx - a.n_queries + 1 + (jr < nrow ? jr / rep : 0);
    if (lim_c > t_end) lim_c = t_end;
  }
  float qn[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) qn[h] = ldexpf(qscale, 14 - __builtin_amdgcn_readlane(qe, 16 * h));
  const float qn_l = hh == 0 ? qn[0] : (hh == 1 ? qn[1] : (hh == 2 ? qn[2] : qn[3]));
  auto qfix = [](float x) { return (int)__builtin_rintf(x); };
  // A operands: MFMA gp takes key bytes 64gp + 16c + i (i < 16), of group
  // 2gp + c/2, routed to row 4 ((2gp + c/2) mod 4) + h
  tq_i32x4 aqh[G / 2], aql[G / 2];
#pragma unroll
  for (int gp = 0; gp < G / 2; ++gp) {
    const int g = 2 * gp + (c >> 1);
    const bool on = ((g & 3) == r) && hvalid(hh);
    const uint16_t* qp = qhead(hh) + 64 * gp + 16 * c;
    const uint4 w0 = on ? *reinterpret_cast<const uint4*>(qp) : make_uint4(0, 0, 0, 0);
    const uint4 w1 = on ? *reinterpret_cast<const uint4*>(qp + 8) : make_uint4(0, 0, 0, 0);
    const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t hw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = key_elem16<KB>(i);  // the key operand's element at byte i
      const float x = (e & 1) ? bf16_hi(ws[e >> 1]) : bf16_lo(ws[e >> 1]);
      const int v = qfix(x * qn_l);
      const int lo = ((v + 128) & 255) - 128;
      const int hi = (v - lo) >> 8;
      hw[i >> 2] |= (uint32_t)(hi & 255) << (8 * (i & 3));
      lw[i >> 2] |= (uint32_t)(lo & 255) << (8 * (i & 3));
    }
    aqh[gp] = tq_i32x4{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
    aql[gp] = tq_i32x4{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
  }
  // per-group sums of the fixed-point query (exact integers)
  float qsum[NSET][4];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int g = 4 * st + c;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      int acc = 0;
      if (g < G && hvalid(h)) {
        const uint4* p = reinterpret_cast<const uint4*>(qhead(h) + kGroup * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 w = p[j];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) acc += qfix(bf16_lo(ws[i]) * qn[h]) + qfix(bf16_hi(ws[i]) * qn[h]);
        }
      }
      qsum[st][h] = (float)acc;
    }
  }
  // value fields: dims 32g + 2n, +1 sit at bits 2VB n of group g's segment;
  // read the dword pair whose funnel shift leaves them at bit 2
  int fk = (2 * VB * n) >> 5, fsh = (2 * VB * n) & 31;
  if constexpr (VB != 8) {
    // the pair's bits go to bit 2 of the table's byte offset
    if (fsh < 2) {
      fk -= 1;
      fsh += 30;
    } else {
      fsh -= 2;
    }
  }
  const int vdw = C::OFF_V / 4 + c * W + fk;  // + 4W i + VB g for token c + 4i, group g
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  tq_float4 acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = tq_float4{0.f, 0.f, 0.f, 0.f};
  int E[G];
#pragma unroll
  for (int g = 0; g < G; ++g) E[g] = -13;

  int slot = 0;
  for (int cb = first; cb < t_end; cb += 4 * CH) {
    // copies of the step S-1 ahead go into the slot freed by the previous step
    const int cbn = cb + 4 * CH * (S - 1);
    const int nslot = slot == 0 ? S - 1 : slot - 1;
    if (cbn + CH <= t_end)
      attn_dma<D, KB, VB, false>(a, wbuf + nslot * C::STAGE, row0 + cbn, CH, lane);
    else if (cbn < t_end)
      attn_dma<D, KB, VB, true>(a, wbuf + nslot * C::STAGE, row0 + cbn, t_end - cbn, lane);
    const int later = (t_end - cb - 1) / (4 * CH);  // steps after this one
    if (later >= 2 && S == 3)
      wait_vmcnt<(S - 1) * C::NI>();
    else if (later >= 1)
      wait_vmcnt<C::NI>();
    else
      wait_vmcnt<0>();

    lds_u8* const sp = wbuf + slot * C::STAGE;
    slot = slot == S - 1 ? 0 : slot + 1;
    const int tl = t_end - cb;
    const bool full = tl >= CH;

    // ---- value scales: zero rows past the context, track E_g, normalise,
    // and rewrite them in place as fp16 pairs (slot 2k, slot 2k+1) per group,
    // slot 8 (t mod 4) + t / 4 for token t: the A operand of PV reads them as is
    stage_value_scales<D, KB, VB>(sp, full, tl, lane, E, acc, [](int t) { return 8 * (t & 3) + (t >> 2); });

    // ---- scores for the two 16-token tiles
    const lds_u16* const ks = (const lds_u16*)(sp + C::OFF_KS);
    const lds_u16* const kz = (const lds_u16*)(sp + C::OFF_KZ);
    float Sc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = 16 * tau + n;
      float T[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSET; ++st) {
        tq_i32x4 dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
          const int gp = 2 * st + gq;
          if (gp < G / 2) {
            // this lane's 16 key indices: elements 64 gp + 16 c .. + 15 of the row
            constexpr int BO = 16 * KB / 8;  // their packed bytes
            const int bo = (4 * gp + c) * BO, ch = bo >> 4;
            tq_i32x4 kw;
            if constexpr (KB == 5)
              kw = keys16_5(sp + t * C::KRB, bo);
            else
              kw = keys16<KB>(sp + 16 * (t * C::CPR + (ch ^ (t & (C::SW - 1)))) + (bo & 15));
            dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(aqh[gp], kw, dh, 0, 0, 0);
            dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(aql[gp], kw, dl, 0, 0, 0);
          }
        }
        const int g = 4 * st + c;
        float sk = 0.f, zk = 0.f;
        if (g < G) {
          sk = f16_value(ks[t * G + g]);
          zk = f16_value(kz[t * G + g]);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float d = (float)(dh[h] * 256 + dl[h]);  // exact: |.| < 2^29
          T[h] = __builtin_fmaf(sk, __builtin_fmaf(zk, qsum[st][h], d), T[h]);
        }
      }
      // lane-group h collects head h: sum over the four lane-groups
      const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[0]), __float_as_uint(T[2]), false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[1]), __float_as_uint(T[3]), false, false);
      const float a02 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
      const float a13 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a02), __float_as_uint(a13), false, false);
      const float sc = (__uint_as_float(y[0]) + __uint_as_float(y[1])) * smul;
      Sc[tau] = (cb + t < lim_c) ? sc : -INFINITY;
    }
    // ---- online softmax for head c (lane-group c)
    // The reference m_run moves only when a score exceeds it by more than
    // 2^kLazy (or on the first scores), so p <= 2^kLazy stays well inside
    // fp16 and the accumulators are rarely rescaled; the result is the same
    // ratio of sums.
    const float cm = row16_max(fmaxf(Sc[0], Sc[1]));
    const float m_new = (cm > m_run + kLazy) ? cm : m_run;
    float alpha = 1.f, p0 = 0.f, p1 = 0.f;
    if (m_new != -INFINITY) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      p0 = __builtin_amdgcn_exp2f(Sc[0] - m_new);
      p1 = __builtin_amdgcn_exp2f(Sc[1] - m_new);
    }
    l_run = l_run * alpha + row16_sum(p0 + p1);
    m_run = m_new;
    // token t sits at contraction slot 8 (t mod 4) + t / 4
    const int sl = 8 * (n & 3) + (n >> 2);
    pb[c * CH + sl] = p0;
    pb[c * CH + sl + 4] = p1;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 16 * i);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[jt][i] *= ai;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- PV.  A (lanes on the diagonal r == c): p * normalised scale of
    // tokens c + 4i; B: centroids of those tokens at this lane's two dims
    const bool diag = (r == c);
    const lds_f32* pp = diag ? pb + hh * CH + 8 * c : pb + C::PB;
    const tq_float4 pa = *(const lds_f32x4*)pp;
    const tq_float4 pc = *(const lds_f32x4*)(pp + 4);
    const uint32_t ph[4] = {half2_bits(pa.x, pa.y), half2_bits(pa.z, pa.w), half2_bits(pc.x, pc.y),
                            half2_bits(pc.z, pc.w)};
    // (s[slot 2k][g], s[slot 2k+1][g]) for the slots 8c .. 8c+7 of this lane-group
    const lds_u32* vsn = diag ? (const lds_u32*)(sp + C::OFF_VS) + 4 * c * G : (const lds_u32*)(pb + C::PB);
    uint32_t sv[4][G];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int g = 0; g < G; ++g) sv[k][g] = vsn[k * G + g];
    // tokens c + 4i for i < 4 and i >= 4; the bases are pinned in registers
    // so that every read of the pair below keeps an immediate offset
    uint32_t va0 = lds_addr(sp) + 4u * (uint32_t)vdw, va1 = va0 + 64u * W;
    asm volatile("" : "+v"(va0), "+v"(va1));
    const lds_u32* const vrow0 = (const lds_u32*)(uintptr_t)va0;
    const lds_u32* const vrow1 = (const lds_u32*)(uintptr_t)va1;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t aw[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) aw[k2] = pk_mul_f16(ph[k2], sv[k2][g]);
      const lds_u32* f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (i < 4 ? vrow0 : vrow1) + 4 * W * (i & 3) + VB * g;
      uint32_t b0[4], b1[4];
      centroid_operands<VB, C::LUT>(f, (uint32_t)fsh, lut, b0, b1);
      const tq_half8 ap = __builtin_bit_cast(tq_half8, aw);
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(tq_half8, b0), acc[2 * g], 0, 0, 0);
      acc[2 * g + 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(tq_half8, b1), acc[2 * g + 1], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- back to true scale, merge lane-groups and waves, write the split partial
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float f = ldexpf(1.f, E[g]);
    acc[2 * g] *= f;
    acc[2 * g + 1] *= f;
  }
  if (n == 0) {
    stats[wave][c][0] = m_run;
    stats[wave][c][1] = l_run;
  }
  __syncthreads();
  lds_f32* const accb = (lds_f32*)smem;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) accb[((wave * NT + jt) * 4 + i) * 64 + lane] = acc[jt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < kHeadTile * D; o += blockDim.x) {
    const int h = o / D, e = o % D;
    if (!hvalid(h)) continue;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, stats[w][h][0]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
      // dim e = 32g + 2n + jj lives in tile 2g + jj, column n
      const int jt = 2 * (e >> 5) + (e & 1), nn = (e & 31) >> 1;
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(stats[w][h][0] - mm);
        ll += stats[w][h][1] * f;
        float s4 = 0.f;
        for (int cc = 0; cc < 4; ++cc) s4 += accb[((w * NT + jt) * 4 + h) * 64 + 16 * cc + nn];
        aa += s4 * f;
      }
    }
    const int jr = tile * kHeadTile + h;
    const int64_t orow = ((int64_t)b * a.n_queries + jr / rep) * a.n_q_heads + gkv * rep + jr % rep;
    const int64_t rec = orow * a.splits + split;
    if (!check_ok(rec < (int64_t)a.batch * a.n_queries * a.n_q_heads * a.splits, kChkAttnPart)) continue;
    float* part = a.part + rec * part_stride<D>();
    part[e] = aa;
    if (e == 0) {
      part[D] = mm;
      part[D + 1] = ll;
    }
  }
}

// All-reduce over the four lane-groups (lanes n, n + 16, n + 32, n + 48):
// two permlane swaps; every lane gets the same bits (one summation order).
__device__ __forceinline__ float lg4_max(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
}
__device__ __forceinline__ float lg4_sum(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// ----------------------------------------------------------------------------
// Matrix-core split kernel for many query rows per kv head (several query
// tokens per sequence, or more than four query heads per kv head).  One block
// serves 16 (query token, head) rows of one (sequence, kv head, context
// split), so each cached token is dequantized and scored once for all of
// them.  The DMA stages, the value-scale normalisation and the PV B operand
// are those of the kernel above; the contractions are laid out the other
// way round:
//  * QK^T on v_mfma_i32_16x16x32_i8, one 32-byte key group per MFMA: A = the
//    stored key bytes of 16 tokens, B = the 16 rows' fixed-point query (hi
//    and lo bytes, two MFMAs), so D[4c+i][n] is token 4c+i's group partial
//    for row n, and the group's key scale and zero apply per element:
//    s = sum_g scale_g (d_g + zero_g * sum_{j in g} q_j).
//  * Lane (c, n) then holds row n's scores for tokens 4c+i and 16+4c+i
//    (i < 4), which are row n's PV A operand at contraction slots 8c .. 8c+7
//    as they are: p never leaves the registers.  Row statistics are
//    all-reduced over the four lane-groups with two permlane swaps.
//  * PV output rows are the 16 rows themselves (no partial sums over token
//    quarters), so one set of PV MFMAs serves all of them.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_attn_mfma16_kernel(AttnArgs a) {
  using C = MfmaCfg<D, KB, VB>;
  constexpr int G = C::G, NT = C::NT, CH = C::CH, W = C::W, S = C::S;
  constexpr int R = 16;  // query rows per block
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[C::OFF_BUF + C::BUF];
  // the other kernel's p buffers hold the row statistics here
  static_assert(C::OFF_STATS - C::OFF_PB >= 4 * R * 2 * 4, "row statistics fit");
  float(*const stats)[R][2] = reinterpret_cast<float(*)[R][2]>(lds_all + C::OFF_PB);
  uint8_t* const smem = lds_all + C::OFF_BUF;

  const int rep = a.n_q_heads / a.n_kv_heads, nrow = a.n_queries * rep;
  const int tiles = (nrow + R - 1) / R;
  int group, tile;
  if (tiles > 1 && gridDim.x % (8u * tiles) == 0) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    tile = j % tiles;
    group = (j / tiles) * 8 + xcd;
  } else {
    tile = (blockIdx.x / a.splits) % tiles;
    group = (blockIdx.x / a.splits / tiles) * a.splits + blockIdx.x % a.splits;
  }
  const int split = group % a.splits;
  const int rest = group / a.splits;
  const int gkv = rest % a.n_kv_heads;
  const int b = rest / a.n_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4, n = lane & 15;
  lds_u8* const wbuf = (lds_u8*)smem + wave * S * C::STAGE;
  lds_u8* const lut = (lds_u8*)lds_all;

  fill_centroid_lut<VB>(lds_all);

  int ctx = a.ctx_lens[check_row(b, a.batch, kChkAttnLen)];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t_begin = split * a.tokens_per_split;
  int t_end = t_begin + a.tokens_per_split;
  if (t_end > ctx) t_end = ctx;
  const int64_t row0 = (int64_t)b * a.seq_stride + (int64_t)gkv * a.head_stride;

  const int first = t_begin + wave * CH;
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    const int cb = first + 4 * CH * k;
    if (cb + CH <= t_end)
      attn_dma<D, KB, VB, false>(a, wbuf + k * C::STAGE, row0 + cb, CH, lane);
    else if (cb < t_end)
      attn_dma<D, KB, VB, true>(a, wbuf + k * C::STAGE, row0 + cb, t_end - cb, lane);
  }

  // ---- query row n of the tile: query jr / rep, head jr % rep of this kv head
  const int jr = tile * R + n;
  const bool rv = jr < nrow;
  const int mq = rv ? jr / rep : 0;
  const uint16_t* const qrow =
      a.q + check_row(((int64_t)b * a.n_queries + mq) * a.n_q_heads + gkv * rep + (rv ? jr % rep : 0),
                      (int64_t)a.batch * a.n_queries * a.n_q_heads, kChkAttnQ) * D;
  // this lane's query elements: 32g + 8c + [0, 8) of every group g
  uint4 qw[G];
  float qmax = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qw[g] = rv ? *reinterpret_cast<const uint4*>(qrow + 32 * g + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t ws[4] = {qw[g].x, qw[g].y, qw[g].z, qw[g].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(ws[i])), fabsf(bf16_hi(ws[i]))));
  }
  const float qscale = a.softmax_scale * kLog2e;
  qmax = lg4_max(qmax) * fabsf(qscale);
  int qe = 0;
  (void)frexpf(qmax, &qe);
  qe = qe < -100 ? -100 : (qe > 100 ? 100 : qe);
  // fixed point q * softmax_scale * log2 e * 2^(14 - qe), |.| <= 2^14, as the
  // exact pair hi * 256 + lo (hi in [-64, 64], lo in [-128, 127])
  const float qn = ldexpf(qscale, 14 - qe);
  const float smul = ldexpf(1.f, qe - 14);
  long qh[G], ql[G];
  float qsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t ws[4] = {qw[g].x, qw[g].y, qw[g].z, qw[g].w};
    uint32_t hw[2] = {0, 0}, lw[2] = {0, 0};
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = key_elem8<KB>(i);  // the key operand's element at byte i
      const float x = (e & 1) ? bf16_hi(ws[e >> 1]) : bf16_lo(ws[e >> 1]);
      const int v = (int)__builtin_rintf(x * qn);
      const int lo = ((v + 128) & 255) - 128;
      const int hi = (v - lo) >> 8;
      hw[i >> 2] |= (uint32_t)(hi & 255) << (8 * (i & 3));
      lw[i >> 2] |= (uint32_t)(lo & 255) << (8 * (i & 3));
      sum += v;
    }
    qh[g] = (long)(((uint64_t)hw[1] << 32) | hw[0]);
    ql[g] = (long)(((uint64_t)lw[1] << 32) | lw[0]);
    qsum[g] = lg4_sum((float)sum);  // exact: an integer below 2^20
  }
  // tokens t < lim are visible to row n
  int lim = rv ? ctx - a.n_queries + 1 + mq : t_end;
  if (lim > t_end) lim = t_end;
  // value fields: as in the kernel above; contraction slot 8c + i is token
  // 4c + i (i < 4) or 16 + 4c + (i - 4)
  int fk = (2 * VB * n) >> 5, fsh = (2 * VB * n) & 31;
  if constexpr (VB != 8) {
    // the pair's bits go to bit 2 of the table's byte offset
    if (fsh < 2) {
      fk -= 1;
      fsh += 30;
    } else {
      fsh -= 2;
    }
  }
  const int vdw = C::OFF_V / 4 + 4 * c * W + fk;
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  tq_float4 acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = tq_float4{0.f, 0.f, 0.f, 0.f};
  int E[G];
#pragma unroll
  for (int g = 0; g < G; ++g) E[g] = -13;
  const tq_i32x4 zero4 = {0, 0, 0, 0};

  int slot = 0;
  for (int cb = first; cb < t_end; cb += 4 * CH) {
    const int cbn = cb + 4 * CH * (S - 1);
    const int nslot = slot == 0 ? S - 1 : slot - 1;
    if (cbn + CH <= t_end)
      attn_dma<D, KB, VB, false>(a, wbuf + nslot * C::STAGE, row0 + cbn, CH, lane);
    else if (cbn < t_end)
      attn_dma<D, KB, VB, true>(a, wbuf + nslot * C::STAGE, row0 + cbn, t_end - cbn, lane);
    const int later = (t_end - cb - 1) / (4 * CH);
    if (later >= 2 && S == 3)
      wait_vmcnt<(S - 1) * C::NI>();
    else if (later >= 1)
      wait_vmcnt<C::NI>();
    else
      wait_vmcnt<0>();

    lds_u8* const sp = wbuf + slot * C::STAGE;
    slot = slot == S - 1 ? 0 : slot + 1;
    const int tl = t_end - cb;
    const bool full = tl >= CH;

    stage_value_scales<D, KB, VB>(sp, full, tl, lane, E, acc,
                              [](int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); });

    // ---- scores: lane (c, n) gets row n at tokens 16 tau + 4c + i
    const lds_u16* const ks = (const lds_u16*)(sp + C::OFF_KS);
    const lds_u16* const kz = (const lds_u16*)(sp + C::OFF_KZ);
    float P[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tk = 16 * tau + n;  // the A operand's token
      const int t0 = 16 * tau + 4 * c;
      float T[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // this lane's 8 key indices: elements 32 g + 8 c .. + 7 of token tk
        constexpr int BO = 8 * KB / 8;
        const int bo = (4 * g + c) * BO, ch = bo >> 4;
        const long kw = keys8<KB>(sp + 16 * (tk * C::CPR + (ch ^ (tk & (C::SW - 1)))) + (bo & 15));
        const tq_i32x4 dh = __builtin_amdgcn_mfma_i32_16x16x32_i8(kw, qh[g], zero4, 0, 0, 0);
        const tq_i32x4 dl = __builtin_amdgcn_mfma_i32_16x16x32_i8(kw, ql[g], zero4, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sk = f16_value(ks[(t0 + i) * G + g]);
          const float zk = f16_value(kz[(t0 + i) * G + g]);
          const float d = (float)(dh[i] * 256 + dl[i]);
          T[i] = __builtin_fmaf(sk, __builtin_fmaf(zk, qsum[g], d), T[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) P[tau][i] = (cb + t0 + i < lim) ? T[i] * smul : -INFINITY;
    }
    // ---- online softmax of row n (lazy running maximum, as above)
    float cm = P[0][0];
#pragma unroll
    for (int k = 1; k < 8; ++k) cm = fmaxf(cm, P[k >> 2][k & 3]);
    cm = lg4_max(cm);
    const float m_new = (cm > m_run + kLazy) ? cm : m_run;
    float alpha = 1.f;
    if (m_new != -INFINITY) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k >> 2][k & 3] = __builtin_amdgcn_exp2f(P[k >> 2][k & 3] - m_new);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k >> 2][k & 3] = 0.f;
    }
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) ps += P[k >> 2][k & 3];
    l_run = l_run * alpha + lg4_sum(ps);
    m_run = m_new;
    if (__any(alpha != 1.f)) {
      // accumulator row 4c + i belongs to the lanes n = 4c + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * c + i);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[jt][i] *= ai;
      }
    }

    // ---- PV.  A: p of row n at slots 8c .. 8c+7 times the normalised value
    // scales of those tokens; B: the centroids of those tokens at this lane's
    // two dims (as in the kernel above)
    const uint32_t ph[4] = {half2_bits(P[0][0], P[0][1]), half2_bits(P[0][2], P[0][3]),
                            half2_bits(P[1][0], P[1][1]), half2_bits(P[1][2], P[1][3])};
    const lds_u32* const vsn = (const lds_u32*)(sp + C::OFF_VS) + 4 * c * G;
    uint32_t sv[4][G];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int g = 0; g < G; ++g) sv[k][g] = vsn[k * G + g];
    uint32_t va0 = lds_addr(sp) + 4u * (uint32_t)vdw, va1 = va0 + 64u * W;
    asm volatile("" : "+v"(va0), "+v"(va1));
    const lds_u32* const vrow0 = (const lds_u32*)(uintptr_t)va0;
    const lds_u32* const vrow1 = (const lds_u32*)(uintptr_t)va1;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t aw[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) aw[k2] = pk_mul_f16(ph[k2], sv[k2][g]);
      const lds_u32* f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (i < 4 ? vrow0 : vrow1) + W * (i & 3) + VB * g;
      uint32_t b0[4], b1[4];
      centroid_operands<VB, C::LUT>(f, (uint32_t)fsh, lut, b0, b1);
      const tq_half8 ap = __builtin_bit_cast(tq_half8, aw);
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(tq_half8, b0), acc[2 * g], 0, 0, 0);
      acc[2 * g + 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(tq_half8, b1), acc[2 * g + 1], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- back to true scale, merge the waves, write the split partials
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float f = ldexpf(1.f, E[g]);
    acc[2 * g] *= f;
    acc[2 * g + 1] *= f;
  }
  if (c == 0) {
    stats[wave][n][0] = m_run;
    stats[wave][n][1] = l_run;
  }
  __syncthreads();
  lds_f32* const accb = (lds_f32*)smem;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) accb[((wave * NT + jt) * 4 + i) * 64 + lane] = acc[jt][i];
  __syncthreads();
  for (int o = threadIdx.x; o < R * D; o += blockDim.x) {
    const int h = o / D, e = o % D;
    const int jh = tile * R + h;
    if (jh >= nrow) continue;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, stats[w][h][0]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
      // dim e = 32g + 2nn + jj sits in tile 2g + jj, column nn; row h is
      // register h % 4 of lane-group h / 4
      const int jt = 2 * (e >> 5) + (e & 1), nn = (e & 31) >> 1;
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(stats[w][h][0] - mm);
        ll += stats[w][h][1] * f;
        aa += accb[((w * NT + jt) * 4 + (h & 3)) * 64 + 16 * (h >> 2) + nn] * f;
      }
    }
    const int64_t orow = ((int64_t)b * a.n_queries + jh / rep) * a.n_q_heads + gkv * rep + jh % rep;
    const int64_t rec = orow * a.splits + split;
    if (!check_ok(rec < (int64_t)a.batch * a.n_queries * a.n_q_heads * a.splits, kChkAttnPart)) continue;
    float* part = a.part + rec * part_stride<D>();
    part[e] = aa;
    if (e == 0) {
      part[D] = mm;
      part[D + 1] = ll;
    }
  }
}

// Merge the partials of splits s0, s0 + ds, ... (NB of them, those below
// `splits`) into the running (mm, ll, acc) of one row slice: all their
// loads issue before the first is used, the batch maximum rescales the
// running sums once, then the batch adds in split order.
template <int D, int NB>
__device__ __forceinline__ void merge_batch(const float* part, int s0, int ds, int splits, int sub, float& mm,
                                            float& ll, float (&acc)[8]) {
  float ms[NB], ls[NB];
  float4 x0[NB], x1[NB];
  // splits past the last re-read the last one (no branch between the loads,
  // so they are all in flight together) and count as empty
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int s = min(s0 + j * ds, splits - 1);
    const float* ps = part + s * part_stride<D>();
    const float2 ml = *reinterpret_cast<const float2*>(ps + D);
    ms[j] = ml.x;
    ls[j] = ml.y;
    x0[j] = *reinterpret_cast<const float4*>(ps + 8 * sub);
    x1[j] = *reinterpret_cast<const float4*>(ps + 8 * sub + 4);
  }
  // keep every load above this point (the scheduler would otherwise trade
  // the overlap for registers, one round trip per split)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (s0 + j * ds >= splits) ms[j] = -INFINITY;
  float mb = mm;
#pragma unroll
  for (int j = 0; j < NB; ++j) mb = fmaxf(mb, ms[j]);
  // A split with no tokens carries m = -inf and adds nothing.  No branch on
  // it either, which would let the compiler hold back the partials' loads:
  // with everything so far empty the reference maximum is 0 and every
  // weight exp2(-inf) = 0.
  const float mref = (mb == -INFINITY) ? 0.f : mb;
  const float c = exp2f(mm - mref);  // 0 while nothing is merged yet
  ll *= c;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= c;
  mm = mb;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float f = exp2f(ms[j] - mref);
    ll += ls[j] * f;
    acc[0] += x0[j].x * f; acc[1] += x0[j].y * f; acc[2] += x0[j].z * f; acc[3] += x0[j].w * f;
    acc[4] += x1[j].x * f; acc[5] += x1[j].y * f; acc[6] += x1[j].z * f; acc[7] += x1[j].w * f;
  }
}

// Splits first, first + ds, ... below `splits` merged in batches sized to
// their count (the count is uniform over the grid; loads for splits that do
// not exist are wasted issue slots).
template <int D>
__device__ __forceinline__ void merge_splits(const float* part, int sub, int first, int ds, int splits, float& mm,
                                             float& ll, float (&acc)[8]) {
  const int n = (splits + ds - 1) / ds;
  if (n <= 1) {
    merge_batch<D, 1>(part, first, ds, splits, sub, mm, ll, acc);
  } else if (n <= 2) {
    merge_batch<D, 2>(part, first, ds, splits, sub, mm, ll, acc);
  } else if (n <= 4) {
    merge_batch<D, 4>(part, first, ds, splits, sub, mm, ll, acc);
  } else {
    for (int s0 = first; s0 < splits; s0 += 8 * ds) merge_batch<D, 8>(part, s0, ds, splits, sub, mm, ll, acc);
  }
}

// Merge the splits of each (sequence, query head), un-rotate once, store bf16.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const int rows = a.batch * a.n_queries * a.n_q_heads;
  const int r0 = ((blockIdx.x * blockDim.x + threadIdx.x) >> 6) * RPW + rw;
  const bool active = r0 < rows;
  const int r = active ? r0 : 0;
  const float* part = a.part + (int64_t)r * a.splits * part_stride<D>();
  // one pass over the splits, SB at a time so that their loads are in
  // flight together; the running maximum rescales what is merged so far
  float mm = -INFINITY, ll = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  merge_splits<D>(part, sub, 0, 1, a.splits, mm, ll, acc);
  const float inv = (ll > 0.f) ? 1.f / ll : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= inv;
  fwht_row<D>(acc, sub);
  const float rd = inv_sqrt_d<D>();
  const uint2 sw = *reinterpret_cast<const uint2*>(a.signs + 8 * sub);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int8_t sb = (int8_t)((i < 4 ? sw.x : sw.y) >> (8 * (i & 3)));
    // a sequence with no cached tokens gets an all-(+0) row
    acc[i] = (ll > 0.f) ? acc[i] * rd * (sb < 0 ? -1.f : 1.f) : 0.f;
  }
  if (active) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    if (check_ok(r < rows, kChkAttnOut)) *reinterpret_cast<uint4*>(a.out + (int64_t)r * D + 8 * sub) = o;
  }
}

// The same merge for many splits: one block per output row.  Slice k of the
// block (LPR lanes) merges splits k, k + NSL, ... into (m_k, l_k, acc_k); the
// slices then meet in LDS and the first LPR lanes finish the row.  At
// d = 512 a row spans a whole wave, so the block has 16 waves (16 slices)
// rather than 4: the VALU kernel's long single-sequence contexts reach 512
// splits, which four slices would merge in 16 dependent batches each.
template <int D>
constexpr int combine_wide_threads() { return D >= 512 ? 1024 : 256; }

template <int D>
__global__ __launch_bounds__(1024) void decode_attn_combine_wide_kernel(AttnArgs a) {
  constexpr int LPR = D / 8, NSL = combine_wide_threads<D>() / LPR;
  __shared__ float s_acc[NSL][D];
  __shared__ float s_ml[NSL][2];
  const int sub = threadIdx.x % LPR, k = threadIdx.x / LPR;
  const int r = blockIdx.x;
  const float* part = a.part + (int64_t)r * a.splits * part_stride<D>();
  float mm = -INFINITY, ll = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  merge_splits<D>(part, sub, k, NSL, a.splits, mm, ll, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) s_acc[k][8 * sub + i] = acc[i];
  if (sub == 0) {
    s_ml[k][0] = mm;
    s_ml[k][1] = ll;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // wave 0: every lane rebuilds row r (lanes >= LPR repeat lanes % LPR and store nothing)
  float m_all = -INFINITY;
  for (int j = 0; j < NSL; ++j) m_all = fmaxf(m_all, s_ml[j][0]);
  float l_all = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (m_all != -INFINITY) {
    for (int j = 0; j < NSL; ++j) {
      const float f = exp2f(s_ml[j][0] - m_all);
      l_all += s_ml[j][1] * f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += s_acc[j][8 * sub + i] * f;
    }
  }
  const float inv = (l_all > 0.f) ? 1.f / l_all : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= inv;
  fwht_row<D>(acc, sub);
  const float rd = inv_sqrt_d<D>();
  const uint2 sw = *reinterpret_cast<const uint2*>(a.signs + 8 * sub);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int8_t sb = (int8_t)((i < 4 ? sw.x : sw.y) >> (8 * (i & 3)));
    acc[i] = (l_all > 0.f) ? acc[i] * rd * (sb < 0 ? -1.f : 1.f) : 0.f;
  }
  if ((int)threadIdx.x < LPR) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    if (check_ok(r < a.batch * a.n_queries * a.n_q_heads, kChkAttnOut)) *reinterpret_cast<uint4*>(a.out + (int64_t)r * D + 8 * sub) = o;
  }
}

uint32_t check_read_clear_attn() { return check_read_clear_file(); }

// Merge kernel choice: the per-row kernel gives a row's splits to one set of
// lanes, the wide one spreads them over a block (worth it once there are
// many splits).
template <int D>
static void launch_combine(const AttnArgs& a, hipStream_t st) {
  const int rows = a.batch * a.n_queries * a.n_q_heads;
  if (a.splits >= 16) {
    decode_attn_combine_wide_kernel<D><<<dim3((unsigned)rows), combine_wide_threads<D>(), 0, st>>>(a);
  } else {
    const int rows_per_block = 4 * (64 / (D / 8));
    decode_attn_combine_kernel<D><<<dim3((rows + rows_per_block - 1) / rows_per_block), 256, 0, st>>>(a);
  }
}

// int8 keys, and packed 5-, 4- and 2-bit keys spread into bytes (5-bit rows
// of d = 64, 40 bytes, do not keep the 16-byte alignment of the copies);
// values of 2 to 5 and 8 bits
bool decode_attn_uses_mfma(int d, int kb, int vb) {
  return d <= 256 && (vb <= 5 || vb == 8) && (kb == 8 || kb == 4 || kb == 2 || (kb == 5 && d >= 128));
}

void decode_attn_geometry(int d, int kb, int vb, int batch, int n_queries, int n_q_heads, int n_kv_heads,
                          int max_ctx, int* splits, int* tokens_per_split) {
  // rows one block consumes per pass: four waves of 32-token steps on the
  // matrix-core path, four waves of kChunk rows per lane-group otherwise
  const bool mfma = decode_attn_uses_mfma(d, kb, vb);
  const int step = mfma ? 4 * 32 : 4 * (64 / (d / 8)) * kChunk;
  const long long rep = n_q_heads / n_kv_heads, nrow = (long long)n_queries * rep;
  // query rows per block: 16 on the matrix-core path once a kv head has more
  // than one tile of four
  const long long rows = mfma && (kb == 8 || kb == 4) && nrow > kHeadTile ? 16 : kHeadTile;
  long long units = (long long)batch * n_kv_heads * ((nrow + rows - 1) / rows);
  if (units < 1) units = 1;  // an empty batch: nothing runs, any split count serves
  // The matrix-core kernel streams through per-wave DMA stages, which pay a
  // pipeline fill per block: aim at one round of resident blocks (two per CU
  // on the 256 CUs of gfx950).  The VALU kernel prefers four rounds of
  // shorter blocks (1024: 512 and 4096 were slower).
  // Each split of the matrix-core kernel also keeps at least four steps per
  // wave, so that the fill is paid over several steps and the combine does
  // not merge dozens of tiny splits, but only while the grid still has 256
  // blocks: a short launch-bound decode does better with more parallel blocks
  // of a step or two (one sequence, 8 kv heads, d = 128: 17.8 -> 13.5 us at
  // 2048 tokens, 18.6 -> 17.0 us at 8192; GQA 6 at d = 256 over 16384 tokens,
  // one 16-row tile per kv head: 32.5 -> 28.4 us).
  const long long target = mfma ? 512 : 1024;
  const long long min_steps = mfma ? 4 : 1;
  long long s = (target + units - 1) / units;
  long long max_s = (max_ctx + min_steps * step - 1) / (min_steps * step);
  if (units * max_s < 256) {
    const long long fill = (256 + units - 1) / units, one_step = (max_ctx + step - 1) / step;
    max_s = fill < one_step ? fill : one_step;
  }
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  long long tps = (max_ctx + s - 1) / s;
  tps = (tps + step - 1) / step * step;
  s = (max_ctx + tps - 1) / tps;
  *splits = (int)s;
  *tokens_per_split = (int)tps;
}

size_t decode_attn_part_bytes(int d, int batch, int n_queries, int n_q_heads, int splits) {
  return (size_t)batch * n_queries * n_q_heads * splits * (size_t)(d + 4) * sizeof(float);
}

template <int D, int KB>
static void launch_split_kb(const AttnArgs& a, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 2: decode_attn_split_kernel<D, KB, 2><<<grid, 256, 0, st>>>(a); break;
    case 3: decode_attn_split_kernel<D, KB, 3><<<grid, 256, 0, st>>>(a); break;
    case 4: decode_attn_split_kernel<D, KB, 4><<<grid, 256, 0, st>>>(a); break;
    case 5: decode_attn_split_kernel<D, KB, 5><<<grid, 256, 0, st>>>(a); break;
    default: decode_attn_split_kernel<D, KB, 8><<<grid, 256, 0, st>>>(a); break;
  }
}

// Matrix-core launches: 16 (query, head) rows per block once a kv head has
// more than four (8- and 4-bit keys; 2- and 5-bit keys take the four-row
// kernel's tiles).
template <int D, int KB>
static void launch_mfma_kb(const AttnArgs& w, int vb, int nrow, dim3 grid, hipStream_t st) {
  if constexpr (KB == 8 || KB == 4) {
    if (nrow > kHeadTile) {
      const dim3 g16((unsigned)(w.batch * w.n_kv_heads * ((nrow + 15) / 16) * w.splits));
      switch (vb) {
        case 2: decode_attn_mfma16_kernel<D, KB, 2><<<g16, 256, 0, st>>>(w); break;
        case 3: decode_attn_mfma16_kernel<D, KB, 3><<<g16, 256, 0, st>>>(w); break;
        case 4: decode_attn_mfma16_kernel<D, KB, 4><<<g16, 256, 0, st>>>(w); break;
        case 5: decode_attn_mfma16_kernel<D, KB, 5><<<g16, 256, 0, st>>>(w); break;
        default: decode_attn_mfma16_kernel<D, KB, 8><<<g16, 256, 0, st>>>(w); break;
      }
      return;
    }
  }
  switch (vb) {
    case 2: decode_attn_mfma_kernel<D, KB, 2><<<grid, 256, 0, st>>>(w); break;
    case 3: decode_attn_mfma_kernel<D, KB, 3><<<grid, 256, 0, st>>>(w); break;
    case 4: decode_attn_mfma_kernel<D, KB, 4><<<grid, 256, 0, st>>>(w); break;
    case 5: decode_attn_mfma_kernel<D, KB, 5><<<grid, 256, 0, st>>>(w); break;
    default: decode_attn_mfma_kernel<D, KB, 8><<<grid, 256, 0, st>>>(w); break;
  }
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, int kb, int vb, hipStream_t st) {
  const int rep = a.n_q_heads / a.n_kv_heads;
  const int tiles = (a.n_queries * rep + kHeadTile - 1) / kHeadTile;
  const dim3 grid((unsigned)(a.batch * a.n_kv_heads * tiles * a.splits));
  if constexpr (D <= 256) {
    // the DMA copies need 16-byte key rows and 4-byte aligned fp16 planes
    const bool aligned = ((uintptr_t)a.k_q & 15u) == 0 && ((uintptr_t)a.k_scale & 3u) == 0 &&
                         ((uintptr_t)a.k_zero & 3u) == 0 && ((uintptr_t)a.v_scale & 3u) == 0 &&
                         ((uintptr_t)a.v_q & 3u) == 0;
    if (decode_attn_uses_mfma(D, kb, vb) && aligned) {
      AttnArgs w = a;
      w.wide = ((uintptr_t)a.v_q & 15u) == 0 && ((uintptr_t)a.k_scale & 15u) == 0 &&
               ((uintptr_t)a.k_zero & 15u) == 0 && (a.seq_stride & 1) == 0 && (a.head_stride & 1) == 0;
      const int nrow = a.n_queries * rep;
      switch (kb) {
        case 2: launch_mfma_kb<D, 2>(w, vb, nrow, grid, st); break;
        case 4: launch_mfma_kb<D, 4>(w, vb, nrow, grid, st); break;
        case 5:
          if constexpr (D >= 128) launch_mfma_kb<D, 5>(w, vb, nrow, grid, st);
          break;
        default: launch_mfma_kb<D, 8>(w, vb, nrow, grid, st); break;
      }
      launch_combine<D>(a, st);
      return hipGetLastError();
    }
  }
  switch (kb) {
    case 2: launch_split_kb<D, 2>(a, vb, grid, st); break;
    case 4: launch_split_kb<D, 4>(a, vb, grid, st); break;
    case 5: launch_split_kb<D, 5>(a, vb, grid, st); break;
    default: launch_split_kb<D, 8>(a, vb, grid, st); break;
  }
  launch_combine<D>(a, st);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const AttnArgs& a, int d, int kb, int vb, hipStream_t st) {
  switch (d) {
    case 64: return launch_attn_d<64>(a, kb, vb, st);
    case 128: return launch_attn_d<128>(a, kb, vb, st);
    case 256: return launch_attn_d<256>(a, kb, vb, st);
    default: return launch_attn_d<512>(a, kb, vb, st);
  }
}

}  // namespace tq
