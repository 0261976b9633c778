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
constexpr int kChunk = 4;      // rows per lane-group between softmax rescales
constexpr float kLog2e = 1.4426950408889634f;

// One split partial per (sequence, query head): acc[d], m, l, two pad words
// (keeps every record 16-byte aligned).
template <int D>
constexpr int part_stride() { return D + 4; }

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
  const int rep = a.n_q_heads / a.n_kv_heads;
  const int tiles = (rep + kHeadTile - 1) / kHeadTile;
  const int tile = rest % tiles;
  rest /= tiles;
  const int g = rest % a.n_kv_heads;
  const int b = rest / a.n_kv_heads;

  for (int i = threadIdx.x; i < (1 << VB); i += blockDim.x)
    cen_lds[i] = __uint_as_float(attn_centroids<VB>()[i]);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, c = lane / LPR;

  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t_begin = split * a.tokens_per_split;
  int t_end = t_begin + a.tokens_per_split;
  if (t_end > ctx) t_end = ctx;

  // query slice (pre-scaled into the log2 domain)
  const float qscale = a.softmax_scale * kLog2e;
  float q[kHeadTile][8];
  bool hv[kHeadTile];
#pragma unroll
  for (int j = 0; j < kHeadTile; ++j) {
    const int hl = tile * kHeadTile + j;
    hv[j] = hl < rep;
    const int hq = g * rep + (hv[j] ? hl : 0);
    const uint4 w = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.n_q_heads + hq) * D + 8 * sub);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[j][2 * i] = hv[j] ? bf16_lo(ws[i]) * qscale : 0.f;
      q[j][2 * i + 1] = hv[j] ? bf16_hi(ws[i]) * qscale : 0.f;
    }
  }
  __syncthreads();

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
      float kh[8];
      if (valid) {
        const int64_t row = row0 + t;
        const uint64_t bits = load_lane_bits<KB>(a.k_q + row * KROW, sub);
        const float s16 = f16_value(a.k_scale[row * G + (sub >> 2)]);
        const float z16 = f16_value(a.k_zero[row * G + (sub >> 2)]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float qi;
          if constexpr (KB == 8)
            qi = (float)(int8_t)(bits >> (8 * i));
          else
            qi = (float)(uint32_t)((bits >> (KB * i)) & ((1u << KB) - 1));
          kh[i] = (qi + z16) * s16;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kh[i] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < kHeadTile; ++j) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = __builtin_fmaf(q[j][i], kh[i], d);
        d = row_sum<D>(d);
        sc[k][j] = valid ? d : -INFINITY;
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
        const int64_t row = row0 + t;
        const uint64_t bits = load_lane_bits<VB>(a.v_q + row * VROW, sub);
        const float vs = f16_value(a.v_scale[row * G + (sub >> 2)]);
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = cen_lds[(bits >> (VB * i)) & ((1u << VB) - 1)] * vs;
#pragma unroll
        for (int j = 0; j < kHeadTile; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] = __builtin_fmaf(p[k][j], z[i], acc[j][i]);
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
    const int hl = tile * kHeadTile + j;
    if (hl >= rep) continue;
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
    const int hq = g * rep + hl;
    float* part = a.part + (((int64_t)b * a.n_q_heads + hq) * a.splits + split) * part_stride<D>();
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
// A wave takes 32 cached tokens per step for a tile of 4 query heads.
//  * QK^T: a key byte b = idx ^ 0x80 becomes the exact fp16 1024 + (idx+128),
//    so each 32-element group g contributes
//        s_g * (sum_j q_j (1024 + u_j) + (zero_g - 1152) * sum_j q_j),
//    i.e. idx + zero times the fp16 scale.  A is block-diagonal over 4 groups
//    (rows 4g + h), so all 16 output rows are used; the 4 lane-groups'
//    per-group partials are then summed with three permlane swaps, leaving
//    lane-group h with head h's scores.
//  * Online softmax per head in the log2 domain (q carries
//    softmax_scale * log2 e), exact rescaling whenever the maximum moves.
//  * PV: the 32 value rows are decoded once into LDS as fp16 centroids
//    (a lookup of two indices at a time), and A = p * value-scale (fp16, block-
//    diagonal over four 8-token sub-chunks) multiplies them: the rotated-domain
//    accumulation z = centroid * scale, with the scale folded into the weights.
// The per-split (m, l, acc) partials match the VALU kernel's, so the same
// combine kernel applies the inverse rotation.
typedef _Float16 tq_half8 __attribute__((ext_vector_type(8)));
typedef float tq_float4 __attribute__((ext_vector_type(4)));
typedef _Float16 tq_half2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// all-reduce over the 16 lanes of a row (quad xor 1, xor 2, rotate 4, rotate 8)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  return v;
}

__device__ __forceinline__ uint32_t half2_bits(float lo, float hi) {
  const tq_float2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, tq_half2));
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(tq_half2, a) * __builtin_bit_cast(tq_half2, b));
}

template <int D, int VB>
__global__ __launch_bounds__(256) void decode_attn_mfma_kernel(AttnArgs a) {
  constexpr int G = D / kGroup, NSET = (G + 3) / 4, NT = D / 16;
  constexpr int CH = 32;                    // tokens per step: the PV MFMA depth
  constexpr int ZS = 2 * D + 16;            // LDS bytes per decoded row (padded)
  constexpr int LW = D * VB / 64;           // packed dwords per decode lane
  constexpr int PB = 4 * CH;                // p[h][t] floats, then 8 zeros
  constexpr int VROW = D * VB / 8;
  constexpr int ACC_BYTES = 4 * NT * 4 * 64 * 4;
  constexpr int ZB_BYTES = 4 * CH * ZS > ACC_BYTES ? 4 * CH * ZS : ACC_BYTES;
  __shared__ uint32_t lut[1 << (2 * VB)];
  __shared__ __attribute__((aligned(16))) uint8_t zb_all[ZB_BYTES];
  __shared__ __attribute__((aligned(16))) float pb_all[4][PB + 8];
  __shared__ float stats[4][4][2];

  const int split = blockIdx.x % a.splits;
  int rest = blockIdx.x / a.splits;
  const int rep = a.n_q_heads / a.n_kv_heads;
  const int tiles = (rep + kHeadTile - 1) / kHeadTile;
  const int tile = rest % tiles;
  rest /= tiles;
  const int gkv = rest % a.n_kv_heads;
  const int b = rest / a.n_kv_heads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, n = lane & 15, r = n >> 2, hh = n & 3;
  uint8_t* zb = zb_all + wave * CH * ZS;
  float* pb = pb_all[wave];

  for (int i = threadIdx.x; i < (1 << (2 * VB)); i += blockDim.x) {
    const uint32_t* cen = attn_centroids<VB>();
    const float c0 = __uint_as_float(cen[i & ((1 << VB) - 1)]);
    const float c1 = __uint_as_float(cen[i >> VB]);
    lut[i] = half2_bits(c0, c1);
  }
  if (lane < 8) pb[PB + lane] = 0.f;

  int ctx = a.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t_begin = split * a.tokens_per_split;
  int t_end = t_begin + a.tokens_per_split;
  if (t_end > ctx) t_end = ctx;
  const int64_t row0 = (int64_t)b * a.seq_stride + (int64_t)gkv * a.head_stride;

  // ---- query: block-diagonal A operands (lane (n = 4r + h, c) carries head h
  // for the group with g % 4 == r) and per-group sums for the zero term
  const float qscale = a.softmax_scale * kLog2e;
  auto qhead = [&](int h) -> const uint16_t* {
    const int hl = tile * kHeadTile + h;
    const int hq = gkv * rep + (hl < rep ? hl : 0);
    return a.q + ((int64_t)b * a.n_q_heads + hq) * D;
  };
  auto hvalid = [&](int h) { return tile * kHeadTile + h < rep; };
  tq_half8 aq[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool on = ((g & 3) == r) && hvalid(hh);
    const uint4 w = on ? *reinterpret_cast<const uint4*>(qhead(hh) + kGroup * g + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      aq[g][2 * i] = (_Float16)(bf16_lo(ws[i]) * qscale);
      aq[g][2 * i + 1] = (_Float16)(bf16_hi(ws[i]) * qscale);
    }
  }
  float qsum[NSET][4];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int g = 4 * st + c;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float acc = 0.f;
      if (g < G && hvalid(h)) {
        const uint4* p = reinterpret_cast<const uint4*>(qhead(h) + kGroup * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 w = p[j];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc += (float)(_Float16)(bf16_lo(ws[i]) * qscale);
            acc += (float)(_Float16)(bf16_hi(ws[i]) * qscale);
          }
        }
      }
      qsum[st][h] = acc;
    }
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  tq_float4 acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = tq_float4{0.f, 0.f, 0.f, 0.f};

  for (int cb = t_begin + wave * CH; cb < t_end; cb += 4 * CH) {
    // ---- decode the 32 value rows of this step into LDS (fp16, row-major)
    {
      const int tt = lane >> 1, half = lane & 1;
      const int t = cb + tt;
      uint32_t wv[LW];
      if (t < t_end) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.v_q + (row0 + t) * VROW + half * (VROW / 2));
#pragma unroll
        for (int i = 0; i < LW; ++i) wv[i] = src[i];
      }
      uint8_t* zrow = zb + tt * ZS + half * D;
#pragma unroll
      for (int q4 = 0; q4 < D / 16; ++q4) {
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = 4 * q4 + k, bit = 2 * VB * p, wd = bit >> 5, off = bit & 31;
          uint32_t f;
          if (off + 2 * VB <= 32)
            f = __builtin_amdgcn_ubfe(wv[wd], off, 2 * VB);
          else
            f = (wv[wd] >> off) | ((wv[wd + 1] << (32 - off)) & ((1u << (2 * VB)) - 1));
          o[k] = (t < t_end) ? lut[f] : 0u;
        }
        *reinterpret_cast<uint4*>(zrow + 16 * q4) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    // ---- scores for the two 16-token tiles
    float S[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = cb + 16 * tau + n;
      const bool tv = t < t_end;
      const int64_t row = row0 + t;
      float T[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSET; ++st) {
        tq_float4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < 4 && 4 * st + gi < G; ++gi) {
          const int g = 4 * st + gi;
          uint2 kw = make_uint2(0x80808080u, 0x80808080u);
          if (tv) kw = *reinterpret_cast<const uint2*>(a.k_q + row * D + kGroup * g + 8 * c);
          const uint32_t u0 = kw.x ^ 0x80808080u, u1 = kw.y ^ 0x80808080u;
          uint32_t bw[4];
          bw[0] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u);
          bw[1] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u);
          bw[2] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u);
          bw[3] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u);
          const tq_half8 bk = __builtin_bit_cast(tq_half8, bw);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[g], bk, d, 0, 0, 0);
        }
        const int g = 4 * st + c;
        float sk = 0.f, zk = 0.f;
        if (tv && g < G) {
          sk = f16_value(a.k_scale[row * G + g]);
          zk = f16_value(a.k_zero[row * G + g]);
        }
        const float zq = zk - 1152.0f;
#pragma unroll
        for (int h = 0; h < 4; ++h) T[h] = __builtin_fmaf(sk, __builtin_fmaf(zq, qsum[st][h], d[h]), T[h]);
      }
      // lane-group h collects head h: sum over the four lane-groups
      const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[0]), __float_as_uint(T[2]), false, false);
      const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[1]), __float_as_uint(T[3]), false, false);
      const float a02 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
      const float a13 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a02), __float_as_uint(a13), false, false);
      const float sc = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      S[tau] = tv ? sc : -INFINITY;
    }
    // ---- online softmax for head c (lane-group c)
    const float cm = row16_max(fmaxf(S[0], S[1]));
    const float m_new = fmaxf(m_run, cm);
    float alpha = 1.f, p0 = 0.f, p1 = 0.f;
    if (m_new != -INFINITY) {
      alpha = exp2f(m_run - m_new);
      p0 = exp2f(S[0] - m_new);
      p1 = exp2f(S[1] - m_new);
    }
    l_run = l_run * alpha + row16_sum(p0 + p1);
    m_run = m_new;
    pb[c * CH + n] = p0;
    pb[c * CH + 16 + n] = p1;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 16 * i);
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[jt][i] *= ai;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- PV: A = p * value scale (fp16), block-diagonal over 8-token sub-chunks
    const bool diag = (r == c);
    const float* pp = diag ? pb + hh * CH + 8 * c : pb + PB;
    const float4 pa = *reinterpret_cast<const float4*>(pp);
    const float4 pc = *reinterpret_cast<const float4*>(pp + 4);
    const uint32_t ph[4] = {half2_bits(pa.x, pa.y), half2_bits(pa.z, pa.w), half2_bits(pc.x, pc.y),
                            half2_bits(pc.z, pc.w)};
    // value scales of tokens cb+8c .. cb+8c+7, G fp16 each
    uint32_t sv[8][(G + 1) / 2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = cb + 8 * c + k;
#pragma unroll
      for (int i = 0; i < (G + 1) / 2; ++i) sv[k][i] = 0;
      if (diag && t < t_end) {
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.v_scale + (row0 + t) * G);
#pragma unroll
        for (int i = 0; i < G / 2; ++i) sv[k][i] = sp[i];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t aw[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        // (scale[2k2][g], scale[2k2+1][g]) as one fp16 pair
        const uint32_t w0 = sv[2 * k2][g >> 1], w1 = sv[2 * k2 + 1][g >> 1];
        const uint32_t spair = (g & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                       : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        aw[k2] = pk_mul_f16(ph[k2], spair);
      }
      const tq_half8 ap = __builtin_bit_cast(tq_half8, aw);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jt = 2 * g + jj;
        const uint16_t* zc = reinterpret_cast<const uint16_t*>(zb + (8 * c) * ZS) + 16 * jt + n;
        uint32_t bw[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
          bw[k2] = (uint32_t)zc[(2 * k2) * (ZS / 2)] | ((uint32_t)zc[(2 * k2 + 1) * (ZS / 2)] << 16);
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(tq_half8, bw), acc[jt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge lane-groups (token sub-chunks) and the four waves, write the split partial
  if (n == 0) {
    stats[wave][c][0] = m_run;
    stats[wave][c][1] = l_run;
  }
  __syncthreads();
  float* accb = reinterpret_cast<float*>(zb_all);
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
      const int jt = e >> 4, nn = e & 15;
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(stats[w][h][0] - mm);
        ll += stats[w][h][1] * f;
        float s4 = 0.f;
        for (int cc = 0; cc < 4; ++cc) s4 += accb[((w * NT + jt) * 4 + h) * 64 + 16 * cc + nn];
        aa += s4 * f;
      }
    }
    const int hq = gkv * rep + tile * kHeadTile + h;
    float* part = a.part + (((int64_t)b * a.n_q_heads + hq) * a.splits + split) * part_stride<D>();
    part[e] = aa;
    if (e == 0) {
      part[D] = mm;
      part[D + 1] = ll;
    }
  }
}

// Merge the splits of each (sequence, query head), un-rotate once, store bf16.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const int rows = a.batch * a.n_q_heads;
  const int r0 = ((blockIdx.x * blockDim.x + threadIdx.x) >> 6) * RPW + rw;
  const bool active = r0 < rows;
  const int r = active ? r0 : 0;
  const float* part = a.part + (int64_t)r * a.splits * part_stride<D>();
  float mm = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mm = fmaxf(mm, part[s * part_stride<D>() + D]);
  float ll = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (mm != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float* ps = part + s * part_stride<D>();
      const float f = exp2f(ps[D] - mm);
      ll += ps[D + 1] * f;
      const float4 x0 = *reinterpret_cast<const float4*>(ps + 8 * sub);
      const float4 x1 = *reinterpret_cast<const float4*>(ps + 8 * sub + 4);
      acc[0] += x0.x * f; acc[1] += x0.y * f; acc[2] += x0.z * f; acc[3] += x0.w * f;
      acc[4] += x1.x * f; acc[5] += x1.y * f; acc[6] += x1.z * f; acc[7] += x1.w * f;
    }
  }
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
    *reinterpret_cast<uint4*>(a.out + (int64_t)r * D + 8 * sub) = o;
  }
}

void decode_attn_geometry(int d, int batch, int n_q_heads, int n_kv_heads, int max_ctx, int* splits,
                          int* tokens_per_split) {
  const int step = 4 * (64 / (d / 8)) * kChunk;  // rows one block consumes per pass
  const int rep = n_q_heads / n_kv_heads;
  const long long units = (long long)batch * n_kv_heads * ((rep + kHeadTile - 1) / kHeadTile);
  long long s = (2048 + units - 1) / units;
  const long long max_s = (max_ctx + step - 1) / step;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  long long tps = (max_ctx + s - 1) / s;
  tps = (tps + step - 1) / step * step;
  s = (max_ctx + tps - 1) / tps;
  *splits = (int)s;
  *tokens_per_split = (int)tps;
}

size_t decode_attn_part_bytes(int d, int batch, int n_q_heads, int splits) {
  return (size_t)batch * n_q_heads * splits * (size_t)(d + 4) * sizeof(float);
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

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, int kb, int vb, hipStream_t st) {
  const int rep = a.n_q_heads / a.n_kv_heads;
  const int tiles = (rep + kHeadTile - 1) / kHeadTile;
  const dim3 grid((unsigned)(a.batch * a.n_kv_heads * tiles * a.splits));
  if constexpr (D <= 256) {
    if (kb == 8 && vb <= 5) {
      switch (vb) {
        case 2: decode_attn_mfma_kernel<D, 2><<<grid, 256, 0, st>>>(a); break;
        case 3: decode_attn_mfma_kernel<D, 3><<<grid, 256, 0, st>>>(a); break;
        case 4: decode_attn_mfma_kernel<D, 4><<<grid, 256, 0, st>>>(a); break;
        default: decode_attn_mfma_kernel<D, 5><<<grid, 256, 0, st>>>(a); break;
      }
      const int rows = a.batch * a.n_q_heads;
      const int rows_per_block = 4 * (64 / (D / 8));
      decode_attn_combine_kernel<D><<<dim3((rows + rows_per_block - 1) / rows_per_block), 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  switch (kb) {
    case 2: launch_split_kb<D, 2>(a, vb, grid, st); break;
    case 4: launch_split_kb<D, 4>(a, vb, grid, st); break;
    case 5: launch_split_kb<D, 5>(a, vb, grid, st); break;
    default: launch_split_kb<D, 8>(a, vb, grid, st); break;
  }
  const int rows = a.batch * a.n_q_heads;
  const int rows_per_block = 4 * (64 / (D / 8));
  decode_attn_combine_kernel<D><<<dim3((rows + rows_per_block - 1) / rows_per_block), 256, 0, st>>>(a);
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
