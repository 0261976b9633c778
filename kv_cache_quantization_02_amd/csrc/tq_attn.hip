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
