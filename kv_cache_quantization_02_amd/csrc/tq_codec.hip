// tq_codec.hip -- quantize / dequantize kernels for gfx950.
//
// TurboQuant page, "Algorithm (vllm-metal reference semantics, exact)":
//   keys   : asymmetric affine per 32-group, fp32 arithmetic, fp16 scale/zero;
//   values : y = FWHT(x * signs) / sqrt(d); RMS per 32-group; Lloyd-Max index
//            of y / (scale + 1e-8); little-endian packed bitstream.
// Every kernel streams rows with the layout described in tq_device.h and a
// grid-stride loop over rows; a wave handles 64*8/d rows per iteration.
#include "tq_codebooks.h"
#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

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

__device__ __forceinline__ void unpack8(const uint4 w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ __forceinline__ void lane_signs(const int8_t* signs, int sub, float (&sg)[8]) {
  const uint2 w = *reinterpret_cast<const uint2*>(signs + 8 * sub);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = i < 4 ? w.x : w.y;
    const int8_t b = (int8_t)(word >> (8 * (i & 3)));
    sg[i] = b < 0 ? -1.f : 1.f;
  }
}

// Count of ascending boundaries strictly below y (searchsorted, left side);
// NaN compares false everywhere and gives 0.
template <int B>
__device__ __forceinline__ uint32_t lloyd_max_index(float y, const float* lds_bnd) {
  if constexpr (B <= 3) {
    const uint32_t* bnd = boundaries<B>();
    uint32_t idx = 0;
#pragma unroll
    for (int k = 0; k < (1 << B) - 1; ++k) idx += (__uint_as_float(bnd[k]) < y) ? 1u : 0u;
    return idx;
  } else {
    uint32_t idx = 0;
#pragma unroll
    for (int step = 1 << (B - 1); step >= 1; step >>= 1)
      idx += (lds_bnd[idx + step - 1] < y) ? (uint32_t)step : 0u;
    return idx;
  }
}

// ------------------------------------------------------------------ keys
template <int D, int KB>
__device__ __forceinline__ void quantize_keys_rows(const QuantArgs& a, uint32_t blk, uint32_t nblk) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, G = D / kGroup;
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t nwave = nblk * 4u;
  const float lo = KB == 8 ? -127.f : 0.f;
  const float hi = KB == 8 ? 127.f : (float)((1 << KB) - 1);
  for (uint32_t base = wave * RPW; base < a.rows; base += nwave * RPW) {
    const uint32_t r = base + rw;
    const bool active = r < a.rows;
    uint32_t s, t, h;
    split_row(active ? r : 0u, a.split, s, t, h);
    const int64_t irow = row_index(a.in, s, t, h), orow = row_index(a.out, s, t, h);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (active) w = *reinterpret_cast<const uint4*>(a.k + irow * D + 8 * sub);
    float x[8];
    unpack8(w, x);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = __builtin_elementwise_minimum(mn, x[i]);
      mx = __builtin_elementwise_maximum(mx, x[i]);
    }
    mn = __builtin_elementwise_minimum(mn, lane_xor<1>(mn));
    mx = __builtin_elementwise_maximum(mx, lane_xor<1>(mx));
    mn = __builtin_elementwise_minimum(mn, lane_xor<2>(mn));
    mx = __builtin_elementwise_maximum(mx, lane_xor<2>(mx));
    float scale, zero;
    if constexpr (KB == 8) {
      scale = (mx - mn) / 254.0f;
      zero = __builtin_rintf((mx + mn) / (2.0f * scale));
    } else {
      scale = (mx - mn) / (float)((1 << KB) - 1);
      zero = __builtin_rintf(mn / scale);
    }
    uint64_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tq = x[i] / scale - zero;
      const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(tq), lo), hi);
      if constexpr (KB == 8)
        bits |= (uint64_t)(uint8_t)(int8_t)(int)q << (8 * i);
      else
        bits |= (uint64_t)(uint32_t)(int)q << (KB * i);
    }
    if (active) {
      store_lane_bits<KB>(a.k_q + orow * (D * KB / 8), sub, bits);
      if ((sub & 3) == 0) {
        a.k_scale[orow * G + (sub >> 2)] = (uint16_t)f16_bits(scale);
        a.k_zero[orow * G + (sub >> 2)] = (uint16_t)f16_bits(zero);
      }
    }
  }
}

// ---------------------------------------------------------------- values
template <int D, int VB>
__device__ __forceinline__ void quantize_values_rows(const QuantArgs& a, uint32_t blk, uint32_t nblk) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, G = D / kGroup;
  __shared__ float bnd_lds[VB >= 4 ? (1 << VB) : 1];
  if constexpr (VB >= 4) {
    for (int i = threadIdx.x; i < (1 << VB) - 1; i += blockDim.x)
      bnd_lds[i] = __uint_as_float(boundaries<VB>()[i]);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t nwave = nblk * 4u;
  float sg[8];
  lane_signs(a.signs, sub, sg);
  const float rd = inv_sqrt_d<D>();
  for (uint32_t base = wave * RPW; base < a.rows; base += nwave * RPW) {
    const uint32_t r = base + rw;
    const bool active = r < a.rows;
    uint32_t s, t, h;
    split_row(active ? r : 0u, a.split, s, t, h);
    const int64_t irow = row_index(a.in, s, t, h), orow = row_index(a.out, s, t, h);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (active) w = *reinterpret_cast<const uint4*>(a.v + irow * D + 8 * sub);
    float y[8];
    unpack8(w, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * sg[i];
    fwht_row<D>(y, sub);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * rd;
    // mean square of the 32-group: adjacent pairs, then pairs of pairs, ...
    const float e01 = y[0] * y[0] + y[1] * y[1];
    const float e23 = y[2] * y[2] + y[3] * y[3];
    const float e45 = y[4] * y[4] + y[5] * y[5];
    const float e67 = y[6] * y[6] + y[7] * y[7];
    float e = (e01 + e23) + (e45 + e67);
    e = e + lane_xor<1>(e);
    e = e + lane_xor<2>(e);
    const float scale = __builtin_sqrtf(e * 0.03125f);
    const float den = scale + 1e-8f;
    uint64_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t idx = lloyd_max_index<VB>(y[i] / den, bnd_lds);
      bits |= (uint64_t)idx << (VB * i);
    }
    if (active) {
      store_lane_bits<VB>(a.v_q + orow * (D * VB / 8), sub, bits);
      if ((sub & 3) == 0) a.v_scale[orow * G + (sub >> 2)] = (uint16_t)f16_bits(scale);
    }
  }
}

// ------------------------------------------------------------- dequantize
template <int D, int KB>
__device__ __forceinline__ void dequantize_keys_rows(const DequantArgs& a, uint32_t blk, uint32_t nblk) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, G = D / kGroup;
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t nwave = nblk * 4u;
  for (uint32_t base = wave * RPW; base < a.rows; base += nwave * RPW) {
    const uint32_t r = base + rw;
    if (r >= a.rows) continue;
    uint32_t s, t, h;
    split_row(r, a.split, s, t, h);
    const int64_t irow = row_index(a.in, s, t, h), orow = row_index(a.out, s, t, h);
    const uint64_t bits = load_lane_bits<KB>(a.k_q + irow * (D * KB / 8), sub);
    const float sc = canon_nan(f16_value(a.k_scale[irow * G + (sub >> 2)]));
    const float zp = canon_nan(f16_value(a.k_zero[irow * G + (sub >> 2)]));
    float k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q;
      if constexpr (KB == 8)
        q = (float)(int8_t)(bits >> (8 * i));
      else
        q = (float)(uint32_t)((bits >> (KB * i)) & ((1u << KB) - 1));
      k[i] = (q + zp) * sc;
    }
    uint4 o;
    o.x = pack_bf16x2(k[0], k[1]);
    o.y = pack_bf16x2(k[2], k[3]);
    o.z = pack_bf16x2(k[4], k[5]);
    o.w = pack_bf16x2(k[6], k[7]);
    *reinterpret_cast<uint4*>(a.k + orow * D + 8 * sub) = o;
  }
}

template <int D, int VB>
__device__ __forceinline__ void dequantize_values_rows(const DequantArgs& a, uint32_t blk, uint32_t nblk) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, G = D / kGroup;
  __shared__ float cen_lds[1 << VB];
  for (int i = threadIdx.x; i < (1 << VB); i += blockDim.x)
    cen_lds[i] = __uint_as_float(centroids<VB>()[i]);
  __syncthreads();
  const int lane = threadIdx.x & 63, sub = lane % LPR, rw = lane / LPR;
  const uint32_t wave = blk * 4u + (threadIdx.x >> 6);
  const uint32_t nwave = nblk * 4u;
  float sg[8];
  lane_signs(a.signs, sub, sg);
  const float rd = inv_sqrt_d<D>();
  for (uint32_t base = wave * RPW; base < a.rows; base += nwave * RPW) {
    const uint32_t r = base + rw;
    const bool active = r < a.rows;
    uint32_t s, t, h;
    split_row(active ? r : 0u, a.split, s, t, h);
    const int64_t irow = row_index(a.in, s, t, h), orow = row_index(a.out, s, t, h);
    uint64_t bits = 0;
    float sc = 0.f;
    if (active) {
      bits = load_lane_bits<VB>(a.v_q + irow * (D * VB / 8), sub);
      sc = canon_nan(f16_value(a.v_scale[irow * G + (sub >> 2)]));
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = cen_lds[(bits >> (VB * i)) & ((1u << VB) - 1)] * sc;
    fwht_row<D>(z, sub);
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (z[i] * rd) * sg[i];
    if (active) {
      uint4 o;
      o.x = pack_bf16x2(z[0], z[1]);
      o.y = pack_bf16x2(z[2], z[3]);
      o.z = pack_bf16x2(z[4], z[5]);
      o.w = pack_bf16x2(z[6], z[7]);
      *reinterpret_cast<uint4*>(a.v + orow * D + 8 * sub) = o;
    }
  }
}

// One launch per call: even blocks stream key rows, odd blocks value rows,
// so both halves progress side by side over the whole grid.
template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  const uint32_t blk = blockIdx.x >> 1, nblk = gridDim.x >> 1;
  if (blockIdx.x & 1)
    quantize_values_rows<D, VB>(a, blk, nblk);
  else
    quantize_keys_rows<D, KB>(a, blk, nblk);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  // with one output skipped every block works on the other
  const bool both = a.k && a.v;
  const uint32_t blk = both ? blockIdx.x >> 1 : blockIdx.x;
  const uint32_t nblk = both ? gridDim.x >> 1 : gridDim.x;
  const bool values = both ? (blockIdx.x & 1) : (a.v != nullptr);
  if (values)
    dequantize_values_rows<D, VB>(a, blk, nblk);
  else
    dequantize_keys_rows<D, KB>(a, blk, nblk);
}

// ------------------------------------------------------------- dispatch
// Blocks per half: enough 16-row chunks to cover the rows, capped so a block
// loops over several chunks on large inputs.
static unsigned blocks_per_half(uint32_t rows, int d, int max_blocks) {
  const uint32_t rows_per_block = 4u * (64u * 8u / (uint32_t)d);
  uint32_t blocks = (rows + rows_per_block - 1) / rows_per_block;
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
  const dim3 grid(2 * blocks_per_half(a.rows, D, max_blocks));
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
  const unsigned half = blocks_per_half(a.rows, D, max_blocks);
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

hipError_t launch_dequantize(const DequantArgs& a, int d, int kb, int vb, hipStream_t st, int max_blocks) {
  switch (d) {
    case 64: return launch_dequant_d<64>(a, kb, vb, st, max_blocks);
    case 128: return launch_dequant_d<128>(a, kb, vb, st, max_blocks);
    case 256: return launch_dequant_d<256>(a, kb, vb, st, max_blocks);
    default: return launch_dequant_d<512>(a, kb, vb, st, max_blocks);
  }
}

}  // namespace tq
