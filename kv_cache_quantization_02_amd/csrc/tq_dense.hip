// tq_dense.hip -- the paper variant of the codec on gfx950 matrix cores.
//
// TurboQuant KV design pages, "Oracle chain": the paper's own codec rotates
// the whole head vector by a dense random orthogonal matrix P (from the QR
// decomposition of a Gaussian matrix), keeps one norm per vector instead of
// per-group scales, codes every rotated coordinate with the Lloyd-Max table
// of a unit normal, and may add a QJL stage: one sign bit per coordinate of a
// Gaussian projection S of the residual, with the residual norm.
//
//   quantize   norm = ||x||;  y = P x;  idx_i = #{boundaries < sqrt(d) y_i / norm}
//              QJL: rho = y - norm * c[idx] / sqrt(d);  gamma = ||rho||;
//                   q_i = [(S rho)_i >= 0]
//   dequantize y_hat = norm * c[idx] / sqrt(d)
//                      (+ sqrt(pi/2) / d * gamma * S^T (2q - 1) with QJL);
//              x_hat = P^T y_hat
//
// Both products are dense d x d contractions, so they run on
// v_mfma_f32_16x16x32_bf16 (operand layout for lane l: A[l%16][8(l/16)+i],
// B[8(l/16)+i][l%16], D[4(l/16)+i][l%16]).  The matrix is the A operand: a
// block copies it once into LDS in fragment order (fragment (t, k) is 1 KB,
// lane l's 16 bytes at 16 l, so every A read is one conflict-free
// ds_read_b128).  Rows of the batch are the 16 columns of the B operand and
// of the result.  Output coordinate o and contraction index are permuted so
// that lane-group g = l/16 owns the W = d/4 consecutive coordinates
// [W g, W g + W) of its row on both sides of every product:
//   result row m of output tile t   <->  coordinate W (m/4) + 4 t + m%4
//   contraction slot 8 g + e of chunk k  <->  coordinate W g + 8 k + e
// so a lane's results are its next product's B operand without any exchange,
// its bf16 input load is 2W contiguous bytes, its code bits are one
// contiguous piece of the row's bitstream, and per-row sums need only the
// four lane-groups (two permlane swaps).
//
// Exactness: bf16 rows and bf16 matrices make every MFMA product exact; sums
// are float32.  Operands that are float32 (the residual, the reconstruction)
// are split into bf16 hi + lo and contracted twice, leaving a relative
// operand error below 2^-16.
#include "tq_codebooks.h"
#include "tq_launch.h"

namespace tq {

namespace {

typedef __bf16 dn_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dn_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t dn_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dn_u32x4 dn_lds_u32x4;
typedef __attribute__((address_space(3))) uint16_t dn_lds_u16;

__constant__ uint32_t kDnCen1[] = {TQ_CENTROIDS_1BIT}, kDnBnd1[] = {TQ_BOUNDARIES_1BIT};
__constant__ uint32_t kDnCen2[] = {TQ_CENTROIDS_2BIT}, kDnBnd2[] = {TQ_BOUNDARIES_2BIT};
__constant__ uint32_t kDnCen3[] = {TQ_CENTROIDS_3BIT}, kDnBnd3[] = {TQ_BOUNDARIES_3BIT};
__constant__ uint32_t kDnCen4[] = {TQ_CENTROIDS_4BIT}, kDnBnd4[] = {TQ_BOUNDARIES_4BIT};

template <int B>
__device__ __forceinline__ const uint32_t* dn_centroids() {
  if constexpr (B == 1) return kDnCen1;
  else if constexpr (B == 2) return kDnCen2;
  else if constexpr (B == 3) return kDnCen3;
  else return kDnCen4;
}
template <int B>
__device__ __forceinline__ const uint32_t* dn_boundaries() {
  if constexpr (B == 1) return kDnBnd1;
  else if constexpr (B == 2) return kDnBnd2;
  else if constexpr (B == 3) return kDnBnd3;
  else return kDnBnd4;
}

template <int D>
struct DenseCfg {
  static constexpr int W = D / 4;      // coordinates per lane and row
  static constexpr int NT = D / 16;    // result tiles of 16 coordinates
  static constexpr int NK = D / 32;    // contraction chunks of 32
  static constexpr int NC = D == 64 ? 4 : 2;  // 16-row column tiles per wave
  static constexpr int RW = 16 * NC;   // rows per wave and step
  static constexpr int MAT = D * D * 2;  // bytes of one matrix in LDS
};

// Sum of v over the four lanes n, n+16, n+32, n+48 (every lane gets it).
__device__ __forceinline__ float dn_sum_groups(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

__device__ __forceinline__ uint32_t dn_pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// Coordinate maps.  Result row m of output tile t, and contraction slot
// 8 gp + e of chunk kc (gp = l/16 of the lane holding it), stand for:
//   kBlocked:     lane-group g owns [W g, W g + W):
//       out(t, m) = W (m/4) + 4 t + m%4,     in(kc, gp, e) = W gp + 8 kc + e
//   kInterleaved: lane-group g owns 32 q + 8 g + [0, 8) for every q:
//       out(t, m) = 32 (t/2) + 8 (m/4) + 4 (t%2) + m%4,   in(kc, gp, e) = 32 kc + 8 gp + e
//   kRows (output only, for the product whose data is the A operand):
//       out(t, n) = NT n + t, so lane n holds NT consecutive coordinates of
//       four data rows
// With the first two a lane's result j = 4 t + e is its B operand element
// j = 8 kc + e of the next product.  The quantizer uses kBlocked (a lane's
// code bits are one piece of the bitstream); the dequantizer reads its codes
// in the kInterleaved order and writes its rows through kRows, so that every
// store instruction covers whole rows.
enum { kBlocked = 0, kInterleaved = 1, kRows = 2 };

template <int D, int MAP>
__device__ __forceinline__ int dn_out_coord(int t, int m) {
  if constexpr (MAP == kInterleaved) return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
  else if constexpr (MAP == kRows) return (D / 16) * m + t;
  else return (D / 4) * (m >> 2) + 4 * t + (m & 3);
}
template <int D, int MAP>
__device__ __forceinline__ int dn_in_coord(int kc, int gp) {
  if constexpr (MAP == kInterleaved) return 32 * kc + 8 * gp;
  else return (D / 4) * gp + 8 * kc;
}
template <int D, int MAP>
__device__ __forceinline__ void dn_out_slot(int o, int& t, int& m) {
  if constexpr (MAP == kInterleaved) {
    const int r = o & 31;
    t = 2 * (o >> 5) + ((r & 7) >> 2);
    m = 4 * (r >> 3) + (r & 3);
  } else if constexpr (MAP == kRows) {
    t = o % (D / 16);
    m = o / (D / 16);
  } else {
    const int j = o % (D / 4);
    t = j >> 2;
    m = 4 * (o / (D / 4)) + (j & 3);
  }
}
template <int D, int MAP>
__device__ __forceinline__ void dn_in_slot(int in, int& kc, int& gp, int& e) {
  if constexpr (MAP == kInterleaved) {
    kc = in >> 5;
    gp = (in >> 3) & 3;
    e = in & 7;
  } else {
    const int j = in % (D / 4);
    gp = in / (D / 4);
    kc = j >> 3;
    e = j & 7;
  }
}

// Copy the d x d bf16 matrix M (row-major) into LDS in fragment order for
// out = Mx (TRANSPOSE = false) or out = M^T x (true).  Fragment (t, kc) lane
// l holds the 8 elements (out(t, l%16), in(kc, l/16, 0..7)); the same bytes
// serve as the A operand (matrix rows = outputs) or, with the data as A, as
// the B operand (matrix columns = outputs).
template <int D, bool TRANSPOSE, int OUT, int IN>
__device__ __forceinline__ void dn_load_matrix(uint8_t* lds, const uint16_t* __restrict__ m) {
  using C = DenseCfg<D>;
  constexpr int NK = C::NK;
  if constexpr (!TRANSPOSE) {
    for (int p = threadIdx.x; p < C::NT * NK * 64; p += 256) {
      const int f = p >> 6, l = p & 63;
      const int t = f / NK, kc = f % NK;
      const int o = dn_out_coord<D, OUT>(t, l & 15);
      const int in0 = dn_in_coord<D, IN>(kc, l >> 4);
      const dn_u32x4 v = *reinterpret_cast<const dn_u32x4*>(m + o * D + in0);
      *(dn_lds_u32x4*)(lds + 16 * p) = v;
    }
  } else {
    // element M[a][b] is (row b, column a) of M^T: read M in 16-byte pieces
    // and scatter the eight elements
    for (int p = threadIdx.x; p < D * D / 8; p += 256) {
      const int a = p / (D / 8), b0 = (p % (D / 8)) * 8;
      const dn_u32x4 v = *reinterpret_cast<const dn_u32x4*>(m + a * D + b0);
      int kc, gp, e;
      dn_in_slot<D, IN>(a, kc, gp, e);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int t, mrow;
        dn_out_slot<D, OUT>(b0 + i, t, mrow);
        const uint16_t val = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
        *(dn_lds_u16*)(lds + 2 * (((t * NK + kc) * 64 + 16 * gp + mrow) * 8 + e)) = val;
      }
    }
  }
}

__device__ __forceinline__ dn_bf16x8 dn_frag(const uint8_t* lds, int f, int lane) {
  const dn_u32x4 v = *(const dn_lds_u32x4*)(lds + 1024 * f + 16 * lane);
  return __builtin_bit_cast(dn_bf16x8, v);
}

__device__ __forceinline__ dn_bf16x8 dn_bits(dn_u32x4 v) { return __builtin_bit_cast(dn_bf16x8, v); }

// acc[c][t] += M x over all chunks, M's fragments in LDS, x the B operands.
// The fragments of tile t+1 are read while tile t's products run; the
// scheduling barrier keeps the compiler from hoisting further reads (which
// would hold every fragment of the matrix in registers).
template <int D>
__device__ __forceinline__ void dn_gemm(dn_f32x4 (&acc)[DenseCfg<D>::NC][DenseCfg<D>::NT], const uint8_t* lds,
                                        const dn_u32x4 (&bx)[DenseCfg<D>::NC][DenseCfg<D>::NK], int lane) {
  using C = DenseCfg<D>;
  dn_bf16x8 cur[C::NK], nxt[C::NK];
#pragma unroll
  for (int kc = 0; kc < C::NK; ++kc) cur[kc] = dn_frag(lds, kc, lane);
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    if (t + 1 < C::NT) {
#pragma unroll
      for (int kc = 0; kc < C::NK; ++kc) nxt[kc] = dn_frag(lds, (t + 1) * C::NK + kc, lane);
    }
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) {
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[kc], dn_bits(bx[c][kc]), acc[c][t], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) cur[kc] = nxt[kc];
  }
}

// acc[c][t] += x M^T with the data as the A operand: lane (n, g) receives
// rows 16 c + 4 g + i (i = 0..3) of the batch at output coordinate out(t, n).
template <int D>
__device__ __forceinline__ void dn_gemm_rows(dn_f32x4 (&acc)[DenseCfg<D>::NC][DenseCfg<D>::NT], const uint8_t* lds,
                                             const dn_u32x4 (&bx)[DenseCfg<D>::NC][DenseCfg<D>::NK], int lane) {
  using C = DenseCfg<D>;
  dn_bf16x8 cur[C::NK], nxt[C::NK];
#pragma unroll
  for (int kc = 0; kc < C::NK; ++kc) cur[kc] = dn_frag(lds, kc, lane);
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    if (t + 1 < C::NT) {
#pragma unroll
      for (int kc = 0; kc < C::NK; ++kc) nxt[kc] = dn_frag(lds, (t + 1) * C::NK + kc, lane);
    }
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) {
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dn_bits(bx[c][kc]), cur[kc], acc[c][t], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) cur[kc] = nxt[kc];
  }
}

// Split float32 values (local coordinates j = 4t + e of acc) into bf16 hi
// and lo B operands: chunk kc holds local coordinates 8kc .. 8kc+7.
template <int D>
__device__ __forceinline__ void dn_split(const dn_f32x4 (&v)[DenseCfg<D>::NC][DenseCfg<D>::NT],
                                         dn_u32x4 (&hi)[DenseCfg<D>::NC][DenseCfg<D>::NK],
                                         dn_u32x4 (&lo)[DenseCfg<D>::NC][DenseCfg<D>::NK]) {
  using C = DenseCfg<D>;
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int j = 8 * kc + 2 * w;
        const float v0 = v[c][j >> 2][j & 3], v1 = v[c][(j + 1) >> 2][(j + 1) & 3];
        const uint32_t h = dn_pack_bf16(v0, v1);
        hi[c][kc][w] = h;
        lo[c][kc][w] = dn_pack_bf16(v0 - bf16_lo(h), v1 - bf16_hi(h));
      }
    }
  }
}

// Bytes of a lane's piece of the index plane row, and of the QJL plane row.
template <int D, int B>
struct DenseSeg {
  static constexpr int BITS = DenseCfg<D>::W * B;
  static constexpr int BYTES = BITS / 8;
  static constexpr int WORDS = (BYTES + 3) / 4;
};

template <int BYTES, int WORDS>
__device__ __forceinline__ void dn_store_seg(uint8_t* p, const uint32_t (&w)[WORDS]) {
  if constexpr (BYTES % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) reinterpret_cast<uint32_t*>(p)[i] = w[i];
  } else {
#pragma unroll
    for (int i = 0; i < BYTES / 2; ++i) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
  }
}

template <int B, int WORDS>
__device__ __forceinline__ void dn_put_field(uint32_t (&w)[WORDS], int j, uint32_t v) {
  const int bit = B * j, wi = bit >> 5, sh = bit & 31;
  w[wi] |= v << sh;
  if (sh + B > 32) w[wi + 1] |= v >> (32 - sh);
}

// ------------------------------------------------------------- quantize
template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void dense_quantize_kernel(DenseArgs a) {
  using C = DenseCfg<D>;
  using Seg = DenseSeg<D, B>;
  constexpr int W = C::W, NT = C::NT, NK = C::NK, NC = C::NC;
  constexpr int HALF = 1 << (B - 1), NP = HALF - 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::MAT * (QJL ? 2 : 1)];
  dn_load_matrix<D, false, kBlocked, kBlocked>(lds, a.rot);
  if constexpr (QJL) dn_load_matrix<D, false, kBlocked, kBlocked>(lds + C::MAT, a.proj);
  __syncthreads();

  const int lane = (int)__lane_id();
  const int n = lane & 15, g = lane >> 4;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // positive half of the symmetric table: boundaries b[HALF + j], centroids c[HALF + j]
  float pbnd[NP > 0 ? NP : 1], pcen[HALF];
#pragma unroll
  for (int j = 0; j < NP; ++j) pbnd[j] = __uint_as_float(dn_boundaries<B>()[HALF + j]);
#pragma unroll
  for (int j = 0; j < HALF; ++j) pcen[j] = __uint_as_float(dn_centroids<B>()[HALF + j]);
  const float rsd = inv_sqrt_d<D>();

  // the rows of a tile: B operands (bf16 x), plane row index, liveness
  dn_u32x4 bx[NC][NK];
  int64_t po[NC];
  bool act[NC];
  auto load_tile = [&](uint32_t tile) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t r = tile * C::RW + 16 * c + n;
      act[c] = r < a.rows;
      uint32_t s, t, h;
      split_row(act[c] ? r : 0u, a.split, s, t, h);
      const int64_t xo = row_index(a.x_map, s, t, h);
      po[c] = row_index(a.plane_map, s, t, h);
      const dn_u32x4* src = reinterpret_cast<const dn_u32x4*>(a.x + xo * D + W * g);
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) bx[c][kc] = act[c] ? src[kc] : dn_u32x4{0u, 0u, 0u, 0u};
    }
  };
  // code words of a zero row: every index is #{b < 0} = HALF - 1
  uint32_t zseg[Seg::WORDS];
#pragma unroll
  for (int i = 0; i < Seg::WORDS; ++i) zseg[i] = 0u;
#pragma unroll
  for (int j = 0; j < W; ++j) dn_put_field<B>(zseg, j, (uint32_t)(HALF - 1));

  uint32_t tile = blockIdx.x * 4u + wave;
  if (tile * (uint32_t)C::RW >= a.rows) return;
  load_tile(tile);
  for (;;) {
    // norms
    float nrm[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float ss = 0.f;
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float v0 = bf16_lo(bx[c][kc][w]), v1 = bf16_hi(bx[c][kc][w]);
          ss = __builtin_fmaf(v0, v0, ss);
          ss = __builtin_fmaf(v1, v1, ss);
        }
      }
      nrm[c] = __builtin_sqrtf(dn_sum_groups(ss));
    }
    // y = P x
    dn_f32x4 acc[NC][NT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
    dn_gemm<D>(acc, lds, bx, lane);

    // the next tile's rows load while this one is coded
    int64_t pc[NC];
    bool ac[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      pc[c] = po[c];
      ac[c] = act[c];
    }
    const uint32_t next = tile + gridDim.x * 4u;
    const bool more = next * (uint32_t)C::RW < a.rows;
    if (more) load_tile(next);

    float gam[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // u > b  <=>  |y| > b * norm / sqrt(d) on the side of y's sign
      const float sc = nrm[c] * rsd;
      float thr[NP > 0 ? NP : 1];
#pragma unroll
      for (int j = 0; j < NP; ++j) thr[j] = pbnd[j] * sc;
      uint32_t seg[Seg::WORDS];
#pragma unroll
      for (int i = 0; i < Seg::WORDS; ++i) seg[i] = 0u;
      float gg = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = acc[c][t][e];
          const float ay = __builtin_fabsf(y);
          uint32_t m = HALF;
          float mag = pcen[0];
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            const bool above = thr[j] < ay;
            m += above ? 1u : 0u;
            if constexpr (QJL) mag = above ? pcen[j + 1] : mag;
          }
          // #{b < u} = HALF + m for y > 0 and HALF - 1 - m = (HALF + m) ^ (2 HALF - 1)
          // for y < 0; all ones where the sign bit is set (y = +0 lies on the
          // middle boundary 0, a tie either way; a zero row is set below)
          const uint32_t neg = (uint32_t)(__float_as_int(y) >> 31);
          const uint32_t idx = m ^ (neg & (uint32_t)(2 * HALF - 1));
          dn_put_field<B>(seg, 4 * t + e, idx);
          if constexpr (QJL) {
            const float yh = __uint_as_float(__float_as_uint(mag) ^ (neg & 0x80000000u));
            const float rho = __builtin_fmaf(-yh, sc, y);
            acc[c][t][e] = rho;
            gg = __builtin_fmaf(rho, rho, gg);
          }
        }
      }
      if (nrm[c] == 0.f) {
#pragma unroll
        for (int i = 0; i < Seg::WORDS; ++i) seg[i] = zseg[i];
      }
      if (ac[c]) {
        dn_store_seg<Seg::BYTES>(a.idx + pc[c] * (D * B / 8) + g * Seg::BYTES, seg);
        if (g == 0) a.norm[pc[c]] = nrm[c];
      }
      if constexpr (QJL) gam[c] = __builtin_sqrtf(dn_sum_groups(gg));
    }

    if constexpr (QJL) {
      dn_u32x4 hi[NC][NK], lo[NC][NK];
      dn_split<D>(acc, hi, lo);
      dn_f32x4 sp[NC][NT];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t) sp[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
      dn_gemm<D>(sp, lds + C::MAT, hi, lane);
      dn_gemm<D>(sp, lds + C::MAT, lo, lane);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t qb[1] = {0u};
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) qb[0] |= (sp[c][t][e] >= 0.f ? 1u : 0u) << (4 * t + e);
        if (ac[c]) {
          dn_store_seg<W / 8>(a.qjl + pc[c] * (D / 8) + g * (W / 8), qb);
          if (g == 0) a.gamma[pc[c]] = gam[c];
        }
      }
    }
    if (!more) break;
    tile = next;
  }
}

// An output element: MSE sums finite centroid products, so the (canonical)
// row scale decides any NaN; QJL sums split operands that may carry any NaN,
// so each element is canonicalised.
template <bool QJL>
__device__ __forceinline__ float dn_out(float v, float f) {
  if constexpr (QJL) return canon_nan(v);
  else return v * f;
}

// ----------------------------------------------------------- dequantize
template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void dense_dequantize_kernel(DenseArgs a) {
  using C = DenseCfg<D>;
  constexpr int NT = C::NT, NK = C::NK, NC = C::NC;
  // P^T for the final product (outputs in kRows order), S^T for the QJL term
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::MAT * (QJL ? 2 : 1)];
  // MSE: centroid as its bf16 hi (low half) and lo (high half); QJL: float32
  __shared__ uint32_t lut[1 << B];
  dn_load_matrix<D, true, kRows, kInterleaved>(lds, a.rot);
  if constexpr (QJL) dn_load_matrix<D, true, kInterleaved, kInterleaved>(lds + C::MAT, a.proj);
  if (threadIdx.x < (1u << B)) {
    const float cv = __uint_as_float(dn_centroids<B>()[threadIdx.x]);
    if constexpr (QJL) {
      lut[threadIdx.x] = __float_as_uint(cv);
    } else {
      const uint32_t h = dn_pack_bf16(cv, 0.f) & 0xffffu;
      const uint32_t l = dn_pack_bf16(cv - bf16_lo(h), 0.f) & 0xffffu;
      lut[threadIdx.x] = h | (l << 16);
    }
  }
  __syncthreads();

  const int lane = (int)__lane_id();
  const int n = lane & 15, g = lane >> 4;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float rsd = inv_sqrt_d<D>();
  constexpr float kQjl = (float)(1.2533141373155002512 / D);  // sqrt(pi/2) / d

  // fb[c][kc]: the 8 code fields of local elements 8 kc .. 8 kc + 7 of row
  // 16 c + n, i.e. of coordinates 32 kc + 8 g + [0, 8): stream bytes
  // B (4 kc + g) ..; qb the matching 8 sign bits, byte 4 kc + g of the QJL row
  uint32_t fb[NC][NK], qb[NC][NK];
  float sc[NC], cg[NC];
  int64_t xo[NC];
  auto load_tile = [&](uint32_t tile) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t r = tile * C::RW + 16 * c + n;
      const bool act = r < a.rows;
      uint32_t s, t, h;
      split_row(act ? r : 0u, a.split, s, t, h);
      xo[c] = row_index(a.x_map, s, t, h);
      const int64_t po = row_index(a.plane_map, s, t, h);
      if (act) {
        const uint8_t* irow = a.idx + po * (D * B / 8);
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) fb[c][kc] = (uint32_t)load_lane_bits<B>(irow, 4 * kc + g);
        sc[c] = a.norm[po];
        if constexpr (QJL) {
          const uint8_t* qrow = a.qjl + po * (D / 8);
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) qb[c][kc] = (uint32_t)load_lane_bits<1>(qrow, 4 * kc + g);
          cg[c] = a.gamma[po];
        }
      } else {
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) fb[c][kc] = 0u;
        sc[c] = 0.f;
        if constexpr (QJL) {
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) qb[c][kc] = 0u;
          cg[c] = 0.f;
        }
      }
    }
  };
  auto field = [&](int c, int j) -> uint32_t {
    return __builtin_amdgcn_ubfe(fb[c][j >> 3], (uint32_t)(B * (j & 7)), (uint32_t)B);
  };

  uint32_t tile = blockIdx.x * 4u + wave;
  if (tile * (uint32_t)C::RW >= a.rows) return;
  load_tile(tile);
  for (;;) {
    // the row scales; a NaN scale is made the default NaN so that every
    // output it reaches rounds to the canonical bf16 NaN
    float scale[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      scale[c] = canon_nan(sc[c] * rsd);
      if constexpr (QJL) cg[c] = canon_nan(cg[c] * kQjl);
    }
    // A operands of the final product: bf16 hi and lo of y_hat (MSE: of the
    // centroids, the norm scale applied to the result)
    dn_u32x4 hi[NC][NK], lo[NC][NK];
    if constexpr (!QJL) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int j = 8 * kc + 2 * w;
            const uint32_t l0 = lut[field(c, j)];
            const uint32_t l1 = lut[field(c, j + 1)];
            hi[c][kc][w] = __builtin_amdgcn_perm(l1, l0, 0x05040100u);
            lo[c][kc][w] = __builtin_amdgcn_perm(l1, l0, 0x07060302u);
          }
        }
      }
    } else {
      // y_hat = norm c[idx] / sqrt(d) + sqrt(pi/2)/d gamma S^T (2q - 1)
      dn_u32x4 bq[NC][NK];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t b0 = (qb[c][kc] >> (2 * w)) & 1u, b1 = (qb[c][kc] >> (2 * w + 1)) & 1u;
            // +1 = 0x3F80, -1 = 0xBF80
            bq[c][kc][w] = (0x3F80u | ((b0 ^ 1u) << 15)) | ((0x3F80u | ((b1 ^ 1u) << 15)) << 16);
          }
        }
      }
      dn_f32x4 sq[NC][NT];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t) sq[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
      dn_gemm<D>(sq, lds + C::MAT, bq, lane);
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float cv = __uint_as_float(lut[field(c, 4 * t + e)]);
            sq[c][t][e] = __builtin_fmaf(cg[c], sq[c][t][e], cv * scale[c]);
          }
      dn_split<D>(sq, hi, lo);
    }

    // the next tile's planes load while this one is rebuilt
    int64_t xc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xc[c] = xo[c];
    const uint32_t next = tile + gridDim.x * 4u;
    const bool more = next * (uint32_t)C::RW < a.rows;
    if (more) load_tile(next);

    // x_hat = P^T y_hat, lane (n, g) receiving rows 16 c + 4 g + i at
    // coordinates NT n .. NT n + NT - 1
    dn_f32x4 acc[NC][NT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
    dn_gemm_rows<D>(acc, lds, hi, lane);
    dn_gemm_rows<D>(acc, lds, lo, lane);

#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = 4 * g + i;  // the lane that addressed row 16 c + 4 g + i
        const uint32_t lo32 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)(uint32_t)xc[c]);
        const uint32_t hi32 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)(uint32_t)((uint64_t)xc[c] >> 32));
        const int64_t row_off = (int64_t)(((uint64_t)hi32 << 32) | lo32);
        const float f = QJL ? 1.f : __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(scale[c])));
        if (tile * C::RW + 16 * c + src >= a.rows) continue;
        uint16_t* row = a.x_out + row_off * D + NT * n;
        if constexpr (NT >= 8) {
#pragma unroll
          for (int q = 0; q < NT / 8; ++q) {
            dn_u32x4 v;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int t = 8 * q + 2 * w;
              v[w] = dn_pack_bf16(dn_out<QJL>(acc[c][t][i], f), dn_out<QJL>(acc[c][t + 1][i], f));
            }
            __builtin_nontemporal_store(v, reinterpret_cast<dn_u32x4*>(row + 8 * q));
          }
        } else {
          const uint32_t v0 = dn_pack_bf16(dn_out<QJL>(acc[c][0][i], f), dn_out<QJL>(acc[c][1][i], f));
          const uint32_t v1 = dn_pack_bf16(dn_out<QJL>(acc[c][2][i], f), dn_out<QJL>(acc[c][3][i], f));
          __builtin_nontemporal_store(v0, reinterpret_cast<uint32_t*>(row));
          __builtin_nontemporal_store(v1, reinterpret_cast<uint32_t*>(row) + 1);
        }
      }
    }
    if (!more) break;
    tile = next;
  }
}

// Resident blocks: one per CU when a block's matrices take more than half
// of the 160 KB LDS, else two; every block copies its matrices once.
template <int D>
unsigned dense_grid(uint32_t rows, bool qjl) {
  using C = DenseCfg<D>;
  const uint32_t tiles = (rows + C::RW - 1) / C::RW;
  const unsigned want = (tiles + 3) / 4;
  const unsigned per_cu = (C::MAT * (qjl ? 2 : 1) > 80 * 1024) ? 1u : 2u;
  const unsigned cap = 256u * per_cu;
  return want < cap ? want : cap;
}

template <int D, int B>
hipError_t dense_quant_db(const DenseArgs& a, bool qjl, hipStream_t st) {
  const dim3 grid(dense_grid<D>(a.rows, qjl));
  if constexpr (D <= 128) {
    if (qjl) {
      dense_quantize_kernel<D, B, true><<<grid, 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  dense_quantize_kernel<D, B, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int B>
hipError_t dense_dequant_db(const DenseArgs& a, bool qjl, hipStream_t st) {
  const dim3 grid(dense_grid<D>(a.rows, qjl));
  if constexpr (D <= 128) {
    if (qjl) {
      dense_dequantize_kernel<D, B, true><<<grid, 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  dense_dequantize_kernel<D, B, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t dense_quant_d(const DenseArgs& a, int bits, bool qjl, hipStream_t st) {
  switch (bits) {
    case 1: return dense_quant_db<D, 1>(a, qjl, st);
    case 2: return dense_quant_db<D, 2>(a, qjl, st);
    case 3: return dense_quant_db<D, 3>(a, qjl, st);
    default: return dense_quant_db<D, 4>(a, qjl, st);
  }
}

template <int D>
hipError_t dense_dequant_d(const DenseArgs& a, int bits, bool qjl, hipStream_t st) {
  switch (bits) {
    case 1: return dense_dequant_db<D, 1>(a, qjl, st);
    case 2: return dense_dequant_db<D, 2>(a, qjl, st);
    case 3: return dense_dequant_db<D, 3>(a, qjl, st);
    default: return dense_dequant_db<D, 4>(a, qjl, st);
  }
}

}  // namespace

hipError_t launch_dense_quantize(const DenseArgs& a, int d, int bits, bool qjl, hipStream_t st) {
  switch (d) {
    case 64: return dense_quant_d<64>(a, bits, qjl, st);
    case 128: return dense_quant_d<128>(a, bits, qjl, st);
    default: return dense_quant_d<256>(a, bits, qjl, st);
  }
}

hipError_t launch_dense_dequantize(const DenseArgs& a, int d, int bits, bool qjl, hipStream_t st) {
  switch (d) {
    case 64: return dense_dequant_d<64>(a, bits, qjl, st);
    case 128: return dense_dequant_d<128>(a, bits, qjl, st);
    default: return dense_dequant_d<256>(a, bits, qjl, st);
  }
}

}  // namespace tq
