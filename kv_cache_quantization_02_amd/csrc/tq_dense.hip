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
// of the result.  Output coordinates and contraction indices are permuted
// (the coordinate maps below) so that lane-group g = l/16 of a row holds the
// coordinates 32 q + 8 g + [0, 8) on both sides of every product: a lane's
// results are its next product's B operand without any exchange, loads and
// code stores are contiguous per row, and per-row sums need only the four
// lane-groups.  The dequantizer's last product takes the data as the A
// operand, so that its results spread over the lanes by rows.
//
// Exactness: bf16 rows and bf16 matrices make every MFMA product exact; sums
// are float32.  Operands that are float32 (the residual, the reconstruction)
// are split into bf16 hi + lo, both contracted against each matrix fragment
// in the same pass, leaving a relative operand error below 2^-16.
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

// NC: 16-row column tiles per wave.  Two let each matrix fragment serve 32
// rows, one needs half the registers.  The dequantizer takes one up to
// d = 128: more resident waves measured 8-9% faster there, while at d = 256
// the doubled fragment reads from LDS cost more than that.  The MSE quantizer
// takes two (its coding of one output tile overlaps the next tile's
// products).  The QJL quantizer takes one, except at d = 128 with 1 or 2
// bits: at d = 128 one tile takes it from 200-262 VGPRs to 116-159, three
// resident waves per SIMD instead of one or two, which made 3 and 4 bits
// 23% and 34% faster but 1 and 2 bits 2-3% slower; at d = 64 one tile was
// 5-13% faster at every width.
template <int D>
constexpr int kDeqNC = D <= 128 ? 1 : 2;
template <int D, int B, bool QJL>
constexpr int kQuantNC = (!QJL || (D == 128 && B <= 2)) ? 2 : 1;
template <int D, int NCV>
struct DenseCfg {
  static constexpr int NT = D / 16;    // result tiles of 16 coordinates
  static constexpr int NK = D / 32;    // contraction chunks of 32
  static constexpr int NC = NCV;
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
//   kInterleaved: lane-group g owns 32 q + 8 g + [0, 8) for every q:
//       out(t, m) = 32 (t/2) + 8 (m/4) + 4 (t%2) + m%4,   in(kc, gp, e) = 32 kc + 8 gp + e
//   kRows (output only, for the product whose data is the A operand):
//       out(t, n) = NT n + t, so lane n holds NT consecutive coordinates of
//       four data rows
//   kGroups (output only, for the MSE quantizer's one product):
//       out(t, m) = (D/4) (m/4) + 4 t + m%4, so lane-group g holds the
//       coordinates (D/4) g + [0, D/4): a contiguous run of the row's
//       bitstream, stored with whole-dword writes
// With kInterleaved a lane's result j = 4 t + e is its B operand element
// j = 8 kc + e of the next product, so products chain without any exchange;
// the four lane-groups of a row load 64 contiguous bytes per instruction; and
// a lane's 8 codes of chunk q are one B-byte piece of the row's bitstream.
// The dequantizer writes its rows through kRows, so that every store
// instruction covers whole rows.
enum { kInterleaved = 1, kRows = 2, kGroups = 3 };

template <int D, int MAP>
__device__ __forceinline__ int dn_out_coord(int t, int m) {
  if constexpr (MAP == kInterleaved) return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
  else if constexpr (MAP == kGroups) return (D / 4) * (m >> 2) + 4 * t + (m & 3);
  else return (D / 16) * m + t;
}
__device__ __forceinline__ int dn_in_coord(int kc, int gp) { return 32 * kc + 8 * gp; }
template <int D, int MAP>
__device__ __forceinline__ void dn_out_slot(int o, int& t, int& m) {
  if constexpr (MAP == kInterleaved) {
    const int r = o & 31;
    t = 2 * (o >> 5) + ((r & 7) >> 2);
    m = 4 * (r >> 3) + (r & 3);
  } else if constexpr (MAP == kGroups) {
    const int r = o % (D / 4);
    t = r >> 2;
    m = 4 * (o / (D / 4)) + (r & 3);
  } else {
    t = o % (D / 16);
    m = o / (D / 16);
  }
}
__device__ __forceinline__ void dn_in_slot(int in, int& kc, int& gp, int& e) {
  kc = in >> 5;
  gp = (in >> 3) & 3;
  e = in & 7;
}

// Copy the d x d bf16 matrix M (row-major) into LDS in fragment order for
// out = Mx (TRANSPOSE = false) or out = M^T x (true).  Fragment (t, kc) lane
// l holds the 8 elements (out(t, l%16), in(kc, l/16, 0..7)); the same bytes
// serve as the A operand (matrix rows = outputs) or, with the data as A, as
// the B operand (matrix columns = outputs).
template <int D, bool TRANSPOSE, int OUT>
__device__ __forceinline__ void dn_load_matrix(uint8_t* lds, const uint16_t* __restrict__ m) {
  using C = DenseCfg<D, 1>;
  constexpr int NK = C::NK;
  if constexpr (!TRANSPOSE) {
    for (int p = threadIdx.x; p < C::NT * NK * 64; p += 256) {
      const int f = p >> 6, l = p & 63;
      const int t = f / NK, kc = f % NK;
      const int o = dn_out_coord<D, OUT>(t, l & 15);
      const int in0 = dn_in_coord(kc, l >> 4);
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
      dn_in_slot(a, kc, gp, e);
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

// acc[c][t] += M x over all chunks, M's fragments in LDS, x the B operands
// (NX = 2: x = hi + lo, both contracted against each fragment read once).
// The fragments of tile t+1 are read while tile t's products run; the
// scheduling barrier keeps the compiler from hoisting further reads (which
// would hold every fragment of the matrix in registers).  ROWS swaps the
// operands: the data is A, so lane (n, g) receives rows 16 c + 4 g + i
// (i = 0..3) of the batch at output coordinate out(t, n).
template <int D, int NC, int NX, bool ROWS = false>
__device__ __forceinline__ void dn_gemm(dn_f32x4 (&acc)[NC][D / 16], const uint8_t* lds,
                                        const dn_u32x4 (&b0)[NC][D / 32], const dn_u32x4 (&b1)[NC][D / 32],
                                        int lane) {
  using C = DenseCfg<D, NC>;
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
      for (int c = 0; c < C::NC; ++c) {
        if constexpr (ROWS) {
          acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dn_bits(b0[c][kc]), cur[kc], acc[c][t], 0, 0, 0);
          if constexpr (NX == 2)
            acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dn_bits(b1[c][kc]), cur[kc], acc[c][t], 0, 0, 0);
        } else {
          acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[kc], dn_bits(b0[c][kc]), acc[c][t], 0, 0, 0);
          if constexpr (NX == 2)
            acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[kc], dn_bits(b1[c][kc]), acc[c][t], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < C::NK; ++kc) cur[kc] = nxt[kc];
  }
}

// Split float32 values (local coordinates j = 4t + e of acc) into bf16 hi
// and lo B operands: chunk kc holds local coordinates 8kc .. 8kc+7.
template <int D, int NC>
__device__ __forceinline__ void dn_split(const dn_f32x4 (&v)[NC][D / 16], dn_u32x4 (&hi)[NC][D / 32],
                                         dn_u32x4 (&lo)[NC][D / 32]) {
  using C = DenseCfg<D, NC>;
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

// Store a lane's run of RB code bytes (RB = d B / 32, a multiple of 2; the
// run starts RB g bytes into a row of d B / 8 bytes): whole dwords when RB is
// a multiple of 4 (the run is then dword-aligned), else 16-bit halves.
template <int RB, int NW>
__device__ __forceinline__ void dn_store_run(uint8_t* p, const uint32_t (&w)[NW]) {
  static_assert(RB % 2 == 0 && (RB + 3) / 4 <= NW, "run size");
  if constexpr (RB % 4 == 0) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < RB / 4; ++i) q[i] = w[i];
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int i = 0; i < RB / 2; ++i) q[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
  }
}

// ------------------------------------------------------------- quantize
template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void dense_quantize_kernel(DenseArgs a) {
  using C = DenseCfg<D, kQuantNC<D, B, QJL>>;
  constexpr int NT = C::NT, NK = C::NK, NC = C::NC;
  constexpr int HALF = 1 << (B - 1), NP = HALF - 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::MAT * (QJL ? 2 : 1)];
  // MSE: codes in contiguous runs (kGroups); QJL: the residual chains into
  // the projection (kInterleaved)
  dn_load_matrix<D, false, QJL ? kInterleaved : kGroups>(lds, a.rot);
  if constexpr (QJL) dn_load_matrix<D, false, kInterleaved>(lds + C::MAT, a.proj);
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

  // the rows of a tile: B operands (bf16 x), plane row index, liveness; the
  // next tile's rows load into the second set while this one is worked on
  dn_u32x4 bx[NC][NK], bn[NC][NK];
  int64_t po[NC], pn[NC];
  bool act[NC], an[NC];
  auto load_tile = [&](uint32_t tile, dn_u32x4 (&dst)[NC][NK], int64_t (&pdst)[NC], bool (&adst)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t r = tile * C::RW + 16 * c + n;
      adst[c] = r < a.rows;
      uint32_t s, t, h;
      split_row(adst[c] ? r : 0u, a.split, s, t, h);
      const int64_t xo = check_row(row_index(a.x_map, s, t, h), a.x_ext, kChkDenseIn);
      pdst[c] = row_index(a.plane_map, s, t, h);
      // a plane row outside the extent is not written (checked build)
      if (kChecked && adst[c]) adst[c] = check_ok(pdst[c] < a.plane_ext, kChkDenseOut);
      // chunk kc: coordinates 32 kc + 8 g + [0, 8), so the four lane-groups
      // of a row read 64 contiguous bytes per instruction
      const uint16_t* src = a.x + xo * D + 8 * g;
#pragma unroll
      for (int kc = 0; kc < NK; ++kc)
        dst[c][kc] = adst[c] ? *reinterpret_cast<const dn_u32x4*>(src + 32 * kc) : dn_u32x4{0u, 0u, 0u, 0u};
    }
  };
  // a zero row: every index is #{b < 0} = HALF - 1; an 8-coordinate piece
  // (QJL) or the words of a lane's run of D/4 coordinates (MSE)
  constexpr int RB = D * B / 32;  // bytes of a lane's run
  uint32_t zpiece = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) zpiece |= (uint32_t)(HALF - 1) << (B * e);
  uint32_t zrun[NK];
#pragma unroll
  for (int q = 0; q < NK; ++q) zrun[q] = 0u;
#pragma unroll
  for (int k = 0; k < D / 4; ++k) {
    zrun[(B * k) >> 5] |= (uint32_t)(HALF - 1) << ((B * k) & 31);
    if (((B * k) & 31) + B > 32) zrun[((B * k) >> 5) + 1] |= (uint32_t)(HALF - 1) >> (32 - ((B * k) & 31));
  }

  uint32_t tile = blockIdx.x * 4u + wave;
  if (tile * (uint32_t)C::RW >= a.rows) return;
  load_tile(tile, bx, po, act);
  for (;;) {
    // the next tile's rows: loaded now into the second set (MSE), or into the
    // first once the rotation has consumed it (QJL, which needs the registers)
    const uint32_t next = tile + gridDim.x * 4u;
    const bool more = next * (uint32_t)C::RW < a.rows;
    int64_t pc[NC];
    bool ac[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      pc[c] = po[c];
      ac[c] = act[c];
    }
    if constexpr (!QJL) {
      if (more) load_tile(next, bn, pn, an);
    }

    // norms: the Gram matrix X X^T of each 16-row column tile on the matrix
    // cores (the B registers serve as both operands: exact products, float32
    // sums); row n's squared norm is its diagonal entry, held by lane
    // (n, n/4) as element n%4, and fetched by every lane of the row
    float nrm[NC], sc[NC], thr[NC][NP > 0 ? NP : 1];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      dn_f32x4 gram = dn_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NK; ++kc)
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dn_bits(bx[c][kc]), dn_bits(bx[c][kc]), gram, 0, 0, 0);
      const float g01 = (n & 1) ? gram[1] : gram[0];
      const float g23 = (n & 1) ? gram[3] : gram[2];
      const float diag = (n & 2) ? g23 : g01;
      const int holder = 16 * (n >> 2) + n;
      const float ss = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * holder, __float_as_int(diag)));
      nrm[c] = __builtin_sqrtf(ss);
      // u > b  <=>  |y| > b * norm / sqrt(d) on the side of y's sign
      sc[c] = nrm[c] * rsd;
#pragma unroll
      for (int j = 0; j < NP; ++j) thr[c][j] = pbnd[j] * sc[c];
    }

    // y = P x, each output tile coded while the next one's products run (MSE).
    // piece[c][]: MSE, the words of the lane's run, coordinates (D/4) g +
    // [0, D/4) of row 16 c + n (stream bytes RB g ..); QJL, piece[c][q] holds
    // the 8 codes of coordinates 32 q + 8 g + [0, 8) (stream bytes B (4 q + g) ..)
    dn_f32x4 acc[NC][NT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t piece[NC][NK];
    float gg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      gg[c] = 0.f;
#pragma unroll
      for (int q = 0; q < NK; ++q) piece[c][q] = 0u;
    }
    auto code_tile = [&](int t) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (!QJL) {
          // codes e = 3 .. 0 of this tile, pushed highest stream position
          // first (#{b < u} is HALF + m above zero and HALF - 1 - m
          // otherwise, m = #{thr < |y|}; a zero row is set below); they are
          // run coordinates 4 t + e, at run bits 4 B t ..
          // The products enter the assembly block through one compiler-visible
          // add: the compiler inserts the wait states a vector read of an MFMA
          // result needs, which it does not do for an inline-assembly operand
          // (+0 also turns -0 into +0; both code as the lower middle cell).
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[c][t][e] + 0.0f;
          uint32_t w = 0u;
          index_pair<B, 2 * B>(y[3], y[2], thr[c], w, w);
          index_pair<B, 2 * B>(y[1], y[0], thr[c], w, w);
          const int off = 4 * B * t;
          piece[c][off >> 5] |= w << (off & 31);
          if ((off & 31) + 4 * B > 32) piece[c][(off >> 5) + 1] |= w >> (32 - (off & 31));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y = acc[c][t][e];
            const float ay = __builtin_fabsf(y);
            uint32_t m = HALF;
            float mag = pcen[0];
            // a linear scan yields the cell's centroid with one select per
            // threshold (and fewer live registers than a search's muxes)
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              const bool above = thr[c][j] < ay;
              m += above ? 1u : 0u;
              mag = above ? pcen[j + 1] : mag;
              // keep the select chain (the compiler would otherwise index
              // the table with the count, through scratch memory)
              asm volatile("" : "+v"(mag));
            }
            // #{b < u} = HALF + m for y > 0 and HALF - 1 - m = (HALF + m) ^ (2 HALF - 1)
            // for y < 0; all ones where the sign bit is set (y = +0 lies on the
            // middle boundary 0, a tie either way; a zero row is set below)
            const uint32_t neg = (uint32_t)(__float_as_int(y) >> 31);
            const uint32_t idx = m ^ (neg & (uint32_t)(2 * HALF - 1));
            piece[c][t >> 1] |= idx << (B * (4 * (t & 1) + e));
            const float yh = __uint_as_float(__float_as_uint(mag) ^ (neg & 0x80000000u));
            const float rho = __builtin_fmaf(-yh, sc[c], y);
            acc[c][t][e] = rho;
            gg[c] = __builtin_fmaf(rho, rho, gg[c]);
          }
        }
      }
    };
    if constexpr (QJL) {
      // (the QJL stage needs the registers: product first, then coding)
      dn_gemm<D, NC, 1>(acc, lds, bx, bx, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t) code_tile(t);
    } else {
      dn_bf16x8 cur[NK], nxt[NK];
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) cur[kc] = dn_frag(lds, kc, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 1 < NT) {
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) nxt[kc] = dn_frag(lds, (t + 1) * NK + kc, lane);
        }
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[kc], dn_bits(bx[c][kc]), acc[c][t], 0, 0, 0);
        }
        if (t > 0) code_tile(t - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) cur[kc] = nxt[kc];
      }
      code_tile(NT - 1);
    }
    if constexpr (QJL) {
      if (more) load_tile(next, bx, po, act);
    }

    float gam[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (nrm[c] == 0.f) {
#pragma unroll
        for (int q = 0; q < NK; ++q) piece[c][q] = QJL ? zpiece : zrun[q];
      }
      if (ac[c]) {
        uint8_t* irow = a.idx + pc[c] * (D * B / 8);
        if constexpr (QJL) {
#pragma unroll
          for (int q = 0; q < NK; ++q) store_lane_bits<B>(irow, 4 * q + g, piece[c][q]);
        } else {
          dn_store_run<RB>(irow + RB * g, piece[c]);
        }
        if (g == 0) a.norm[pc[c]] = nrm[c];
      }
      if constexpr (QJL) gam[c] = __builtin_sqrtf(dn_sum_groups(gg[c]));
    }

    if constexpr (QJL) {
      dn_u32x4 hi[NC][NK], lo[NC][NK];
      dn_split<D, NC>(acc, hi, lo);
      dn_f32x4 sp[NC][NT];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t) sp[c][t] = dn_f32x4{0.f, 0.f, 0.f, 0.f};
      dn_gemm<D, NC, 2>(sp, lds + C::MAT, hi, lo, lane);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // sign bits of coordinates 32 q + 8 g + [0, 8): byte 4 q + g of the row
        uint32_t qb[NK];
#pragma unroll
        for (int q = 0; q < NK; ++q) qb[q] = 0u;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) qb[t >> 1] |= (sp[c][t][e] >= 0.f ? 1u : 0u) << (4 * (t & 1) + e);
        if (ac[c]) {
          uint8_t* qrow = a.qjl + pc[c] * (D / 8);
#pragma unroll
          for (int q = 0; q < NK; ++q) store_lane_bits<1>(qrow, 4 * q + g, qb[q]);
          if (g == 0) a.gamma[pc[c]] = gam[c];
        }
      }
    }
    if (!more) break;
    tile = next;
    if constexpr (!QJL) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        po[c] = pn[c];
        act[c] = an[c];
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) bx[c][kc] = bn[c][kc];
      }
    }
  }
}

// A lane's 8-code piece of a packed row: B bytes at byte offset B * sub,
// read as the aligned dword(s) that hold it (the second one clamped into the
// row; rows are multiples of 8 bytes) and combined only when used, so that
// prefetched pieces stay in flight until then.
template <int B>
__device__ __forceinline__ void dn_piece_load(const uint8_t* row, int sub, int row_bytes, uint32_t& w0, uint32_t& w1) {
  const int a = (B * sub) & ~3;
  w0 = *reinterpret_cast<const uint32_t*>(row + a);
  if constexpr (B == 3) {
    const int a1 = (a + 4 < row_bytes - 4) ? a + 4 : row_bytes - 4;
    w1 = *reinterpret_cast<const uint32_t*>(row + a1);
  } else {
    w1 = 0u;
  }
}
template <int B>
__device__ __forceinline__ uint32_t dn_piece_bits(uint32_t w0, uint32_t w1, int sub) {
  const uint32_t sh = (uint32_t)((B * sub) & 3) * 8u;
  if constexpr (B == 3) return __builtin_amdgcn_alignbit(w1, w0, sh);
  else return w0 >> sh;
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
  using C = DenseCfg<D, kDeqNC<D>>;
  constexpr int NT = C::NT, NK = C::NK, NC = C::NC;
  // P^T for the final product (outputs in kRows order), S^T for the QJL term
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::MAT * (QJL ? 2 : 1)];
  // MSE: centroid as its bf16 hi (low half) and lo (high half); QJL: float32
  __shared__ uint32_t lut[1 << B];
  dn_load_matrix<D, true, kRows>(lds, a.rot);
  if constexpr (QJL) dn_load_matrix<D, true, kInterleaved>(lds + C::MAT, a.proj);
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

  // Raw plane words of a tile, as loaded: (fw0, fw1)[c][kc] hold the 8 code
  // fields of local elements 8 kc .. 8 kc + 7 of row 16 c + n, i.e. of
  // coordinates 32 kc + 8 g + [0, 8) (stream bytes B (4 kc + g) ..); qw the
  // word holding their 8 sign bits (byte 4 kc + g of the QJL row).
  uint32_t fw0[NC][NK], fw1[NC][NK], qw[NC][NK];
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
      const int64_t po = check_row(row_index(a.plane_map, s, t, h), a.plane_ext, kChkDenseIn);
      // an output row outside the extent is marked -1 and not written (checked build)
      if (kChecked && act && !check_ok(xo[c] < a.x_ext, kChkDenseOut)) xo[c] = -1;
      if (act) {
        const uint8_t* irow = a.idx + po * (D * B / 8);
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) dn_piece_load<B>(irow, 4 * kc + g, D * B / 8, fw0[c][kc], fw1[c][kc]);
        sc[c] = a.norm[po];
        if constexpr (QJL) {
          const uint8_t* qrow = a.qjl + po * (D / 8);
          uint32_t unused;
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) dn_piece_load<1>(qrow, 4 * kc + g, D / 8, qw[c][kc], unused);
          cg[c] = a.gamma[po];
        }
      } else {
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) fw0[c][kc] = fw1[c][kc] = 0u;
        sc[c] = 0.f;
        if constexpr (QJL) {
#pragma unroll
          for (int kc = 0; kc < NK; ++kc) qw[c][kc] = 0u;
          cg[c] = 0.f;
        }
      }
    }
  };
  uint32_t fb[NC][NK], qb[NC][NK];
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
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
        fb[c][kc] = dn_piece_bits<B>(fw0[c][kc], fw1[c][kc], 4 * kc + g);
        if constexpr (QJL) qb[c][kc] = dn_piece_bits<1>(qw[c][kc], 0u, 4 * kc + g);
      }
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
      dn_gemm<D, NC, 1>(sq, lds + C::MAT, bq, bq, lane);
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float cv = __uint_as_float(lut[field(c, 4 * t + e)]);
            sq[c][t][e] = __builtin_fmaf(cg[c], sq[c][t][e], cv * scale[c]);
          }
      dn_split<D, NC>(sq, hi, lo);
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
    dn_gemm<D, NC, 2, true>(acc, lds, hi, lo, lane);

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
        if (kChecked && row_off < 0) continue;
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

// One round of resident blocks: the occupancy the compiled kernel allows (its
// registers and LDS), times the compute units; every block copies its
// matrices once and then loops over row tiles.
template <int D, int B, bool QJL, bool DEQ>
unsigned dense_grid(void (*kernel)(DenseArgs), uint32_t rows) {
  constexpr int rows_per_wave = DenseCfg<D, DEQ ? kDeqNC<D> : kQuantNC<D, B, QJL>>::RW;
  static int per_cu = 0, cus = 0;  // one pair per kernel
  if (per_cu == 0) {
    int occ = 0, dev = 0, n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess || occ < 1) occ = 1;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 256;
    cus = n;
    per_cu = occ;
  }
  const uint32_t tiles = (rows + rows_per_wave - 1) / rows_per_wave;
  const unsigned want = (tiles + 3) / 4;
  const unsigned cap = (unsigned)(cus * per_cu);
  return want < cap ? want : cap;
}

template <int D, int B>
hipError_t dense_quant_db(const DenseArgs& a, bool qjl, hipStream_t st) {
  if constexpr (D <= 128) {
    if (qjl) {
      const dim3 grid(dense_grid<D, B, true, false>(dense_quantize_kernel<D, B, true>, a.rows));
      dense_quantize_kernel<D, B, true><<<grid, 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  const dim3 grid(dense_grid<D, B, false, false>(dense_quantize_kernel<D, B, false>, a.rows));
  dense_quantize_kernel<D, B, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int B>
hipError_t dense_dequant_db(const DenseArgs& a, bool qjl, hipStream_t st) {
  if constexpr (D <= 128) {
    if (qjl) {
      const dim3 grid(dense_grid<D, B, true, true>(dense_dequantize_kernel<D, B, true>, a.rows));
      dense_dequantize_kernel<D, B, true><<<grid, 256, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  const dim3 grid(dense_grid<D, B, false, true>(dense_dequantize_kernel<D, B, false>, a.rows));
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

uint32_t check_read_clear_dense() { return check_read_clear_file(); }

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
