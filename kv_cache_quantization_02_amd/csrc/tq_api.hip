// tq_api.hip -- the C ABI declared in include/tq.h: host-side validation,
// row-index set-up and kernel dispatch.  Nothing here allocates.
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/tq.h"
#include "tq_codebooks.h"
#include "tq_launch.h"

namespace {

const uint32_t kCen1[] = {TQ_CENTROIDS_1BIT}, kBnd1[] = {TQ_BOUNDARIES_1BIT};
const uint32_t kCen2[] = {TQ_CENTROIDS_2BIT}, kBnd2[] = {TQ_BOUNDARIES_2BIT};
const uint32_t kCen3[] = {TQ_CENTROIDS_3BIT}, kBnd3[] = {TQ_BOUNDARIES_3BIT};
const uint32_t kCen4[] = {TQ_CENTROIDS_4BIT}, kBnd4[] = {TQ_BOUNDARIES_4BIT};
const uint32_t kCen5[] = {TQ_CENTROIDS_5BIT}, kBnd5[] = {TQ_BOUNDARIES_5BIT};
const uint32_t kCen8[] = {TQ_CENTROIDS_8BIT}, kBnd8[] = {TQ_BOUNDARIES_8BIT};

// Cap on the blocks of each half (keys / values) of a codec launch: 8192
// four-wave blocks per half keep every one of the 256 CUs loaded while the
// hardware balances the remainder dynamically.
#ifndef TQ_MAX_CODEC_BLOCKS
#define TQ_MAX_CODEC_BLOCKS 8192
#endif
constexpr int kMaxCodecBlocks = TQ_MAX_CODEC_BLOCKS;

// Cap on the blocks of a cache re-lay (16 KB each); a grid-stride loop covers
// the rest.  32768 was 2% faster than 8192 on the 1.7 GB growth of the decode
// cache, and as fast as 65536.
#ifndef TQ_MAX_GROW_BLOCKS
#define TQ_MAX_GROW_BLOCKS 32768
#endif
constexpr int kMaxGrowBlocks = TQ_MAX_GROW_BLOCKS;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int32_t check_scheme(const tq_scheme* s) {
  if (!s) return TQ_E_NULL;
  const int d = s->head_dim;
  if (d != 64 && d != 128 && d != 256 && d != 512) return TQ_E_HEAD_DIM;
  const int k = s->k_bits, v = s->v_bits;
  if (k != 2 && k != 4 && k != 5 && k != 8) return TQ_E_BITS;
  if (v != 2 && v != 3 && v != 4 && v != 5 && v != 8) return TQ_E_BITS;
  return TQ_OK;
}

tq::FastDiv make_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
  const uint64_t m = (uint64_t)((num + d - 1) / d);
  return tq::FastDiv{(uint32_t)m, 31 + l, d};
}

// Validates a row block; on success fills the row count and index split.
int32_t check_rows(const tq_rows* r, uint32_t* rows, tq::RowSplit* split) {
  if (!r) return TQ_E_NULL;
  if (r->n_seq < 0 || r->n_tok < 0 || r->n_head < 0) return TQ_E_SHAPE;
  if (r->seq_stride < 0 || r->tok_stride < 0 || r->head_stride < 0) return TQ_E_SHAPE;
  // each count below 2^31 first, so that the product (at most 93 bits) is exact
  const int64_t lim = (int64_t)1 << 31;
  if (r->n_seq >= lim || r->n_tok >= lim || r->n_head >= lim) return TQ_E_SHAPE;
  const unsigned __int128 n = (unsigned __int128)r->n_seq * r->n_tok * r->n_head;
  if (n >= ((unsigned __int128)1 << 31)) return TQ_E_SHAPE;
  *rows = (uint32_t)n;
  if (n) {
    split->div_head = make_div((uint32_t)r->n_head);
    split->div_tok = make_div((uint32_t)r->n_tok);
  }
  return TQ_OK;
}

bool same_counts(const tq_rows* a, const tq_rows* b) {
  return a->n_seq == b->n_seq && a->n_tok == b->n_tok && a->n_head == b->n_head;
}

tq::RowMap map_of(const tq_rows* r) { return tq::RowMap{r->seq_stride, r->tok_stride, r->head_stride}; }

// The checked build's positive control: rows (bytes, for growth) taken off
// every extent handed to the kernels (tq_check_set_margin).
std::atomic<int64_t> g_check_margin{0};

int64_t shrink(int64_t e) {
  if (!tq::kChecked) return e;
  const int64_t m = g_check_margin.load();
  return e > m ? e - m : 0;
}

// Rows a map addresses, as handed to the kernels' bounds tests.
int64_t ext_of(int64_t n_seq, int64_t n_tok, int64_t n_head, int64_t ss, int64_t ts, int64_t hs) {
  return shrink(tq::map_extent(n_seq, n_tok, n_head, ss, ts, hs));
}
int64_t ext_of(const tq_rows* r) {
  return ext_of(r->n_seq, r->n_tok, r->n_head, r->seq_stride, r->tok_stride, r->head_stride);
}

int32_t check_planes(const tq_planes* p) {
  if (!p) return TQ_E_NULL;
  if (!p->k_q || !p->k_scale || !p->k_zero || !p->v_q || !p->v_scale) return TQ_E_NULL;
  // packed planes are read and written in naturally aligned words of up to
  // 8 bytes, the fp16 planes in 2-byte words (every plane row length is a
  // multiple of these, so any row offset keeps the alignment)
  if (!aligned(p->k_q, 8) || !aligned(p->v_q, 8) || !aligned(p->k_scale, 2) || !aligned(p->k_zero, 2) ||
      !aligned(p->v_scale, 2))
    return TQ_E_ALIGN;
  return TQ_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_E_HIP; }

}  // namespace

extern "C" {

int32_t tq_check_scheme(const tq_scheme* scheme) { return check_scheme(scheme); }

int64_t tq_plane_row_bytes(const tq_scheme* s, int32_t plane) {
  const int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  const int64_t d = s->head_dim, g = d / 32;
  switch (plane) {
    case TQ_PLANE_K_Q: return d * s->k_bits / 8;
    case TQ_PLANE_K_SCALE:
    case TQ_PLANE_K_ZERO:
    case TQ_PLANE_V_SCALE: return 2 * g;
    case TQ_PLANE_V_Q: return d * s->v_bits / 8;
    default: return TQ_E_PLANE;
  }
}

int64_t tq_row_bytes(const tq_scheme* s) {
  const int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  int64_t total = 0;
  for (int p = 0; p < 5; ++p) total += tq_plane_row_bytes(s, p);
  return total;
}

int32_t tq_codebook(int32_t bits, float* centroids, float* boundaries) {
  const uint32_t *c = nullptr, *b = nullptr;
  switch (bits) {
    case 1: c = kCen1; b = kBnd1; break;
    case 2: c = kCen2; b = kBnd2; break;
    case 3: c = kCen3; b = kBnd3; break;
    case 4: c = kCen4; b = kBnd4; break;
    case 5: c = kCen5; b = kBnd5; break;
    case 8: c = kCen8; b = kBnd8; break;
    default: return TQ_E_BITS;
  }
  if (!centroids || !boundaries) return TQ_E_NULL;
  memcpy(centroids, c, sizeof(float) << bits);
  memcpy(boundaries, b, sizeof(float) * ((1u << bits) - 1));
  return TQ_OK;
}

int32_t tq_quantize_kv(const tq_scheme* s, const uint16_t* k_bf16, const uint16_t* v_bf16,
                       const tq_rows* in_rows, const int8_t* signs, const tq_planes* out,
                       const tq_rows* out_rows, void* stream) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if (!k_bf16 || !v_bf16 || !signs) return TQ_E_NULL;
  if ((st = check_planes(out)) != TQ_OK) return st;
  if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(signs)) return TQ_E_ALIGN;
  tq::QuantArgs a{};
  tq::RowSplit split{};
  uint32_t rows = 0, rows_out = 0;
  if ((st = check_rows(in_rows, &rows, &split)) != TQ_OK) return st;
  if ((st = check_rows(out_rows, &rows_out, &split)) != TQ_OK) return st;
  if (!same_counts(in_rows, out_rows)) return TQ_E_SHAPE;
  if (rows == 0) return TQ_OK;
  a.k = k_bf16;
  a.v = v_bf16;
  a.signs = signs;
  a.k_q = (uint8_t*)out->k_q;
  a.k_scale = (uint16_t*)out->k_scale;
  a.k_zero = (uint16_t*)out->k_zero;
  a.v_q = (uint8_t*)out->v_q;
  a.v_scale = (uint16_t*)out->v_scale;
  a.rows = rows;
  a.split = split;
  a.in = map_of(in_rows);
  a.out = map_of(out_rows);
  a.in_ext = ext_of(in_rows);
  a.out_ext = ext_of(out_rows);
  return hip_status(tq::launch_quantize(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream,
                                        kMaxCodecBlocks));
}

int32_t tq_dequantize_kv(const tq_scheme* s, const tq_planes* in, const tq_rows* in_rows,
                         const int8_t* signs, uint16_t* k_bf16, uint16_t* v_bf16,
                         const tq_rows* out_rows, void* stream) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if ((st = check_planes(in)) != TQ_OK) return st;
  if (!k_bf16 && !v_bf16) return TQ_E_NULL;
  if (v_bf16 && !signs) return TQ_E_NULL;
  if ((k_bf16 && !aligned16(k_bf16)) || (v_bf16 && !aligned16(v_bf16)) || (signs && !aligned16(signs)))
    return TQ_E_ALIGN;
  tq::DequantArgs a{};
  tq::RowSplit split{};
  uint32_t rows = 0, rows_out = 0;
  if ((st = check_rows(in_rows, &rows, &split)) != TQ_OK) return st;
  if ((st = check_rows(out_rows, &rows_out, &split)) != TQ_OK) return st;
  if (!same_counts(in_rows, out_rows)) return TQ_E_SHAPE;
  if (rows == 0) return TQ_OK;
  a.k_q = (const uint8_t*)in->k_q;
  a.k_scale = (const uint16_t*)in->k_scale;
  a.k_zero = (const uint16_t*)in->k_zero;
  a.v_q = (const uint8_t*)in->v_q;
  a.v_scale = (const uint16_t*)in->v_scale;
  a.signs = signs;
  a.k = k_bf16;
  a.v = v_bf16;
  a.rows = rows;
  a.split = split;
  a.in = map_of(in_rows);
  a.out = map_of(out_rows);
  a.in_ext = ext_of(in_rows);
  a.out_ext = ext_of(out_rows);
  return hip_status(tq::launch_dequantize(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream,
                                          kMaxCodecBlocks));
}

int32_t tq_append_kv(const tq_scheme* s, const uint16_t* k_bf16, const uint16_t* v_bf16, int32_t batch,
                     int32_t n_new, int32_t n_kv_heads, const int8_t* signs, const tq_planes* cache,
                     int64_t seq_stride_rows, int64_t head_stride_rows, const int32_t* positions,
                     int32_t capacity, void* stream) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if (!k_bf16 || !v_bf16 || !signs || !positions) return TQ_E_NULL;
  if ((st = check_planes(cache)) != TQ_OK) return st;
  if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(signs)) return TQ_E_ALIGN;
  if (batch < 0 || n_new < 0 || n_kv_heads < 0 || capacity < 0 || seq_stride_rows < 0 || head_stride_rows < 0)
    return TQ_E_SHAPE;
  // new tokens arrive as a contiguous [batch, n_new, n_kv_heads, d] block
  const tq_rows in{batch, n_new, n_kv_heads, (int64_t)n_new * n_kv_heads, n_kv_heads, 1};
  const tq_rows out{batch, n_new, n_kv_heads, seq_stride_rows, 1, head_stride_rows};
  tq::QuantArgs a{};
  tq::RowSplit split{};
  uint32_t rows = 0;
  if ((st = check_rows(&in, &rows, &split)) != TQ_OK) return st;
  if (rows == 0 || capacity == 0) return TQ_OK;
  a.k = k_bf16;
  a.v = v_bf16;
  a.signs = signs;
  a.k_q = (uint8_t*)cache->k_q;
  a.k_scale = (uint16_t*)cache->k_scale;
  a.k_zero = (uint16_t*)cache->k_zero;
  a.v_q = (uint8_t*)cache->v_q;
  a.v_scale = (uint16_t*)cache->v_scale;
  a.rows = rows;
  a.split = split;
  a.in = map_of(&in);
  a.out = map_of(&out);
  a.out_pos = positions;
  a.out_cap = capacity;
  a.in_ext = ext_of(&in);
  // tokens land at positions[b] + j within [0, capacity)
  a.out_ext = ext_of(batch, capacity, n_kv_heads, seq_stride_rows, 1, head_stride_rows);
  return hip_status(tq::launch_quantize(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream,
                                        kMaxCodecBlocks));
}

int32_t tq_fetch_kv(const tq_scheme* s, const tq_planes* cache, int32_t batch, int32_t n_kv_heads,
                    int64_t seq_stride_rows, int64_t head_stride_rows, int32_t capacity, const int32_t* lens,
                    int32_t window, const int8_t* signs, int32_t values_rotated, uint16_t* k_bf16,
                    uint16_t* v_bf16, void* stream) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if ((st = check_planes(cache)) != TQ_OK) return st;
  if (!lens || (!k_bf16 && !v_bf16)) return TQ_E_NULL;
  if (v_bf16 && !values_rotated && !signs) return TQ_E_NULL;
  if ((k_bf16 && !aligned16(k_bf16)) || (v_bf16 && !aligned16(v_bf16)) || (signs && !aligned16(signs)))
    return TQ_E_ALIGN;
  if (batch < 0 || n_kv_heads < 0 || window < 0 || capacity < 0 || seq_stride_rows < 0 || head_stride_rows < 0)
    return TQ_E_SHAPE;
  // rows (b, g, t) of the cache window -> a contiguous [batch, n_kv_heads, window, d]
  // output; the token is the fastest index, so a wave's rows are consecutive
  // tokens of one kv head on both sides
  const tq_rows in{batch, n_kv_heads, window, seq_stride_rows, head_stride_rows, 1};
  const tq_rows out{batch, n_kv_heads, window, (int64_t)n_kv_heads * window, window, 1};
  tq::DequantArgs a{};
  tq::RowSplit split{};
  uint32_t rows = 0;
  if ((st = check_rows(&in, &rows, &split)) != TQ_OK) return st;
  if (rows == 0) return TQ_OK;
  a.k_q = (const uint8_t*)cache->k_q;
  a.k_scale = (const uint16_t*)cache->k_scale;
  a.k_zero = (const uint16_t*)cache->k_zero;
  a.v_q = (const uint8_t*)cache->v_q;
  a.v_scale = (const uint16_t*)cache->v_scale;
  a.signs = signs;
  a.k = k_bf16;
  a.v = v_bf16;
  a.rows = rows;
  a.split = split;
  a.in = map_of(&in);
  a.out = map_of(&out);
  a.in_len = lens;
  a.in_cap = capacity;
  // tokens read lie below min(lens[b], capacity, window)
  a.in_ext = ext_of(batch, n_kv_heads, window < capacity ? window : capacity, seq_stride_rows, head_stride_rows, 1);
  a.out_ext = ext_of(&out);
  a.rotated = values_rotated ? 1 : 0;
  return hip_status(tq::launch_dequantize(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream,
                                          kMaxCodecBlocks));
}

int64_t tq_grown_capacity(int64_t tokens) {
  if (tokens < 0) return TQ_E_SHAPE;
  if (tokens > (int64_t)INT32_MAX - (TQ_CAPACITY_STEP - 1)) return TQ_E_SHAPE;
  return (tokens + TQ_CAPACITY_STEP - 1) / TQ_CAPACITY_STEP * TQ_CAPACITY_STEP;
}

}  // extern "C"

namespace {

// The (b, g) segments of `cap` consecutive rows at b*ss + g*hs are nested:
// along the axis of smaller stride they sit one after another, and the
// other axis steps past that whole run.
bool segments_apart(int64_t B, int64_t H, int64_t ss, int64_t hs, int64_t cap) {
  if (cap == 0 || B == 0 || H == 0) return true;
  if (B == 1 && H == 1) return true;
  if (B == 1) return hs >= cap;
  if (H == 1) return ss >= cap;
  int64_t n1 = H, s1 = hs, s2 = ss;
  if (ss < hs) {
    n1 = B;
    s1 = ss;
    s2 = hs;
  }
  if (s1 < cap) return false;
  const __int128 run = (__int128)(n1 - 1) * s1 + cap;
  return (__int128)s2 >= run;
}

// Byte range [lo, hi) of one plane over B x H segments of `rows` rows.
struct Span {
  uintptr_t lo, hi;
};

bool plane_span(const void* base, int64_t rb, int64_t B, int64_t H, int64_t ss, int64_t hs, int64_t rows,
                Span* out) {
  const __int128 last = (__int128)(B - 1) * ss + (__int128)(H - 1) * hs + rows;
  const __int128 bytes = last * rb;
  if (bytes > ((__int128)1 << 62)) return false;
  out->lo = (uintptr_t)base;
  out->hi = (uintptr_t)base + (uintptr_t)bytes;
  return true;
}

bool spans_meet(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

}  // namespace

extern "C" {

int32_t tq_grow_kv(const tq_scheme* s, int32_t batch, int32_t n_kv_heads, const tq_planes* src,
                   int64_t src_seq_stride_rows, int64_t src_head_stride_rows, int32_t src_capacity,
                   const tq_planes* dst, int64_t dst_seq_stride_rows, int64_t dst_head_stride_rows,
                   int32_t dst_capacity, void* stream) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if (!src || !dst) return TQ_E_NULL;
  if ((st = check_planes(src)) != TQ_OK) return st;
  if ((st = check_planes(dst)) != TQ_OK) return st;
  if (batch < 0 || n_kv_heads < 0 || src_capacity < 0 || dst_capacity < 0 || src_seq_stride_rows < 0 ||
      src_head_stride_rows < 0 || dst_seq_stride_rows < 0 || dst_head_stride_rows < 0)
    return TQ_E_SHAPE;
  if (!segments_apart(batch, n_kv_heads, dst_seq_stride_rows, dst_head_stride_rows, dst_capacity))
    return TQ_E_SHAPE;
  if (batch == 0 || n_kv_heads == 0 || dst_capacity == 0) return TQ_OK;
  const int64_t keep = src_capacity < dst_capacity ? src_capacity : dst_capacity;
  // an axis of extent 1 never steps, so its stride plays no part (and is not
  // multiplied out below: the byte spans bound every product that is)
  const int64_t sss = batch > 1 ? src_seq_stride_rows : 0, shs = n_kv_heads > 1 ? src_head_stride_rows : 0;
  const int64_t dss = batch > 1 ? dst_seq_stride_rows : 0, dhs = n_kv_heads > 1 ? dst_head_stride_rows : 0;
  const void* sp[5] = {src->k_q, src->k_scale, src->k_zero, src->v_q, src->v_scale};
  void* dp[5] = {dst->k_q, dst->k_scale, dst->k_zero, dst->v_q, dst->v_scale};
  Span rd[5], wr[5];
  tq::GrowArgs a{};
  uint64_t total = 0;
  for (int p = 0; p < 5; ++p) {
    const int64_t rb = tq_plane_row_bytes(s, p);
    if (!plane_span(sp[p], rb, batch, n_kv_heads, sss, shs, keep, &rd[p]) ||
        !plane_span(dp[p], rb, batch, n_kv_heads, dss, dhs, dst_capacity, &wr[p]))
      return TQ_E_SHAPE;
    tq::GrowPlane& g = a.plane[p];
    g.src = (const uint8_t*)sp[p];
    g.dst = (uint8_t*)dp[p];
    g.src_seq = sss * rb;
    g.src_head = shs * rb;
    g.dst_seq = dss * rb;
    g.dst_head = dhs * rb;
    g.copy = keep * rb;
    g.dst_bytes = (int64_t)dst_capacity * rb;
    const uint64_t chunks = (uint64_t)((g.dst_bytes + tq::kGrowChunkBytes - 1) / tq::kGrowChunkBytes);
    g.chunks = (uint32_t)chunks;
    g.vec16 = aligned16(sp[p]) && aligned16(dp[p]) && g.src_seq % 16 == 0 && g.src_head % 16 == 0 &&
              g.dst_seq % 16 == 0 && g.dst_head % 16 == 0;
    g.src_ext = shrink((int64_t)(rd[p].hi - rd[p].lo));
    g.dst_ext = shrink((int64_t)(wr[p].hi - wr[p].lo));
    a.first[p] = (uint32_t)total;
    total += (uint64_t)batch * (uint64_t)n_kv_heads * chunks;
    if (total > UINT32_MAX) return TQ_E_SHAPE;
  }
  for (int p = 0; p < 5; ++p)
    for (int q = 0; q < 5; ++q)
      if (spans_meet(wr[p], rd[q]) || (q != p && spans_meet(wr[p], wr[q]))) return TQ_E_OVERLAP;
  a.total = (uint32_t)total;
  a.n_kv_heads = (uint32_t)n_kv_heads;
  return hip_status(tq::launch_grow(a, (hipStream_t)stream, kMaxGrowBlocks));
}

int32_t tq_unrotate_rows(int32_t head_dim, const uint16_t* in_bf16, const tq_rows* in_rows, const int8_t* signs,
                         uint16_t* out_bf16, const tq_rows* out_rows, void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512) return TQ_E_HEAD_DIM;
  if (!in_bf16 || !signs || !out_bf16) return TQ_E_NULL;
  if (!aligned16(in_bf16) || !aligned16(signs) || !aligned16(out_bf16)) return TQ_E_ALIGN;
  int32_t st;
  tq::UnrotateArgs a{};
  tq::RowSplit split{};
  uint32_t rows = 0, rows_out = 0;
  if ((st = check_rows(in_rows, &rows, &split)) != TQ_OK) return st;
  if ((st = check_rows(out_rows, &rows_out, &split)) != TQ_OK) return st;
  if (!same_counts(in_rows, out_rows)) return TQ_E_SHAPE;
  if (rows == 0) return TQ_OK;
  a.in = in_bf16;
  a.signs = signs;
  a.out = out_bf16;
  a.rows = rows;
  a.split = split;
  a.in_map = map_of(in_rows);
  a.out_map = map_of(out_rows);
  a.in_ext = ext_of(in_rows);
  a.out_ext = ext_of(out_rows);
  return hip_status(tq::launch_unrotate(a, head_dim, (hipStream_t)stream, kMaxCodecBlocks));
}

size_t tq_attn_quant_workspace_bytes(const tq_scheme* s, int32_t batch, int32_t n_queries, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t max_ctx) {
  if (check_scheme(s) != TQ_OK) return 0;
  if (batch < 0 || n_queries < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || max_ctx < 1)
    return 0;
  if ((__int128)batch * n_queries * n_q_heads >= ((__int128)1 << 30)) return 0;
  if (batch == 0) return 0;  // nothing runs
  int splits = 0, tps = 0;
  tq::decode_attn_geometry(s->head_dim, s->k_bits, s->v_bits, batch, n_queries, n_q_heads, n_kv_heads, max_ctx,
                           &splits, &tps);
  return tq::decode_attn_part_bytes(s->head_dim, batch, n_queries, n_q_heads, splits);
}

size_t tq_decode_attn_workspace_bytes(const tq_scheme* s, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t max_ctx) {
  return tq_attn_quant_workspace_bytes(s, batch, 1, n_q_heads, n_kv_heads, max_ctx);
}

}  // extern "C"

namespace {

// Validates an attention call and fills every argument but the partials'
// buffer (a->part); *need is that buffer's size in bytes.  TQ_OK with
// a->batch == 0 means there is nothing to launch.
int32_t attn_prepare(const tq_scheme* s, const uint16_t* q_bf16, int32_t batch, int32_t n_queries,
                     int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache, int64_t seq_stride_rows,
                     int64_t head_stride_rows, const int32_t* ctx_lens, int32_t max_ctx, float softmax_scale,
                     const int8_t* signs, uint16_t* out_bf16, tq::AttnArgs* a, size_t* need) {
  int32_t st = check_scheme(s);
  if (st != TQ_OK) return st;
  if (batch < 0 || n_queries < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || max_ctx < 1 ||
      seq_stride_rows < 0 || head_stride_rows < 0)
    return TQ_E_SHAPE;
  // below 2^30 query rows, so that no row or tile count in the launch arithmetic
  // (int32 on host and device) comes near overflow
  if ((__int128)batch * n_queries * n_q_heads >= ((__int128)1 << 30)) return TQ_E_SHAPE;
  *a = tq::AttnArgs{};
  *need = 0;
  if (batch == 0) return TQ_OK;
  if (!q_bf16 || !ctx_lens || !signs || !out_bf16) return TQ_E_NULL;
  if ((st = check_planes(cache)) != TQ_OK) return st;
  if (!aligned16(q_bf16) || !aligned16(signs) || !aligned16(out_bf16)) return TQ_E_ALIGN;
  int splits = 0, tps = 0;
  tq::decode_attn_geometry(s->head_dim, s->k_bits, s->v_bits, batch, n_queries, n_q_heads, n_kv_heads, max_ctx,
                           &splits, &tps);
  *need = tq::decode_attn_part_bytes(s->head_dim, batch, n_queries, n_q_heads, splits);
  a->q = q_bf16;
  a->k_q = (const uint8_t*)cache->k_q;
  a->k_scale = (const uint16_t*)cache->k_scale;
  a->k_zero = (const uint16_t*)cache->k_zero;
  a->v_q = (const uint8_t*)cache->v_q;
  a->v_scale = (const uint16_t*)cache->v_scale;
  a->signs = signs;
  a->ctx_lens = ctx_lens;
  a->out = out_bf16;
  a->seq_stride = seq_stride_rows;
  a->head_stride = head_stride_rows;
  a->batch = batch;
  a->n_q_heads = n_q_heads;
  a->n_kv_heads = n_kv_heads;
  a->max_ctx = max_ctx;
  a->splits = splits;
  a->tokens_per_split = tps;
  a->softmax_scale = softmax_scale;
  a->n_queries = n_queries;
  a->cache_ext = ext_of(batch, n_kv_heads, max_ctx, seq_stride_rows, head_stride_rows, 1);
  return TQ_OK;
}

// Split partials of tq_attn_quant_noalloc.  Each device holds its own copy
// of this array from the library's load to the end of the process; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// device (the array's name on the host is a stand-in, not a device address).
constexpr size_t kScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call made
// with that device current and kept.
int32_t device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

int32_t tq_attn_quant(const tq_scheme* s, const uint16_t* q_bf16, int32_t batch, int32_t n_queries,
                      int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache, int64_t seq_stride_rows,
                      int64_t head_stride_rows, const int32_t* ctx_lens, int32_t max_ctx, float softmax_scale,
                      const int8_t* signs, uint16_t* out_bf16, void* workspace, size_t workspace_bytes,
                      void* stream) {
  tq::AttnArgs a;
  size_t need = 0;
  const int32_t st = attn_prepare(s, q_bf16, batch, n_queries, n_q_heads, n_kv_heads, cache, seq_stride_rows,
                                  head_stride_rows, ctx_lens, max_ctx, softmax_scale, signs, out_bf16, &a, &need);
  if (st != TQ_OK || a.batch == 0) return st;
  if (!workspace || workspace_bytes < need) return TQ_E_WORKSPACE;
  if (!aligned16(workspace)) return TQ_E_ALIGN;
  a.part = (float*)workspace;
  return hip_status(tq::launch_decode_attn(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream));
}

int32_t tq_attn_quant_noalloc(const tq_scheme* s, const uint16_t* q_bf16, int32_t batch, int32_t n_queries,
                              int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache,
                              int64_t seq_stride_rows, int64_t head_stride_rows, const int32_t* ctx_lens,
                              int32_t max_ctx, float softmax_scale, const int8_t* signs, uint16_t* out_bf16,
                              void* stream) {
  tq::AttnArgs a;
  size_t need = 0;
  int32_t st = attn_prepare(s, q_bf16, batch, n_queries, n_q_heads, n_kv_heads, cache, seq_stride_rows,
                            head_stride_rows, ctx_lens, max_ctx, softmax_scale, signs, out_bf16, &a, &need);
  if (st != TQ_OK || a.batch == 0) return st;
  if (need > kScratchBytes) return TQ_E_WORKSPACE;
  void* part = nullptr;
  if ((st = device_scratch(&part)) != TQ_OK) return st;
  // every partial the combine reads is written by the split kernel first,
  // so the scratch needs no clearing between calls
  a.part = (float*)part;
  return hip_status(tq::launch_decode_attn(a, s->head_dim, s->k_bits, s->v_bits, (hipStream_t)stream));
}

int32_t tq_decode_attn_quant(const tq_scheme* s, const uint16_t* q_bf16, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache,
                             int64_t seq_stride_rows, int64_t head_stride_rows,
                             const int32_t* ctx_lens, int32_t max_ctx, float softmax_scale,
                             const int8_t* signs, uint16_t* out_bf16, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return tq_attn_quant(s, q_bf16, batch, 1, n_q_heads, n_kv_heads, cache, seq_stride_rows, head_stride_rows,
                       ctx_lens, max_ctx, softmax_scale, signs, out_bf16, workspace, workspace_bytes, stream);
}

int32_t tq_dense_check_scheme(const tq_dense_scheme* s) {
  if (!s) return TQ_E_NULL;
  const int d = s->head_dim;
  if (d != 64 && d != 128 && d != 256) return TQ_E_HEAD_DIM;
  if (s->bits < 1 || s->bits > 4 || (s->qjl != 0 && s->qjl != 1)) return TQ_E_BITS;
  if (s->qjl && d > 128) return TQ_E_HEAD_DIM;
  return TQ_OK;
}

int64_t tq_dense_plane_row_bytes(const tq_dense_scheme* s, int32_t plane) {
  const int32_t st = tq_dense_check_scheme(s);
  if (st != TQ_OK) return st;
  switch (plane) {
    case TQ_DENSE_IDX: return (int64_t)s->head_dim * s->bits / 8;
    case TQ_DENSE_NORM: return 4;
    case TQ_DENSE_QJL: return s->qjl ? s->head_dim / 8 : 0;
    case TQ_DENSE_GAMMA: return s->qjl ? 4 : 0;
    default: return TQ_E_PLANE;
  }
}

}  // extern "C"

namespace {

int32_t check_dense_call(const tq_dense_scheme* s, const uint16_t* x, const uint16_t* rot, const uint16_t* proj,
                         const tq_dense_planes* p, const tq_rows* x_rows, const tq_rows* p_rows,
                         tq::DenseArgs* a) {
  int32_t st = tq_dense_check_scheme(s);
  if (st != TQ_OK) return st;
  if (!x || !rot || !p || (s->qjl && !proj)) return TQ_E_NULL;
  if (!p->idx || !p->norm || (s->qjl && (!p->qjl || !p->gamma))) return TQ_E_NULL;
  if (!aligned16(x) || !aligned16(rot) || (s->qjl && !aligned16(proj))) return TQ_E_ALIGN;
  if (!aligned(p->idx, 8) || !aligned(p->norm, 4) || (s->qjl && (!aligned(p->qjl, 8) || !aligned(p->gamma, 4))))
    return TQ_E_ALIGN;
  uint32_t rows = 0, rows_p = 0;
  tq::RowSplit split{};
  if ((st = check_rows(x_rows, &rows, &split)) != TQ_OK) return st;
  if ((st = check_rows(p_rows, &rows_p, &split)) != TQ_OK) return st;
  if (!same_counts(x_rows, p_rows)) return TQ_E_SHAPE;
  a->rot = rot;
  a->proj = s->qjl ? proj : nullptr;
  a->idx = (uint8_t*)p->idx;
  a->norm = p->norm;
  a->qjl = s->qjl ? (uint8_t*)p->qjl : nullptr;
  a->gamma = s->qjl ? p->gamma : nullptr;
  a->rows = rows;
  a->split = split;
  a->x_map = map_of(x_rows);
  a->plane_map = map_of(p_rows);
  a->x_ext = ext_of(x_rows);
  a->plane_ext = ext_of(p_rows);
  return TQ_OK;
}

}  // namespace

extern "C" {

int32_t tq_dense_quantize(const tq_dense_scheme* s, const uint16_t* x_bf16, const tq_rows* in_rows,
                          const uint16_t* rot_bf16, const uint16_t* proj_bf16, const tq_dense_planes* out,
                          const tq_rows* out_rows, void* stream) {
  tq::DenseArgs a{};
  const int32_t st = check_dense_call(s, x_bf16, rot_bf16, proj_bf16, out, in_rows, out_rows, &a);
  if (st != TQ_OK) return st;
  if (a.rows == 0) return TQ_OK;
  a.x = x_bf16;
  return hip_status(tq::launch_dense_quantize(a, s->head_dim, s->bits, s->qjl != 0, (hipStream_t)stream));
}

int32_t tq_dense_dequantize(const tq_dense_scheme* s, const tq_dense_planes* in, const tq_rows* in_rows,
                            const uint16_t* rot_bf16, const uint16_t* proj_bf16, uint16_t* x_bf16,
                            const tq_rows* out_rows, void* stream) {
  tq::DenseArgs a{};
  const int32_t st = check_dense_call(s, x_bf16, rot_bf16, proj_bf16, in, out_rows, in_rows, &a);
  if (st != TQ_OK) return st;
  if (a.rows == 0) return TQ_OK;
  a.x_out = x_bf16;
  return hip_status(tq::launch_dense_dequantize(a, s->head_dim, s->bits, s->qjl != 0, (hipStream_t)stream));
}

int64_t tq_check_flags(void) {
  if (!tq::kChecked) return -1;
  if (hipDeviceSynchronize() != hipSuccess) return TQ_E_HIP;
  const uint32_t v = tq::check_read_clear_codec() | tq::check_read_clear_attn() | tq::check_read_clear_cache() |
                     tq::check_read_clear_dense();
  return (int64_t)v;
}

int64_t tq_check_set_margin(int64_t margin) {
  if (!tq::kChecked) return -1;
  if (margin < 0) return TQ_E_SHAPE;
  g_check_margin.store(margin);
  return TQ_OK;
}

const char* tq_status_string(int32_t status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_E_HEAD_DIM: return "head_dim not served by this call (64, 128, 256 or 512; paper variant 64..256, QJL <= 128)";
    case TQ_E_BITS: return "k_bits must be 2, 4, 5 or 8 and v_bits 2, 3, 4, 5 or 8 (paper variant: bits 1..4, qjl 0 or 1)";
    case TQ_E_NULL: return "a required pointer is null";
    case TQ_E_SHAPE: return "invalid counts or strides";
    case TQ_E_ALIGN: return "a base pointer is not suitably aligned";
    case TQ_E_WORKSPACE: return "decode workspace missing or too small";
    case TQ_E_HIP: return "HIP launch error";
    case TQ_E_PLANE: return "plane index out of range";
    case TQ_E_OVERLAP: return "an output buffer overlaps an input or another output";
    default: return "unknown status";
  }
}

}  // extern "C"
