// Paged-attention decode for gfx950.
//
// What is computed (per row r at position p of sequence s, per query head h):
// out = softmax over t in [0, p] of (q_h . K_t / sqrt(d)) applied to V_t, with
// K_t, V_t fetched page by page through the sequence's block table and reduced
// by an online softmax in fp32 ("Building an LLM runtime from scratch on NVIDIA
// H100", section "Bug #1"; pages and block tables: "GPU inference engine
// engineering", section "Batching without running out of cache").
//
// Work unit: one 64-lane wavefront per (row, kv head[, position chunk]).  The
// G query heads sharing the kv head are the 16 columns of matrix-core tiles:
//   S^T[32 tokens x 16 heads] = K_page[32 x d] . Q^T[d x 16]   (MFMA)
//   O^T[d x 16 heads]        += V_page^T[d x 32] . P^T[32 x 16] (MFMA)
// The pool layout (include/pkd.h) puts each 16-byte vector a lane loads exactly
// where the matrix-core operand wants it, so a page arrives with fully
// contiguous 1 KiB wave loads and no LDS round trip; the score accumulator of a
// lane is already the P operand of the P.V product for the same lane, so the
// softmax needs no data movement except the per-head max and sum across the
// four 16-lane groups.  P enters the bf16 matrix core as a hi + lo pair of bf16
// numbers so that the weights keep ~16 significant bits.
//
// Long contexts are split into fixed chunks of `attn_chunk_pages` pages (a pool
// constant) merged in ascending chunk order afterwards ("llm-rs", section 4,
// lesson 2).  Every reduction has a fixed order, so a row's result does not
// depend on the batch ("GPU inference engine engineering", section "The same
// bits in any batch").  Barriers: none; each wave works alone.

#include <math.h>

#include <type_traits>

#include "common.h"

namespace pkd {

struct AttnParams {
  const uint8_t* pages;
  uint64_t page_stride;  // bytes per physical page: n_kv * 2 * block_bytes
  uint32_t block_bytes;
  const int32_t* table;
  const int32_t* counts;
  int32_t max_pages;
  int32_t max_seqs;
  int32_t num_pages;  // physical pages in the pool: a table entry outside [0, num_pages) is refused
  uint32_t* err;
  const int32_t* seq;
  const int32_t* pos;
  int32_t n_rows;
  int32_t n_kv;
  int32_t G;
  const void* q;
  int64_t q_stride;
  void* out;
  int32_t out_bf16;
  int64_t out_stride;
  float qk_scale;  // log2(e) / sqrt(d) * k_scale
  float v_scale;
  int32_t chunk_pages;
  int32_t max_ch;              // chunked: page chunks of the longest possible row
  float* part_ml;              // chunked: [units * n_kv * G][2]  (m, l)
  float* part_o;               // chunked: [units * n_kv * G][d]
  const void* new_k;           // [n_rows][n_kv][d] in q's dtype, or null
  const void* new_v;
  int64_t new_stride;          // elements between rows of new_k / new_v
  float enc_k_scale;           // fp8 pool: codes = E4M3(value / scale)
  float enc_v_scale;
  int32_t tile_rows;           // > 0: runs of rows of one sequence are read as tiles of this many rows
};

// Chunk count of a row (0 for a refused row) and the record of its chunk c:
// records are laid out per (row, chunk, kv head, query head of the group).
__device__ __forceinline__ int seq_count(const AttnParams& P, int s) {
  return (s >= 0 && s < P.max_seqs) ? min(P.counts[s], P.max_pages) : 0;
}
__device__ __forceinline__ int row_chunks(const AttnParams& P, int s, int p) {
  if (s < 0 || s >= P.max_seqs || p < 0 || p >= kPage * seq_count(P, s)) return 0;
  return ((p + kPage) / kPage + P.chunk_pages - 1) / P.chunk_pages;
}
__device__ __forceinline__ int64_t rec_of(const AttnParams& P, int r, int c, int g, int n) {
  return (((int64_t)r * P.max_ch + c) * P.n_kv + g) * P.G + n;
}

// Per-KV-dtype geometry.  kvt: 0 f32, 1 bf16, 2 fp8.  NL = 16-byte loads per lane
// for one K (or V) block of a page.
template <int KVT, int D>
struct Geo {
  static constexpr int ES = KVT == 0 ? 4 : KVT == 1 ? 2 : 1;
  static constexpr int NL = D * ES / 32;
  static constexpr int NMT = D / 16;                // 16-dim output tiles
  static constexpr int NQ = KVT == 0 ? D / 4 : D / 32;  // matrix-core k-steps per half page
};

template <int KVT, int D>
using PageRegs = u32x4[Geo<KVT, D>::NL];
template <int KVT, int D>
using QRegs = u32x4[Geo<KVT, D>::NQ];
template <int KVT, int D>
using QFRegs = float[Geo<KVT, D>::NQ];
template <int KVT, int D>
using ORegs = f32x4_t[Geo<KVT, D>::NMT];

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4 load16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// First block-table window of sequence s (lane i: logical page i), read in
// the same round trip as the page count; zeros for an out-of-range sequence.
// The count is clamped to the table length, so that no row reads past its
// sequence's table row whatever the device copy of the counts holds.
__device__ __forceinline__ void row_meta(const AttnParams& P, int s, int& count, int& tab) {
  const bool s_ok = s >= 0 && s < P.max_seqs;
  const int l = lane_id();
  count = s_ok ? min(P.counts[s], P.max_pages) : 0;
  tab = (s_ok && l < P.max_pages) ? P.table[(int64_t)s * P.max_pages + l] : 0;
}

// True (in every lane) when some lane l < n holds a table entry outside the
// pool; such entries are replaced by page 0 in `tab`, so that no load or store
// of the unit leaves the pool.  The unit is then refused (kErrPage).
__device__ __forceinline__ bool refuse_window(const AttnParams& P, int n, int& tab) {
  const bool b = lane_id() < n && (unsigned)tab >= (unsigned)P.num_pages;
  tab = b ? 0 : tab;
  return __builtin_amdgcn_ballot_w64(b) != 0;
}

// Row validity and context length; sets the sticky error word on a bad row.
__device__ __forceinline__ bool row_ok(const AttnParams& P, int s, int p, int count, bool report) {
  unsigned e = 0;
  if (s < 0 || s >= P.max_seqs) e = kErrSeq;
  else if (p < 0 || p >= kPage * count) e = kErrPos;
  if (e && report && lane_id() == 0) atomicOr(P.err, e);
  return e == 0;
}

// Loads the query registers (B operand of the score product): this lane's
// column is query head h of row r (zeros when not live).
template <int KVT, int D>
__device__ __forceinline__ void load_q_at(const AttnParams& P, int r, int h, bool live, QRegs<KVT, D>& qv,
                                          QFRegs<KVT, D>& qf) {
  using GE = Geo<KVT, D>;
  const int grp = lane_id() >> 4;
  if constexpr (KVT == 0) {
    const float* q = reinterpret_cast<const float*>(P.q) + (int64_t)r * P.q_stride + (int64_t)h * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      u32x4 v = live ? load16(reinterpret_cast<const uint8_t*>(q + 16 * i + 4 * grp)) : u32x4{0, 0, 0, 0};
      qf[4 * i + 0] = __uint_as_float(v.x);
      qf[4 * i + 1] = __uint_as_float(v.y);
      qf[4 * i + 2] = __uint_as_float(v.z);
      qf[4 * i + 3] = __uint_as_float(v.w);
    }
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(P.q) + (int64_t)r * P.q_stride + (int64_t)h * D;
#pragma unroll
    for (int s = 0; s < GE::NQ; ++s) {
      // bf16 pool: step s covers dims 32s + 8grp; fp8 pool: step s = 2i + e covers 64i + 16grp + 8e
      int c = KVT == 1 ? 32 * s + 8 * grp : 64 * (s >> 1) + 16 * grp + 8 * (s & 1);
      qv[s] = live ? load16(reinterpret_cast<const uint8_t*>(q + c)) : u32x4{0, 0, 0, 0};
    }
  }
}

// The G query heads of kv head g of row r as the 16 columns.
template <int KVT, int D>
__device__ __forceinline__ void load_q(const AttnParams& P, int r, int g, QRegs<KVT, D>& qv,
                                       QFRegs<KVT, D>& qf) {
  const int n = lane_id() & 15;
  const bool live = n < P.G;
  load_q_at<KVT, D>(P, r, g * P.G + (live ? n : 0), live, qv, qf);
}

// Scores of one page: S[a][i] = q_n . K[16a + 4grp + i] (unscaled), a = half page.
template <int KVT, int D>
__device__ __forceinline__ void page_scores(const PageRegs<KVT, D>& kr, const QRegs<KVT, D>& qv,
                                            const QFRegs<KVT, D>& qf, f32x4_t (&S)[2]) {
  using GE = Geo<KVT, D>;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KVT == 1) {
#pragma unroll
      for (int s = 0; s < GE::NQ; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[a * GE::NQ + s]), as_bf16x8(qv[s]), acc, 0, 0, 0);
    } else if constexpr (KVT == 2) {
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        u32x4 w = kr[a * (D / 64) + i];
        u32x2 b0 = fp8x4_to_bf16x4(w.x), b1 = fp8x4_to_bf16x4(w.y);
        u32x2 b2 = fp8x4_to_bf16x4(w.z), b3 = fp8x4_to_bf16x4(w.w);
        u32x4 lo = {b0.x, b0.y, b1.x, b1.y}, hi = {b2.x, b2.y, b3.x, b3.y};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), as_bf16x8(qv[2 * i]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), as_bf16x8(qv[2 * i + 1]), acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        u32x4 w = kr[a * (D / 16) + i];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), qf[4 * i + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), qf[4 * i + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), qf[4 * i + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), qf[4 * i + 3], acc, 0, 0, 0);
      }
    }
    S[a] = acc;
  }
}

// Zeroes the V elements of tokens at or past the context end (0 * NaN would
// poison the product otherwise).  valid[a][i] for token 16a + 4grp + i.
template <int KVT, int D>
__device__ __forceinline__ void mask_v(PageRegs<KVT, D>& vr, const bool (&valid)[2][4]) {
  using GE = Geo<KVT, D>;
  if constexpr (KVT == 1) {
    // dword w holds elements 2w, 2w + 1 = tokens (a = w / 2, i = 2(w % 2) + {0, 1})
    unsigned m[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      m[w] = (valid[w >> 1][2 * (w & 1)] ? 0xffffu : 0u) | (valid[w >> 1][2 * (w & 1) + 1] ? 0xffff0000u : 0u);
#pragma unroll
    for (int j = 0; j < GE::NL; ++j) {
      vr[j].x &= m[0]; vr[j].y &= m[1]; vr[j].z &= m[2]; vr[j].w &= m[3];
    }
  } else if constexpr (KVT == 2) {
    unsigned m[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
      m[a] = (valid[a][0] ? 0xffu : 0u) | (valid[a][1] ? 0xff00u : 0u) | (valid[a][2] ? 0xff0000u : 0u) |
             (valid[a][3] ? 0xff000000u : 0u);
#pragma unroll
    for (int j = 0; j < GE::NL; ++j) {
      vr[j].x &= m[0]; vr[j].y &= m[1]; vr[j].z &= m[0]; vr[j].w &= m[1];
    }
  } else {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int mt = 0; mt < GE::NMT; ++mt) {
        u32x4& v = vr[a * GE::NMT + mt];
        v.x = valid[a][0] ? v.x : 0u;
        v.y = valid[a][1] ? v.y : 0u;
        v.z = valid[a][2] ? v.z : 0u;
        v.w = valid[a][3] ? v.w : 0u;
      }
  }
}

// Zeroes the V elements of the page's tokens past position plast.
template <int KVT, int D>
__device__ __forceinline__ void mask_v_past(PageRegs<KVT, D>& vr, int pg, int plast) {
  bool valid[2][4];
  const int t0 = pg * kPage + 4 * (lane_id() >> 4);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) valid[a][i] = t0 + 16 * a + i <= plast;
  mask_v<KVT, D>(vr, valid);
}

// O^T += V^T . P^T for one page.  p[a][i] are the lane's softmax weights.
template <int KVT, int D>
__device__ __forceinline__ void page_pv(const PageRegs<KVT, D>& vr, const float (&p)[2][4],
                                        ORegs<KVT, D>& O) {
  using GE = Geo<KVT, D>;
  if constexpr (KVT == 0) {
#pragma unroll
    for (int mt = 0; mt < GE::NMT; ++mt)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        u32x4 v = vr[a * GE::NMT + mt];
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), p[a][0], O[mt], 0, 0, 0);
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), p[a][1], O[mt], 0, 0, 0);
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), p[a][2], O[mt], 0, 0, 0);
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), p[a][3], O[mt], 0, 0, 0);
      }
  } else {
    // P as hi + lo bf16 pairs; element e of the operand is token 16(e / 4) + 4grp + e % 4.
    unsigned hi[4], lo[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float p0 = p[w >> 1][2 * (w & 1)], p1 = p[w >> 1][2 * (w & 1) + 1];
      unsigned h0 = __float_as_uint(p0) & 0xffff0000u, h1 = __float_as_uint(p1) & 0xffff0000u;
      hi[w] = (h0 >> 16) | h1;
      lo[w] = pack_bf16(p0 - __uint_as_float(h0), p1 - __uint_as_float(h1));
    }
    bf16x8_t Ph = as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]});
    bf16x8_t Pl = as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]});
    if constexpr (KVT == 1) {
#pragma unroll
      for (int mt = 0; mt < GE::NMT; ++mt) {
        bf16x8_t A = as_bf16x8(vr[mt]);
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Ph, O[mt], 0, 0, 0);
        O[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Pl, O[mt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < GE::NL; ++j) {
        u32x2 b0 = fp8x4_to_bf16x4(vr[j].x), b1 = fp8x4_to_bf16x4(vr[j].y);
        u32x2 b2 = fp8x4_to_bf16x4(vr[j].z), b3 = fp8x4_to_bf16x4(vr[j].w);
        bf16x8_t A0 = as_bf16x8(u32x4{b0.x, b0.y, b1.x, b1.y});
        bf16x8_t A1 = as_bf16x8(u32x4{b2.x, b2.y, b3.x, b3.y});
        O[2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Ph, O[2 * j], 0, 0, 0);
        O[2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, Pl, O[2 * j], 0, 0, 0);
        O[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Ph, O[2 * j + 1], 0, 0, 0);
        O[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Pl, O[2 * j + 1], 0, 0, 0);
      }
    }
  }
}

// State of one work unit's online softmax.
template <int KVT, int D>
struct Acc {
  ORegs<KVT, D> O;
  float m;  // reference maximum (base-2 scaled scores) of the lane's column, see page_weights
  float l;  // this lane's partial sum of weights
};

// 2^x by the hardware instruction: results below 2^-126 flush to zero, which
// no softmax weight or rescale factor here can notice (the running sum is at
// least 1: the largest score is within kSlack above the reference).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax with a lagging reference maximum.  Each column keeps m, the
// reference its weights and sums are taken against, and moves it only when a
// score exceeds it by more than kSlack (base-2 units; the first valid score
// always sets it).  So weights lie in [0, 2^kSlack], and O and l are rescaled
// on the rare pages where the reference moves instead of on every page whose
// maximum grows; the result, O / l after the merge, is the same softmax.
constexpr float kSlack = 8.0f;

// Moves the reference m to cover the page maximum m_page when that exceeds it
// by more than kSlack, and returns the factor for O and l (1 when it stays; 0
// on the first valid page, where O and l are still zero).  A column with no
// valid score so far keeps m = -inf and factor 1.
__device__ __forceinline__ float next_reference(float& m, float m_page) {
  const float cand = fmaxf(m, m_page);
  const bool move = cand > m + kSlack;
  const float alpha = move ? fast_exp2(m - cand) : 1.0f;
  m = move ? cand : m;
  return alpha;
}

// Weights of one page from its scores S (q . K): the token of score S at or
// before position p_row gets p = 2^(s - m) with s = S qk_scale, and the
// others 0 (MASK = false: the caller knows every token of the page is valid).
// The empty asm keeps the compiler from fusing the scaling product into the
// subtraction (a fused multiply-add would round once where this rounds twice,
// and the token that sets the reference would not get weight exactly 1), so
// both forms give the same bits wherever every token is valid, whatever the
// kernel.  Updates the column's reference m and sum l, and returns the factor
// by which the caller rescales O (rescale).
template <bool MASK, int KVT, int D>
__device__ __forceinline__ float page_weights(const AttnParams& P, Acc<KVT, D>& A, const f32x4_t (&S)[2], int pg,
                                              int p_row, float (&p)[2][4]) {
  const int t0 = pg * kPage + 4 * (lane_id() >> 4);
  float s[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[a][i] = S[a][i] * P.qk_scale;
      asm("" : "+v"(s[a][i]));
      mx = fmaxf(mx, (!MASK || t0 + 16 * a + i <= p_row) ? s[a][i] : -INFINITY);
    }
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  const float alpha = next_reference(A.m, mx);
  // the lane's sum starts at its first weight (no weight is -0)
  float ls = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[a][i] = (!MASK || t0 + 16 * a + i <= p_row) ? fast_exp2(s[a][i] - A.m) : 0.f;
      ls = (a == 0 && i == 0) ? p[a][i] : ls + p[a][i];
    }
  A.l = fmaf(A.l, alpha, ls);
  return alpha;
}

// O *= alpha, skipped when no column's reference moved (alpha == 1 in every
// lane: the product would leave every bit as it is).
template <int KVT, int D>
__device__ __forceinline__ void rescale(Acc<KVT, D>& A, float alpha) {
  using GE = Geo<KVT, D>;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) == 0) return;
#pragma unroll
  for (int mt = 0; mt < GE::NMT; ++mt) A.O[mt] *= alpha;
}

// One page of a row's online softmax: weights p (masked on the row's last
// page only) and the rescale of O.
template <int KVT, int D>
__device__ __forceinline__ void page_softmax(const AttnParams& P, Acc<KVT, D>& A, const f32x4_t (&S)[2], int pg,
                                             int p_row, float (&p)[2][4]) {
  const float alpha = (pg + 1) * kPage <= p_row + 1 ? page_weights<false, KVT, D>(P, A, S, pg, p_row, p)
                                                    : page_weights<true, KVT, D>(P, A, S, pg, p_row, p);
  rescale<KVT, D>(A, alpha);
}

template <int KVT, int D>
__device__ __forceinline__ void load_block(const uint8_t* b, PageRegs<KVT, D>& r) {
  using GE = Geo<KVT, D>;
  const uint8_t* k = b + 16 * lane_id();
#pragma unroll
  for (int j = 0; j < GE::NL; ++j) r[j] = load16(k + 1024 * j);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// The same block from its staged copy in LDS (identical byte layout).
template <int KVT, int D>
__device__ __forceinline__ void load_block_lds(const lds_u8* b, PageRegs<KVT, D>& r) {
  using GE = Geo<KVT, D>;
  const lds_u8* k = b + 16 * lane_id();
#pragma unroll
  for (int j = 0; j < GE::NL; ++j) r[j] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(k + 1024 * j);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (lds wave-uniform).  The host compilation pass never sees the
// device builtin.
__device__ __forceinline__ void dma16(const uint8_t* g, lds_u8* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#else
  (void)g;
  (void)lds;
#endif
}

// Row r's own key and value for kv head g, as the pool stores them: lane l
// holds dims l and l + 64 (and so on) of each, already converted to the pool
// dtype (bits in the low bytes).  Loaded early; stored by append_store.
template <int KVT, int D>
struct NewToken {
  static constexpr int PER = (D + kWave - 1) / kWave;
  uint32_t k[PER], v[PER];
};

template <int KVT, int D>
__device__ __forceinline__ void append_load(const AttnParams& P, int r, int g, NewToken<KVT, D>& nt) {
  const int l = lane_id();
  const int64_t src = (int64_t)r * P.new_stride + (int64_t)g * D;
#pragma unroll
  for (int j = 0; j < NewToken<KVT, D>::PER; ++j) {
    const int c = l + kWave * j;
    if (c >= D) break;
    if constexpr (KVT == 0) {
      nt.k[j] = __float_as_uint(reinterpret_cast<const float*>(P.new_k)[src + c]);
      nt.v[j] = __float_as_uint(reinterpret_cast<const float*>(P.new_v)[src + c]);
    } else {
      nt.k[j] = reinterpret_cast<const uint16_t*>(P.new_k)[src + c];
      nt.v[j] = reinterpret_cast<const uint16_t*>(P.new_v)[src + c];
    }
  }
}

// Writes the token at slot t of physical page `page`, in the layout of
// include/pkd.h; fp8 pools take E4M3 RNE of value / scale (fp32 division),
// saturating.
template <int KVT, int D>
__device__ __forceinline__ void append_store(const AttnParams& P, int g, int page, int t,
                                             const NewToken<KVT, D>& nt) {
  uint8_t* kb = const_cast<uint8_t*>(P.pages) + (uint64_t)page * P.page_stride + (uint64_t)g * 2 * P.block_bytes;
  uint8_t* vb = kb + P.block_bytes;
  const int l = lane_id();
  const int a = t / 16, b = (t % 16) / 4, i = t % 4;
#pragma unroll
  for (int j = 0; j < NewToken<KVT, D>::PER; ++j) {
    const int c = l + kWave * j;
    if (c >= D) break;
    if constexpr (KVT == 0) {
      reinterpret_cast<uint32_t*>(kb)[((t / 16) * (D / 4) + c / 4) * 64 + (t % 16) * 4 + c % 4] = nt.k[j];
      reinterpret_cast<uint32_t*>(vb)[(((a * (D / 16) + c / 16) * 4 + b) * 16 + c % 16) * 4 + i] = nt.v[j];
    } else if constexpr (KVT == 1) {
      reinterpret_cast<uint16_t*>(kb)[((t / 16) * (D / 8) + c / 8) * 128 + (t % 16) * 8 + c % 8] = (uint16_t)nt.k[j];
      reinterpret_cast<uint16_t*>(vb)[(((c / 16) * 4 + b) * 16 + c % 16) * 8 + 4 * a + i] = (uint16_t)nt.v[j];
    } else {
      const unsigned codes = f32x2_to_fp8x2(bf16_bits_to_f32(nt.k[j]) / P.enc_k_scale,
                                            bf16_bits_to_f32(nt.v[j]) / P.enc_v_scale);
      kb[((t / 16) * (D / 16) + c / 16) * 256 + (t % 16) * 16 + c % 16] = (uint8_t)(codes & 0xff);
      vb[(((c / 32) * 4 + b) * 16 + c % 16) * 16 + 8 * ((c / 16) % 2) + 4 * a + i] = (uint8_t)(codes >> 8);
    }
  }
}

// Runs pages [pg0, pg1) of row r, kv head g, with the row's query registers
// qv / qf (load_q; callers issue that load early, since it depends on the row
// and kv head alone).  One K and one V block live in
// registers: the next page's K is requested as soon as the score products have
// consumed the current K, and its V once the P.V products have consumed the
// current V, so a wave keeps about one page in flight with half the registers
// of a double buffer and three waves fit on a SIMD.
// staged / n_staged: logical pages [0, n_staged) of the row are shared with the
// other rows of the workgroup and were staged in LDS once for all of them
// (page j's K block at staged + 2 j block_bytes, its V block after it); they
// are read from there, byte for byte what the global loads would return.
// Returns true when a table entry of the unit's pages lies outside the pool:
// page 0 was read in its place and nothing was appended, and the caller
// refuses the unit (zeros, kErrPage).
template <int KVT, int D, bool FUSE = false>
__device__ __forceinline__ bool run_unit(const AttnParams& P, Acc<KVT, D>& A, int r, int s, int p_row, int g,
                                         int pg0, int pg1, int tab, const QRegs<KVT, D>& qv,
                                         const QFRegs<KVT, D>& qf, const lds_u8* staged = nullptr,
                                         int n_staged = 0) {
  using GE = Geo<KVT, D>;
#pragma unroll
  for (int mt = 0; mt < GE::NMT; ++mt) A.O[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  A.m = -INFINITY;
  A.l = 0.f;
  const int32_t* trow = P.table + (int64_t)s * P.max_pages;
  const uint8_t* base = P.pages + (uint64_t)g * 2 * P.block_bytes;
  // lane i holds the physical page of logical page win + i (tab: the caller's
  // window at pg0): the unit's table entries arrive in one load instead of one
  // dependent load per page
  int win = pg0;
  bool bad = refuse_window(P, pg1 - win, tab);
  auto page_of = [&](int pg) {
    if (pg - win >= kWave) {
      win += kWave;
      tab = win + lane_id() < pg1 ? trow[win + lane_id()] : 0;
      bad = refuse_window(P, pg1 - win, tab) || bad;
    }
    return __shfl(tab, pg - win, kWave);
  };
  // FUSE: the row's own token is stored into its page here, and every load of
  // that page waits for the stores (vmcnt(0) covers this wave's stores), so
  // the page is read exactly as a separate append pass would leave it.  No
  // other wave of the launch reads that page.
  const int own = FUSE ? p_row / kPage : -1;
  // the own page's table entry is read directly: the lane window above only
  // moves forward one page at a time, and the own page may lie 64 or more
  // pages past pg0.  An entry outside the pool is not written to.
  int own_page = FUSE ? trow[own] : 0;
  const bool own_ok = !FUSE || (unsigned)own_page < (unsigned)P.num_pages;
  if (!own_ok) {
    own_page = 0;
    bad = true;
  }
  NewToken<KVT, D> nt;
  if constexpr (FUSE) append_load<KVT, D>(P, r, g, nt);
  u32x4 kr[GE::NL], vr[GE::NL];
  // K (c = 0) or V (c = 1) block of logical page pg, from LDS when staged
  auto load = [&](int pg, int c, PageRegs<KVT, D>& regs) {
    if (pg < n_staged) load_block_lds<KVT, D>(staged + (2 * pg + c) * P.block_bytes, regs);
    else load_block<KVT, D>(base + (uint64_t)page_of(pg) * P.page_stride + c * P.block_bytes, regs);
  };
  if (FUSE && own == pg0) {
    if (own_ok) append_store<KVT, D>(P, g, own_page, p_row % kPage, nt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  load(pg0, 0, kr);
  load(pg0, 1, vr);
  if (FUSE && own != pg0 && own_ok) append_store<KVT, D>(P, g, own_page, p_row % kPage, nt);
  for (int pg = pg0; pg < pg1; ++pg) {
    const bool nxt = pg + 1 < pg1;
    f32x4_t S[2];
    page_scores<KVT, D>(kr, qv, qf, S);
    if (FUSE && pg + 1 == own) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (nxt) load(pg + 1, 0, kr);
    float p[2][4];
    page_softmax<KVT, D>(P, A, S, pg, p_row, p);
    if ((pg + 1) * kPage > p_row + 1) mask_v_past<KVT, D>(vr, pg, p_row);  // partial last page
    page_pv<KVT, D>(vr, p, A.O);
    if (nxt) load(pg + 1, 1, vr);
  }
  return bad;
}

// Sum of the lane-partial l over the four 16-lane groups (fixed butterfly).
__device__ __forceinline__ float group_sum(float l) {
  return add_xor32(add_xor16(l));
}

template <int D>
__device__ __forceinline__ void store_out4(const AttnParams& P, int r, int h, int c, f32x4_t v) {
  if (P.out_bf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(P.out) + (int64_t)r * P.out_stride + (int64_t)h * D + c;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
    float* o = reinterpret_cast<float*>(P.out) + (int64_t)r * P.out_stride + (int64_t)h * D + c;
    *reinterpret_cast<f32x4_t*>(o) = v;
  }
}

// Final normalisation and store of the G heads of kv head g.
template <int KVT, int D>
__device__ __forceinline__ void finish(const AttnParams& P, const Acc<KVT, D>& A, int r, int g) {
  using GE = Geo<KVT, D>;
  const int l = lane_id(), grp = l >> 4, n = l & 15;
  const float lsum = group_sum(A.l);
  if (n >= P.G) return;
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int mt = 0; mt < GE::NMT; ++mt) {
    f32x4_t v = A.O[mt] * inv * P.v_scale;
    store_out4<D>(P, r, g * P.G + n, 16 * mt + 4 * grp, v);
  }
}

template <int D>
__device__ __forceinline__ void zero_heads(const AttnParams& P, int r, int g) {
  const int l = lane_id(), grp = l >> 4, n = l & 15;
  if (n >= P.G) return;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) store_out4<D>(P, r, g * P.G + n, 16 * mt + 4 * grp, f32x4_t{0.f, 0.f, 0.f, 0.f});
}

// Tiles for prompt slices: rows [t T, t T + T) (T = P.tile_rows) form a
// shared tile when there are at least two of them and they are one sequence
// at consecutive positions from 0 up (a prompt slice).  Tiles were faster
// than the per-row kernels at every measured context (256-row slices of a
// 7B-shaped layer starting at positions 0, 256, 512, 768, 1024 and 2304:
// 23, 28, 30, 32, 35 and 49 us tiled against 24, 33, 37, 42, 48 and 73 us per
// row).  Every kernel that schedules rows evaluates this the same way: the
// per-row kernels leave such rows to the tile workgroups (tile_unit).  Rows
// are checked one per lane, so the whole wave calls it.

// Lane j reads row r0 + j of tile t (a tile has at most 64 rows); s0 and p0
// return its first row's sequence and position.
__device__ __forceinline__ bool tile_probe(const AttnParams& P, int t, int& s0, int& p0) {
  const int T = P.tile_rows, r0 = t * T, nr = min(P.n_rows, r0 + T) - r0;
  s0 = -1;
  p0 = 0;
  if (T <= 0 || nr < 2) return false;
  const int j = lane_id();
  const bool in = j < nr;
  const int sj = in ? P.seq[r0 + j] : 0, pj = in ? P.pos[r0 + j] : 0;
  s0 = __shfl(sj, 0, kWave);
  p0 = __shfl(pj, 0, kWave);
  if (p0 < 0) return false;  // the per-row kernels refuse such rows
  return __builtin_amdgcn_ballot_w64(in && (sj != s0 || pj != p0 + j)) == 0;
}

__device__ __forceinline__ bool tile_shared(const AttnParams& P, int t) {
  int s0, p0;
  return tile_probe(P, t, s0, p0);
}

// One wave per (row, kv head); every row is a single chunk.
//   FUSE: every sequence has one row in the launch; the wave also appends its
//   row's token (see run_unit).
// A workgroup holds four consecutive rows (one wave each) for one kv head.
// Leading logical pages that every valid row of the workgroup maps to the same
// physical page (a shared prompt prefix), other than any row's last page (the
// page its own token goes to), are loaded into LDS once and read from there by
// all four waves.
template <int KVT, int D>
struct Stage {
  static constexpr int BLOCK = kPage * D * Geo<KVT, D>::ES;  // bytes of one K or V block
  static constexpr int PAGES = (32768 / (2 * BLOCK)) < 4 ? (32768 / (2 * BLOCK)) : 4;
  static constexpr int BYTES = PAGES * 2 * BLOCK;            // at most 32 KiB
};

// Stages into `stage_mem` the leading pages that every valid row of the
// workgroup shares, and returns how many there are.  Each wave passes its
// row's position p, first table window tab and validity ok.  Holds the
// workgroup's only barriers, reached by all four waves.
template <int KVT, int D>
__device__ __forceinline__ int stage_shared(const AttnParams& P, int g, int p, int tab, bool ok,
                                            uint8_t* stage_mem) {
  using ST = Stage<KVT, D>;
  __shared__ int meta[4][2 + ST::PAGES];  // per wave: valid, page count, first table entries
  const int wave = threadIdx.x >> 6, l = lane_id();
  if (l < ST::PAGES) meta[wave][2 + l] = tab;
  if (l == 0) {
    meta[wave][0] = ok ? 1 : 0;
    meta[wave][1] = ok ? (p + kPage) / kPage : 0;
  }
  __syncthreads();
  // pages every valid row shares (same for all four waves)
  int n_valid = 0, lead = -1, n_staged = ST::PAGES;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (!meta[w][0]) continue;
    ++n_valid;
    if (lead < 0) lead = w;
    n_staged = min(n_staged, meta[w][1] - 1);  // never a row's last page
  }
  if (n_valid < 2) n_staged = 0;
  for (int j = 0; j < n_staged; ++j) {
    bool same = true;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (meta[w][0] && meta[w][2 + j] != meta[lead][2 + j]) same = false;
    if (!same) {
      n_staged = j;
      break;
    }
  }
  if (n_staged > 0) {
    // 1 KiB wave loads: page j, block c, part i; dealt round-robin to the waves
    constexpr int PARTS = ST::BLOCK / 1024;
    lds_u8* staged = (lds_u8*)stage_mem;
    const uint8_t* gbase = P.pages + (uint64_t)g * 2 * P.block_bytes;
    for (int q = wave; q < n_staged * 2 * PARTS; q += 4) {
      const int j = q / (2 * PARTS), c = (q / PARTS) % 2, i = q % PARTS;
      const uint8_t* src = gbase + (uint64_t)meta[lead][2 + j] * P.page_stride + c * P.block_bytes + 1024 * i + 16 * l;
      dma16(src, staged + (2 * j + c) * ST::BLOCK + 1024 * i);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  return n_staged;
}

// STAGE: the pool has pages listed by two or more sequences (a shared prompt
// prefix), so the workgroup looks for leading pages its rows share and stages
// them in LDS.  Without shared pages the kernel holds no LDS and no barrier,
// and more waves fit on a CU.  A staged page is read byte for byte as its
// global copy, so both variants give identical results.
//   Grid: with STAGE, (row quads) x kv heads, so that a workgroup holds four
//   rows of one kv head; without, units u = row * n_kv + kv head dealt four
//   to a workgroup, so that the kv heads of a row, whose blocks lie side by
//   side in each page, are read together.
template <int KVT, int D, bool FUSE, bool STAGE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_direct_kernel(AttnParams P) {
  using ST = Stage<KVT, D>;
  const int wave = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + wave;
  const int r = STAGE ? u : u / P.n_kv, g = STAGE ? (int)blockIdx.y : u % P.n_kv;
  // the query depends on the row and kv head alone: requested first, so that
  // it arrives while the row's metadata and any staged pages are read
  u32x4 qv[Geo<KVT, D>::NQ];
  float qf[Geo<KVT, D>::NQ];
  load_q<KVT, D>(P, r < P.n_rows ? r : 0, g, qv, qf);
  // rows of a shared tile are tile_unit's: treated here as absent
  const bool in_range = r < P.n_rows && !(P.tile_rows > 0 && tile_shared(P, r / P.tile_rows));
  const int s = in_range ? P.seq[r] : -1, p = in_range ? P.pos[r] : 0;
  int count, tab;
  row_meta(P, s, count, tab);
  bool ok = in_range && row_ok(P, s, p, count, g == 0);
  // the row's first table window must name pool pages (the staging below
  // reads the shared ones); later windows are checked as run_unit reaches them
  if (ok && refuse_window(P, (p + kPage) / kPage, tab)) {
    ok = false;
    if (g == 0 && lane_id() == 0) atomicOr(P.err, kErrPage);
  }
  int n_staged = 0;
  const lds_u8* staged = nullptr;
  if constexpr (STAGE) {
    __shared__ __attribute__((aligned(16))) uint8_t stage_mem[ST::BYTES];
    n_staged = stage_shared<KVT, D>(P, g, p, tab, ok, stage_mem);
    staged = (const lds_u8*)stage_mem;
  }
  if (!in_range) return;
  if (!ok) {
    zero_heads<D>(P, r, g);
    return;
  }
  Acc<KVT, D> A;
  if (run_unit<KVT, D, FUSE>(P, A, r, s, p, g, 0, (p + kPage) / kPage, tab, qv, qf, staged, n_staged)) {
    if (lane_id() == 0) atomicOr(P.err, kErrPage);
    zero_heads<D>(P, r, g);
    return;
  }
  finish<KVT, D>(P, A, r, g);
}

// Chunked mode: one wave per (row, page chunk, kv head); a workgroup is four
// kv heads of one (row, chunk), whose blocks lie side by side in every page,
// rows x chunks x ceil(n_kv / 4) workgroups (chunk_wg), the kv-head quads
// innermost in dispatch order, then the chunks, then the rows.  Waves past
// the row's chunks, or whose row a shared tile covers, exit at once: the grid
// maps units directly, with no counter to contend on; the chunks past a short
// row's last are whole workgroups that exit together.  (Four chunks of one
// row per workgroup, measured on the 0.6B mixed step: 241-243 us cold against
// 238-240; visiting all rows' first chunks first: 248.)  A row with one chunk
// is finished here; the others leave (m, l, O) at record (row, chunk) for the
// ordered merge.  A refused row is reported here (chunk 0, kv head 0) and
// zeroed by the merge.
//   FUSE: every sequence has one row in the launch; the wave of the row's last
//   chunk (the one holding its own page) also appends the row's token, as in
//   the direct kernel, and no other chunk reads that page.
template <int KVT, int D, bool FUSE>
__device__ __forceinline__ void chunked_unit(const AttnParams& P, int wg) {
  using GE = Geo<KVT, D>;
  const int nq4 = (P.n_kv + 3) / 4;
  const int g = 4 * (wg % nq4) + (threadIdx.x >> 6);
  const int c = (wg / nq4) % P.max_ch, r = wg / nq4 / P.max_ch;
  if (c >= P.max_ch || g >= P.n_kv) return;
  const int l = lane_id(), grp = l >> 4, n = l & 15;
  const int s = P.seq[r], p = P.pos[r];
  const int npg = (p + kPage) / kPage;
  // chunks past the row's context (most waves of a batch of short rows) leave
  // after this one load; chunk 0 stays to report a refused row
  if (c > 0 && c * P.chunk_pages >= npg) return;
  // the shared-tile check, the row's count and the chunk's table window in
  // one round trip (window lanes past the row's pages are never used)
  const bool tiled = P.tile_rows > 0 && tile_shared(P, r / P.tile_rows);
  const int count = seq_count(P, s);
  const int pg0 = c * P.chunk_pages;
  const bool s_ok = s >= 0 && s < P.max_seqs;
  const int tab =
      (s_ok && pg0 + l < min(P.max_pages, pg0 + P.chunk_pages)) ? P.table[(int64_t)s * P.max_pages + pg0 + l] : 0;
  if (tiled) return;
  u32x4 qv[GE::NQ];
  float qf[GE::NQ];
  load_q<KVT, D>(P, r, g, qv, qf);
  if (!row_ok(P, s, p, count, c == 0 && g == 0)) return;
  const int nch = (npg + P.chunk_pages - 1) / P.chunk_pages;
  if (c >= nch) return;
  const int pg1 = min(npg, pg0 + P.chunk_pages);
  Acc<KVT, D> A;
  const bool bad = (FUSE && c == nch - 1) ? run_unit<KVT, D, true>(P, A, r, s, p, g, pg0, pg1, tab, qv, qf)
                                          : run_unit<KVT, D, false>(P, A, r, s, p, g, pg0, pg1, tab, qv, qf);
  if (bad && l == 0) atomicOr(P.err, kErrPage);
  if (nch == 1) {
    if (bad) zero_heads<D>(P, r, g);
    else finish<KVT, D>(P, A, r, g);
    return;
  }
  // a refused chunk leaves l = -1, which makes the merge zero the row
  const float lsum = bad ? -1.0f : group_sum(A.l);
  if (n < P.G) {
    const int64_t rec = rec_of(P, r, c, g, n);
    if (grp == 0) {
      P.part_ml[2 * rec] = A.m;
      P.part_ml[2 * rec + 1] = lsum;
    }
#pragma unroll
    for (int mt = 0; mt < GE::NMT; ++mt)
      *reinterpret_cast<f32x4_t*>(P.part_o + rec * D + 16 * mt + 4 * grp) = A.O[mt];
  }
}

template <int KVT, int D, bool FUSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_chunked_kernel(AttnParams P) {
  chunked_unit<KVT, D, FUSE>(P, blockIdx.x);
}

// Shared tiles (prompt slices): one workgroup of NW waves per (tile, page
// chunk, kv head).  The tile's rows x G query heads are its columns, packed
// densely: column j is (row j / G, query head j % G), and wave w holds columns
// [16 NB w, 16 NB (w + 1)) as NB matrix-core blocks of 16 (a tile has at most
// 16 NB NW columns).  The chunk's pages are fetched once per workgroup, straight
// into an LDS ring of NBUF pages: each wave loads its share of every page, NBUF
// - 1 pages ahead, and every wave reads each page from LDS in the byte layout
// a global load would give.  Every column runs the per-row arithmetic: the
// same pages in the same order, and the pages and tokens past its own position
// are exact no-ops for it (no valid token: weights 0, rescale 1).  V is masked
// past the tile's last position; the tokens between a column's own position
// and the tile's last are tokens of this slice, all written before the kernel
// runs.  So each row's output is bit-identical to the per-row kernels'.
// Used with chunked pools only (the page chunks are what give a tile's pages
// parallelism): a row with one chunk is finished here, the others leave
// records for the ordered merge, and a refused row is reported here and
// zeroed by the merge.
constexpr int kTileWaves = 4;  // waves per tile workgroup

template <int KVT, int D>
struct TileCfg {
  static constexpr int NW = kTileWaves;
  static constexpr int NB = 1;                 // 16-column blocks per wave
  static constexpr int COLS = 16 * NB * NW;    // columns of a tile
  static constexpr int BLOCK = kPage * D * Geo<KVT, D>::ES;  // bytes of one K or V block
  static constexpr int SLOT = 2 * BLOCK;                     // one page of one kv head: K block, V block
  static constexpr int LOADS = 2 * Geo<KVT, D>::NL / NW;     // 1 KiB wave loads per page and wave
  static constexpr int RING = 49152;                         // LDS bytes of the page ring (at least two pages)
  static constexpr int NBUF = RING / SLOT < 2 ? 2 : RING / SLOT > 8 ? 8 : RING / SLOT;
  static_assert(2 * Geo<KVT, D>::NL % NW == 0 && LOADS >= 1, "page loads must split evenly over the waves");
  static_assert(NBUF >= 2 && LOADS * (NBUF - 2) <= 63, "ring deeper than the vmcnt counter");
};

// Waits until this wave's loads of all pages but the last `ahead` (< MAXA) it
// issued have landed in LDS (vmcnt counts this wave's loads in issue order),
// and until its own LDS reads are done.
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_pages(int ahead) {
  if constexpr (MAXA <= 1) {
    __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
    wait_lds_reads();
  } else if (ahead >= MAXA - 1) {
    __builtin_amdgcn_s_waitcnt(PKD_VMCNT(LOADS * (MAXA - 1)));
    wait_lds_reads();
  } else {
    wait_pages<LOADS, MAXA - 1>(ahead);
  }
}

// Workgroup bx of 8 ceil(units / 8) n_tiles, for units = chunks x kv heads.
// Workgroup i runs on XCD i mod 8 (the tile workgroups come first in their
// grid); the tiles of one (chunk, kv head) unit are given to one XCD, so that
// its pages are fetched into one L2.
template <int KVT, int D>
__device__ __forceinline__ void tile_unit(const AttnParams& P, int bx, int n_tiles, int n_units) {
  using GE = Geo<KVT, D>;
  using TC = TileCfg<KVT, D>;
  constexpr int NB = TC::NB;
  __shared__ __attribute__((aligned(16))) uint8_t ring[TC::NBUF * TC::SLOT];
  const int xcd = bx % 8, y = bx / 8;
  const int u = xcd + 8 * (y / n_tiles), t = y % n_tiles;
  if (u >= n_units) return;
  const int c = u / P.n_kv, g = u % P.n_kv;
  const int wave = threadIdx.x >> 6, l = lane_id(), grp = l >> 4, n = l & 15;
  const int G = P.G;
  const int r0 = t * P.tile_rows, nr = min(P.n_rows, r0 + P.tile_rows) - r0;
  // the queries depend on the tile's rows alone: requested before the rows
  // are read, so that they arrive meanwhile (rows past the call are not read)
  int jr[NB];
  u32x4 qv[NB][GE::NQ];
  float qf[NB][GE::NQ];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = (wave * NB + b) * 16 + n;
    jr[b] = j / G;
    const bool live = jr[b] < nr;
    load_q_at<KVT, D>(P, live ? r0 + jr[b] : r0, live ? g * G + j % G : g * G, live, qv[b], qf[b]);
  }
  int s, p0;
  if (!tile_probe(P, t, s, p0)) return;
  const bool s_ok = s >= 0 && s < P.max_seqs;
  // the sequence's count and the table window of this chunk, in one round trip
  const int32_t* trow = P.table + (int64_t)(s_ok ? s : 0) * P.max_pages;
  const int pg0 = c * P.chunk_pages;
  const int count = seq_count(P, s);
  int win = pg0;
  int tab = (s_ok && pg0 + l < min(P.max_pages, pg0 + P.chunk_pages)) ? trow[pg0 + l] : 0;
  // rows r0 + j are at positions p0 + j (p0 >= 0, see tile_shared); the
  // valid ones are a prefix, ending at the last position the table covers
  const int plast = s_ok ? min(p0 + nr - 1, kPage * count - 1) : -1;
  // refused rows: reported once (chunk 0, kv head 0), zeroed by the merge
  if (plast < p0 + nr - 1 && c == 0 && g == 0 && threadIdx.x == 0) atomicOr(P.err, !s_ok ? kErrSeq : kErrPos);
  if (plast < p0) return;
  const int npg = (plast + kPage) / kPage;
  const int pg1 = min(npg, pg0 + P.chunk_pages);
  if (pg0 >= npg) return;
  int rw[NB], hh[NB], prow[NB], nch[NB];
  bool act[NB], on[NB];
  Acc<KVT, D> A[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = (wave * NB + b) * 16 + n;
    const int pc = p0 + jr[b];
    rw[b] = r0 + jr[b];
    hh[b] = g * G + j % G;
    nch[b] = (jr[b] < nr && pc <= plast) ? ((pc + kPage) / kPage + P.chunk_pages - 1) / P.chunk_pages : 0;
    act[b] = c < nch[b];
    prow[b] = act[b] ? pc : -1;
    on[b] = __builtin_amdgcn_ballot_w64(act[b]) != 0;  // the block has work in this chunk
#pragma unroll
    for (int mt = 0; mt < GE::NMT; ++mt) A[b].O[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    A[b].m = -INFINITY;
    A[b].l = 0.f;
  }
  bool bad = refuse_window(P, pg1 - win, tab);
  auto page_of = [&](int pg) {
    if (pg - win >= kWave) {
      win += kWave;
      tab = win + l < pg1 ? trow[win + l] : 0;
      bad = refuse_window(P, pg1 - win, tab) || bad;
    }
    return __shfl(tab, pg - win, kWave);
  };
  const uint8_t* base = P.pages + (uint64_t)g * 2 * P.block_bytes;
  // this wave's share of logical page pg (K block, then V block) into ring slot `slot`
  auto issue = [&](int pg, int slot) {
    const int page = __builtin_amdgcn_readfirstlane(page_of(pg));
    const __amdgpu_buffer_rsrc_t v = operand_view(base + (uint64_t)page * P.page_stride, 2 * TC::BLOCK);
#pragma unroll
    for (int k = 0; k < TC::LOADS; ++k) {
      const int q = wave + TC::NW * k;  // 1 KiB part q of the page's two blocks
      lds_load16(v, (uint32_t)(1024 * q + 16 * l), 0, ring + slot * TC::SLOT + 1024 * q);
    }
  };
  const int np = pg1 - pg0;
  for (int k = 0; k < TC::NBUF - 1 && k < np; ++k) issue(pg0 + k, k);
  u32x4 kr[GE::NL], vr[GE::NL];
  for (int i = 0; i < np; ++i) {
    const int pg = pg0 + i;
    // page i has landed for every wave, and every wave is done with page i - 1,
    // whose slot the next request refills
    wait_pages<TC::LOADS, TC::NBUF - 1>(min(np - 1 - i, TC::NBUF - 2));
    lds_barrier();
    if (i + TC::NBUF - 1 < np) issue(pg + TC::NBUF - 1, (i + TC::NBUF - 1) % TC::NBUF);
    const lds_u8* kb = (const lds_u8*)ring + (i % TC::NBUF) * TC::SLOT;
    load_block_lds<KVT, D>(kb, kr);
    f32x4_t S[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (on[b]) page_scores<KVT, D>(kr, qv[b], qf[b], S[b]);
    load_block_lds<KVT, D>(kb + TC::BLOCK, vr);
    float p[NB][2][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (!on[b]) continue;
      // every active column of the block sees the whole page: the unmasked
      // weights (inactive columns are never stored; their queries are zero or
      // real, so they stay finite).  O is rescaled in one place, after either
      // form.
      const float alpha = __builtin_amdgcn_ballot_w64(act[b] && prow[b] < pg * kPage + kPage - 1) == 0
                              ? page_weights<false, KVT, D>(P, A[b], S[b], pg, prow[b], p[b])
                              : page_weights<true, KVT, D>(P, A[b], S[b], pg, prow[b], p[b]);
      rescale<KVT, D>(A[b], alpha);
    }
    if ((pg + 1) * kPage > plast + 1) mask_v_past<KVT, D>(vr, pg, plast);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (on[b]) page_pv<KVT, D>(vr, p[b], A[b].O);
  }
  if (bad && threadIdx.x == 0) atomicOr(P.err, kErrPage);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    // a refused chunk leaves l = -1, which makes the merge zero the row
    const float lsum = bad ? -1.0f : group_sum(A[b].l);
    if (!act[b]) continue;
    if (nch[b] == 1) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int mt = 0; mt < GE::NMT; ++mt)
        store_out4<D>(P, rw[b], hh[b], 16 * mt + 4 * grp,
                      bad ? f32x4_t{0.f, 0.f, 0.f, 0.f} : A[b].O[mt] * inv * P.v_scale);
    } else {
      const int64_t rec = rec_of(P, rw[b], c, g, hh[b] - g * G);
      if (grp == 0) {
        P.part_ml[2 * rec] = A[b].m;
        P.part_ml[2 * rec + 1] = lsum;
      }
#pragma unroll
      for (int mt = 0; mt < GE::NMT; ++mt)
        *reinterpret_cast<f32x4_t*>(P.part_o + rec * D + 16 * mt + 4 * grp) = A[b].O[mt];
    }
  }
}

// Calls with shared tiles: the tile workgroups, then the per-row chunk
// workgroups (attn_chunked_kernel's, in its order), in one launch; the per-row
// workgroups of tiled rows leave after the tile check while the tiles run.
template <int KVT, int D>
__global__ __launch_bounds__(64 * kTileWaves) __attribute__((amdgpu_waves_per_eu(3))) void attn_tiles_rows_kernel(
    AttnParams P, int n_tile_wgs, int n_tiles, int n_units) {
  static_assert(kTileWaves == 4, "the per-row workgroups hold four waves");
  if ((int)blockIdx.x < n_tile_wgs) {
    tile_unit<KVT, D>(P, blockIdx.x, n_tiles, n_units);
  } else {
    chunked_unit<KVT, D, false>(P, blockIdx.x - n_tile_wgs);
  }
}

// Chunked mode, last step: one wave per (row, query head) merges the chunk
// results of rows with more than one chunk; refused rows get zeros.  Lane c
// holds chunk c's (m, l) (64 chunks at a time), so the maximum is one wave
// reduction and the weights are computed in parallel; the weighted sums of l
// and of O are then taken in ascending chunk order, with the O loads of
// several chunks in flight at once.
// UMAX: the largest number of chunk records requested at a time past the
// first four (4 or 16; the same sums either way).  16 serves pools whose rows
// can have many chunks; 4 keeps the kernel at 48 VGPRs, so that every wave of
// a large merge is resident at once.
template <int D, int UMAX>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnParams P) {
  const int hq = P.n_kv * P.G;
  const int r = blockIdx.x / hq, h = blockIdx.x % hq, g = h / P.G, n = h % P.G;
  const int l = lane_id();
  constexpr int PER = D / 64;  // dims per lane
  // The records of the first chunks are requested before the row's chunk
  // count is known (records past it hold stale values and are not used): lane
  // c's (m, l) of chunk c < 64, and the O records of chunks 0..3.
  float ms = -INFINITY, lsv = 0.f;
  if (l < min(P.max_ch, kWave)) {
    const int64_t rec = rec_of(P, r, l, g, n);
    ms = P.part_ml[2 * rec];
    lsv = P.part_ml[2 * rec + 1];
  }
  float v0[4][PER];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t rec = rec_of(P, r, min(u, P.max_ch - 1), g, n);
#pragma unroll
    for (int j = 0; j < PER; ++j) v0[u][j] = P.part_o[rec * D + PER * l + j];
  }
  const int nch = row_chunks(P, P.seq[r], P.pos[r]);
  if (nch == 1) return;
  float o[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = 0.f;
  if (nch > 0) {
    // lane c holds (m, l) of chunk c; chunks past the first 64 are read again
    // below, once the maximum is known
    const float m0 = l < nch ? ms : -INFINITY, l0 = l < nch ? lsv : 0.f;
    float M = m0;
    // a chunk that met a table entry outside the pool left l = -1: the row is
    // refused and written as zeros
    bool refused = l0 < 0.f;
    for (int c0 = kWave; c0 < nch; c0 += kWave)
      if (c0 + l < nch) {
        const int64_t rec = rec_of(P, r, c0 + l, g, n);
        M = fmaxf(M, P.part_ml[2 * rec]);
        refused = refused || P.part_ml[2 * rec + 1] < 0.f;
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor(M, m));
    float L = 0.f;
    const int nsum = __builtin_amdgcn_ballot_w64(refused) ? 0 : nch;
    for (int c0 = 0; c0 < nsum; c0 += kWave) {
      float wl = 0.f, ll = 0.f;
      if (c0 == 0) {
        if (l < nch) {
          wl = fast_exp2(m0 - M);
          ll = l0;
        }
      } else if (c0 + l < nch) {
        const int64_t rec = rec_of(P, r, c0 + l, g, n);
        wl = fast_exp2(P.part_ml[2 * rec] - M);
        ll = P.part_ml[2 * rec + 1];
      }
      const int cn = min(kWave, nch - c0);
      // U chunk records requested at a time (one round trip for up to U
      // chunks; 4 for short rows, so that the clamped extra requests stay
      // few), then added in chunk order.  No branch between the loads and the
      // sums (a break there let the compiler wait for each record in turn);
      // records past cn are selected away, so every bit is that of adding
      // chunks c .. cn - 1 in order.
      int c = 0;
      if (c0 == 0) {  // chunks 0..3, from the records requested up front
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool in = u < cn;
          const float w = __shfl(wl, min(u, cn - 1), kWave);
          const float Ln = L + __shfl(ll, min(u, cn - 1), kWave) * w;
          L = in ? Ln : L;
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const float on = o[j] + v0[u][j] * w;
            o[j] = in ? on : o[j];
          }
        }
        c = 4;
      }
      auto accumulate = [&](auto u_const) {
        constexpr int U = decltype(u_const)::value;
        for (; c < cn; c += U) {
          float v[U][PER];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t rec = rec_of(P, r, c0 + min(c + u, cn - 1), g, n);
#pragma unroll
            for (int j = 0; j < PER; ++j) v[u][j] = P.part_o[rec * D + PER * l + j];
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const bool in = c + u < cn;
            const float w = __shfl(wl, min(c + u, cn - 1), kWave);
            const float Ln = L + __shfl(ll, min(c + u, cn - 1), kWave) * w;
            L = in ? Ln : L;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
              const float on = o[j] + v[u][j] * w;
              o[j] = in ? on : o[j];
            }
          }
        }
      };
      if (UMAX == 4 || cn - c <= 4) accumulate(std::integral_constant<int, 4>{});
      else accumulate(std::integral_constant<int, UMAX>{});
    }
    const float inv = nsum ? 1.0f / L : 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] = o[j] * inv * P.v_scale;
  }
  if (P.out_bf16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(P.out) + (int64_t)r * P.out_stride + (int64_t)h * D + PER * l;
#pragma unroll
    for (int j = 0; j < PER; ++j) dst[j] = (uint16_t)f32_to_bf16_bits(o[j]);
  } else {
    float* dst = reinterpret_cast<float*>(P.out) + (int64_t)r * P.out_stride + (int64_t)h * D + PER * l;
#pragma unroll
    for (int j = 0; j < PER; ++j) dst[j] = o[j];
  }
}

// ------------------------------------------------------------------ append
// One wave per (row, kv head); every append lands before the attention
// kernel that follows on the stream reads the pool.
template <int KVT, int D>
__global__ __launch_bounds__(64) void append_kernel(AttnParams P) {
  const int r = blockIdx.x / P.n_kv, g = blockIdx.x % P.n_kv;
  const int s = P.seq[r], p = P.pos[r];
  const int count = seq_count(P, s);
  if (!row_ok(P, s, p, count, g == 0)) return;
  const int page = P.table[(int64_t)s * P.max_pages + p / kPage];
  if ((unsigned)page >= (unsigned)P.num_pages) {  // not written; the attention kernel refuses the row
    if (g == 0 && lane_id() == 0) atomicOr(P.err, kErrPage);
    return;
  }
  NewToken<KVT, D> nt;
  append_load<KVT, D>(P, r, g, nt);
  append_store<KVT, D>(P, g, page, p % kPage, nt);
}

// ------------------------------------------------------------------ host
struct AttnWs {
  float* part_ml;
  float* part_o;
};

static bool chunked(const pkd_pool* pool) {
  return pool->desc.attn_chunk_pages < pool->desc.max_pages_per_seq;
}

static size_t max_units(const pkd_pool* pool, int32_t rows) {
  const int64_t per = (pool->desc.max_pages_per_seq + pool->desc.attn_chunk_pages - 1) / pool->desc.attn_chunk_pages;
  return (size_t)rows * (size_t)per;
}

static size_t carve(const pkd_pool* pool, int32_t n_q_heads, int32_t rows, uint8_t* base, AttnWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  if (!chunked(pool)) {
    if (w) *w = AttnWs{};
    return 0;
  }
  const int G = n_q_heads / pool->desc.num_kv_heads;
  const size_t units = max_units(pool, rows) * pool->desc.num_kv_heads * G;
  AttnWs t;
  t.part_ml = (float*)take(sizeof(float) * 2 * units);
  t.part_o = (float*)take(sizeof(float) * (size_t)pool->desc.head_dim * units);
  if (w) *w = t;
  return off;
}

size_t attn_workspace_bytes(const pkd_pool* pool, int32_t n_q_heads, int32_t max_rows) {
  if (!pool || max_rows < 0 || n_q_heads <= 0) return 0;
  return carve(pool, n_q_heads, max_rows, nullptr, nullptr);
}

// Rows per shared tile: the largest power of two whose rows x G query heads
// fit the tile's columns (0: no tiles).  A power of two keeps a slice that
// starts at an aligned row (after a batch of decode rows) on the tile grid.
template <int KVT, int D>
static int tile_rows_cfg(int G) {
  int T = 0;
  for (int t = 2; t * G <= TileCfg<KVT, D>::COLS && t <= kWave; t *= 2) T = t;
  return T;
}

static int tile_rows_for(int kvt, int D, int G) {
  if (D == 128) return kvt == PKD_F32 ? tile_rows_cfg<0, 128>(G) : kvt == PKD_BF16 ? tile_rows_cfg<1, 128>(G)
                                                                                   : tile_rows_cfg<2, 128>(G);
  return kvt == PKD_F32 ? tile_rows_cfg<0, 64>(G) : kvt == PKD_BF16 ? tile_rows_cfg<1, 64>(G) : tile_rows_cfg<2, 64>(G);
}

// The ordered merge, one wave per (row, query head): records requested 16 at a
// time on pools whose rows may have more than 12 chunks, 4 otherwise.
template <int D>
static void launch_merge(const AttnParams& P, int waves, hipStream_t st) {
  if (P.max_ch > 12) hipLaunchKernelGGL((attn_merge_kernel<D, 16>), dim3(waves), dim3(64), 0, st, P);
  else hipLaunchKernelGGL((attn_merge_kernel<D, 4>), dim3(waves), dim3(64), 0, st, P);
}

template <int KVT, int D>
static void launch_all(const AttnParams& P, const AttnArgs& a, const AttnWs& w, int n_kv, bool chunk, int n_ch,
                       bool stage, hipStream_t st) {
  const int units = a.n_rows * n_kv;
  const dim3 tiles((a.n_rows + 3) / 4, n_kv);  // direct mode, staging: four rows of one kv head per workgroup
  const dim3 quads((units + 3) / 4);          // direct mode: four (row, kv head) units per workgroup
  if (!chunk && a.k_new && a.distinct) {
    if (stage) hipLaunchKernelGGL((attn_direct_kernel<KVT, D, true, true>), tiles, dim3(256), 0, st, P);
    else hipLaunchKernelGGL((attn_direct_kernel<KVT, D, true, false>), quads, dim3(256), 0, st, P);
    return;
  }
  const unsigned chunk_wg = (unsigned)(a.n_rows * n_ch * ((n_kv + 3) / 4));  // chunked_unit's workgroups
  if (chunk && a.k_new && a.distinct) {
    hipLaunchKernelGGL((attn_chunked_kernel<KVT, D, true>), dim3(chunk_wg), dim3(256), 0, st, P);
    launch_merge<D>(P, units * P.G, st);
    return;
  }
  if (a.k_new) hipLaunchKernelGGL((append_kernel<KVT, D>), dim3(units), dim3(64), 0, st, P);
  const int n_tiles = P.tile_rows > 0 ? (a.n_rows + P.tile_rows - 1) / P.tile_rows : 0;
  if (!chunk) {
    if (stage) hipLaunchKernelGGL((attn_direct_kernel<KVT, D, false, true>), tiles, dim3(256), 0, st, P);
    else hipLaunchKernelGGL((attn_direct_kernel<KVT, D, false, false>), quads, dim3(256), 0, st, P);
    return;
  }
  if (n_tiles) {
    const int n_units = n_ch * n_kv, n_tile_wgs = 8 * ((n_units + 7) / 8) * n_tiles;
    hipLaunchKernelGGL((attn_tiles_rows_kernel<KVT, D>), dim3(n_tile_wgs + chunk_wg), dim3(256), 0, st, P,
                       n_tile_wgs, n_tiles, n_units);
  } else {
    hipLaunchKernelGGL((attn_chunked_kernel<KVT, D, false>), dim3(chunk_wg), dim3(256), 0, st, P);
  }
  launch_merge<D>(P, units * P.G, st);
}

pkd_status attn_launch(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err) {
  const pkd_pool* pool = a.pool;
  const pkd_pool_desc& d = pool->desc;
  if (a.n_rows == 0) return ok(err);
  const size_t need = carve(pool, a.n_q_heads, a.n_rows, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)(ws ? ws_bytes : 0),
                "attention workspace too small: need %zu bytes", need);
  if (need > 0 && ((uintptr_t)ws & 255))
    return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "workspace must be 256-byte aligned");
  AttnWs w;
  carve(pool, a.n_q_heads, a.n_rows, (uint8_t*)ws, &w);
  AttnParams P{};
  P.pages = pool->base + pool->info.pages_offset;
  P.block_bytes = (uint32_t)pool->info.block_bytes;
  P.page_stride = (uint64_t)d.num_kv_heads * 2 * pool->info.block_bytes;
  P.table = (const int32_t*)(pool->base + pool->info.table_offset);
  P.counts = (const int32_t*)(pool->base + pool->info.counts_offset);
  P.max_pages = d.max_pages_per_seq;
  P.max_seqs = d.max_seqs;
  P.num_pages = d.num_pages;
  P.err = (uint32_t*)(pool->base + pool->info.error_offset);
  P.seq = a.seq;
  P.pos = a.pos;
  P.n_rows = a.n_rows;
  P.n_kv = d.num_kv_heads;
  P.G = a.n_q_heads / d.num_kv_heads;
  P.q = a.q;
  P.q_stride = a.q_stride;
  P.out = a.out;
  P.out_bf16 = a.out_dtype == PKD_BF16;
  P.out_stride = a.out_stride;
  P.qk_scale = (float)(1.4426950408889634 / sqrt((double)d.head_dim)) * d.k_scale;
  P.v_scale = d.v_scale;
  P.chunk_pages = d.attn_chunk_pages;
  P.part_ml = w.part_ml;
  P.part_o = w.part_o;
  P.new_k = a.k_new;
  P.new_v = a.v_new;
  P.new_stride = a.kv_new_stride;
  P.enc_k_scale = d.k_scale;
  P.enc_v_scale = d.v_scale;
  const bool ch = chunked(pool);
  const int kvt = d.kv_dtype;
  const int n_ch = ch ? (d.max_pages_per_seq + d.attn_chunk_pages - 1) / d.attn_chunk_pages : 1;
  P.max_ch = n_ch;
  // Shared tiles run on chunked pools (the page chunks give a tile's pages
  // parallelism, and the merge takes their records) in calls of at least
  // kTileMinRows rows: below that they were no faster (16- to 64-row slices of
  // a 7B-shaped layer: 2 us slower at position 1024, 3 us faster at 2304).  A
  // pure decode batch has no two rows of one sequence.
  constexpr int kTileMinRows = 128;
  P.tile_rows = (a.distinct || !ch || a.n_rows < kTileMinRows) ? 0 : tile_rows_for(kvt, d.head_dim, P.G);
  // leading-page staging only where some page is listed by two sequences
  const bool stage = pool->shared_pages > 0;
  if (d.head_dim == 128) {
    if (kvt == PKD_F32) launch_all<0, 128>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
    else if (kvt == PKD_BF16) launch_all<1, 128>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
    else launch_all<2, 128>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
  } else {
    if (kvt == PKD_F32) launch_all<0, 64>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
    else if (kvt == PKD_BF16) launch_all<1, 64>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
    else launch_all<2, 64>(P, a, w, d.num_kv_heads, ch, n_ch, stage, stream);
  }
  return check_launch(err, "paged attention");
}

}  // namespace pkd
