// Weight matrix-vector products for decode batches (vector ALU, fp32 accumulate).
//
// At decode batch sizes a projection reads every weight once per step, so its
// speed is the speed at which the weight rows stream in from HBM ("llm-rs",
// section 2); the small-matvec speed is set by how a row maps onto the lanes
// and onto memory transactions (section 3), which the one-warp-per-output-row
// kernel of section 4 addresses.  Here: one 64-lane wavefront owns NR weight
// rows; lane l reads the 16-byte vectors l, l + 64, l + 128, ... of each row,
// so every load instruction of the wave is one contiguous 1 KiB run.  The R
// activation rows of the launch are held in registers per k-vector and each
// weight is used R times from its register ("GPU inference engine
// engineering", section "The same bits in any batch": register-tiled
// projections).  Each output is a lane-sequential fp32 sum over its k-vectors
// followed by a butterfly over the 64 lanes whose tree (pairs at distance 32,
// 16, 8, 4, 2, 1) is the same for every R, so the result of an activation row
// does not depend on how many rows share the launch.  Matrices with few rows
// (fewer than ~8K waves' worth) split K over the four waves of a block: wave w
// takes the 1 KiB runs w, w + 4, w + 8, ... of each row and the four partial
// sums are added through LDS in the order w = 0, 1, 2, 3.  The split is a
// function of the matrix shape only, so it never varies with the batch.

#include "common.h"

namespace pkd {

struct GemvParams {
  const uint8_t* W;
  int32_t rows;  // weight rows (outputs; 2F with silu)
  int32_t cols;
  float w_scale;
  const uint8_t* x;
  int64_t x_stride;  // elements
  int32_t n_rows;
  void* y;
  int32_t y_bf16;
  int64_t y_stride;  // elements
  const float* residual;
  uint16_t* y2;  // optional bf16 copy
  int32_t n_out;  // outputs per activation row (rows, or rows / 2 with silu)
  const float* row_scale;  // optional per-row factor (a norm's 1/rms)
  const float* rope_cs;    // optional rotary table [n_rows][rope_hd / 2][2]
  int32_t rope_cols;
  int32_t rope_hd;
  // Gathered rows: activation row r evaluates only the weight rows
  // cand[r][0 .. n_cand[r]) (y is then [n_rows][max_cand] f32).
  const int32_t* cand;
  const int32_t* n_cand;
  int32_t max_cand;
};

// Element count of one 16-byte weight vector.
template <int WT>
struct WV {
  static constexpr int E = WT == 0 ? 4 : WT == 1 ? 8 : 16;
};

// Decodes one 16-byte weight vector into E floats.
template <int WT>
__device__ __forceinline__ void decode_w(u32x4 v, float* w) {
  if constexpr (WT == 0) {
    w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y);
    w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
  } else if constexpr (WT == 1) {
    unsigned d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[2 * i] = bf16lo(d[i]); w[2 * i + 1] = bf16hi(d[i]); }
  } else {
    unsigned d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2_t a = fp8x2_to_f32(d[i], false), b = fp8x2_to_f32(d[i], true);
      w[4 * i] = a[0]; w[4 * i + 1] = a[1]; w[4 * i + 2] = b[0]; w[4 * i + 3] = b[1];
    }
  }
}

// Loads E activation values of row r at element k (XT 0: f32, 1: bf16, 3: f32
// rounded to bf16 as loaded).
template <int XT, int E>
__device__ __forceinline__ void load_x(const uint8_t* x, int64_t stride, int r, int k, float* out) {
  if constexpr (XT == 3) {
    const float* p = reinterpret_cast<const float*>(x) + (int64_t)r * stride + k;
#pragma unroll
    for (int i = 0; i < E; i += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p + i);
      const unsigned a = pack_bf16(v[0], v[1]), b = pack_bf16(v[2], v[3]);
      out[i] = bf16lo(a); out[i + 1] = bf16hi(a); out[i + 2] = bf16lo(b); out[i + 3] = bf16hi(b);
    }
  } else if constexpr (XT == 0) {
    const float* p = reinterpret_cast<const float*>(x) + (int64_t)r * stride + k;
#pragma unroll
    for (int i = 0; i < E; i += 4) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(p + i);
      out[i] = v[0]; out[i + 1] = v[1]; out[i + 2] = v[2]; out[i + 3] = v[3];
    }
  } else if constexpr (E == 4) {
    // f32 weights (4 per 16-byte vector) against bf16 activations: 8 bytes
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(x) + (int64_t)r * stride + k);
    out[0] = bf16lo(v.x); out[1] = bf16hi(v.x); out[2] = bf16lo(v.y); out[3] = bf16hi(v.y);
  } else {
    static_assert(E % 8 == 0, "bf16 activations come in 8-element vectors");
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + (int64_t)r * stride + k;
#pragma unroll
    for (int i = 0; i < E; i += 8) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + i);
      unsigned d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) { out[i + 2 * j] = bf16lo(d[j]); out[i + 2 * j + 1] = bf16hi(d[j]); }
    }
  }
}

// Reduces v[0..R) over the 64 lanes; afterwards the lanes whose bits 5..(6 -
// log2 R) spell row j hold that row's total (all four lanes of a group of 4
// when R = 16).  Returns the row this lane holds.
template <int C, int M, int R>
__device__ __forceinline__ void transpose_step(float (&v)[R], int l, int& row) {
  if constexpr (C > 1) {
    const bool b = (l & M) != 0;
#pragma unroll
    for (int j = 0; j < C / 2; ++j) {
      const float send = b ? v[j] : v[C / 2 + j];
      const float recv = shfl_xor(send, M);
      v[j] = (b ? v[C / 2 + j] : v[j]) + recv;
    }
    row = 2 * row + (b ? 1 : 0);
    transpose_step<C / 2, M / 2, R>(v, l, row);
  } else {
#pragma unroll
    for (int m = M; m >= 1; m >>= 1) v[0] += shfl_xor(v[0], m);
  }
}

template <int R>
__device__ __forceinline__ int transpose_reduce(float (&v)[R]) {
  int row = 0;
  transpose_step<R, 32, R>(v, lane_id(), row);
  return row;
}

// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs a, b (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// NR weight rows per row group (SILU: NR / 2 gate rows j and the matching up
// rows F + j), R activation rows per launch tile (blockIdx.y), 4 waves per
// block: 4 row groups (KS = 1) or one row group split over K (KS = 4).
// GATHER (R = 1): the row group's NR outputs are the entries o0 .. o0 + NR of
// the activation row's candidate list, and their weight rows are the listed
// ones; everything else, the summation order included, is the dense path's.
template <int WT, int XT, int R, int NR, bool SILU, int KS, bool GATHER = false>
__global__ __launch_bounds__(256) void gemv_kernel(GemvParams P) {
  static_assert(!GATHER || (R == 1 && !SILU), "gathered rows: one activation row, no silu pair");
  constexpr int E = WV<WT>::E;
  constexpr int NP = SILU ? NR / 2 : NR;  // outputs per row group
  const int wib = threadIdx.x >> 6;
  const int kw = KS == 1 ? 0 : wib;                               // k-slice of this wave
  const int wave = KS == 1 ? blockIdx.x * 4 + wib : blockIdx.x;   // row group
  const int l = lane_id();
  const int o0 = wave * NP;  // first output of this wave
  const int r0 = blockIdx.y * R;
  int n_out = P.n_out;
  if constexpr (GATHER) n_out = min(max(P.n_cand[r0], 0), P.max_cand);
  if (o0 >= n_out) return;  // uniform over the block when KS > 1
  const int F = P.n_out;
  int wrow[NR];
  bool bad[NR];  // gathered index outside the matrix: row 0 is read, NaN is stored
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if constexpr (GATHER) {
      const int j = P.cand[(int64_t)r0 * P.max_cand + min(o0 + i, n_out - 1)];
      bad[i] = j < 0 || j >= P.rows;
      wrow[i] = bad[i] ? 0 : j;
    } else {
      int o = SILU ? (i < NP ? o0 + i : F + o0 + (i - NP)) : o0 + i;
      const int last = SILU ? (i < NP ? F - 1 : 2 * F - 1) : P.rows - 1;
      wrow[i] = min(o, last);  // rows past the end repeat the last row; not stored
      bad[i] = false;
    }
  }
  const int64_t row_bytes = (int64_t)P.cols * (WT == 0 ? 4 : WT == 1 ? 2 : 1);
  const int nvec = P.cols / E;
  float acc[NR][R];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;
  constexpr int U = 4;  // k-vectors per lane in flight per row
  for (int j0 = 64 * kw + l; j0 < nvec; j0 += 64 * KS * U) {
    u32x4 wv[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 64 * KS * u;
#pragma unroll
      for (int i = 0; i < NR; ++i)
        wv[u][i] = j < nvec ? *reinterpret_cast<const u32x4*>(P.W + wrow[i] * row_bytes + 16 * (int64_t)j)
                            : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 64 * KS * u;
      if (j >= nvec) break;
      if constexpr (WT == 1 && (XT == 1 || XT == 3)) {
        // bf16 x bf16: the packed pairs go straight into the dot-2 instruction
        // (exact products, fp32 sums), pairs (0,1), (2,3), (4,5), (6,7) in order
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r0 + r >= P.n_rows) break;
          u32x4 xv;
          if constexpr (XT == 1) {
            xv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(P.x) +
                                                 (int64_t)(r0 + r) * P.x_stride + 8 * j);
          } else {
            const float* xf = reinterpret_cast<const float*>(P.x) + (int64_t)(r0 + r) * P.x_stride + 8 * j;
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(xf), b = *reinterpret_cast<const f32x4_t*>(xf + 4);
            xv = u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
          }
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            float a = acc[i][r];
            a = dot2_bf16(wv[u][i].x, xv.x, a);
            a = dot2_bf16(wv[u][i].y, xv.y, a);
            a = dot2_bf16(wv[u][i].z, xv.z, a);
            a = dot2_bf16(wv[u][i].w, xv.w, a);
            acc[i][r] = a;
          }
        }
        continue;
      }
      float w[NR][E];
#pragma unroll
      for (int i = 0; i < NR; ++i) decode_w<WT>(wv[u][i], w[i]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r0 + r >= P.n_rows) break;  // uniform: rows past the batch keep zero sums
        float xv[E];
        load_x<XT, E>(P.x, P.x_stride, r0 + r, E * j, xv);
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[i][r] = fmaf(w[i][e], xv[e], acc[i][r]);
      }
    }
  }
  int row = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) row = transpose_reduce<R>(acc[i]);
  // one writer lane per activation row: the lane whose low bits are zero
  constexpr int LOG_R = R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : R == 8 ? 3 : 4;
  const bool writer = (l & ((64 >> LOG_R) - 1)) == 0;
  if constexpr (KS > 1) {
    // the four k-slices' partial sums, added in slice order by wave 0
    __shared__ float part[KS][NR][R];
    if (writer) {
#pragma unroll
      for (int i = 0; i < NR; ++i) part[kw][i][row] = acc[i][0];
    }
    __syncthreads();
    if (kw != 0) return;
    if (writer) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        float t = part[0][i][row];
#pragma unroll
        for (int w = 1; w < KS; ++w) t += part[w][i][row];
        acc[i][0] = t;
      }
    }
  }
  const int r = r0 + row;
  if (!writer || r >= P.n_rows) return;
  if constexpr (GATHER) {
    float* y = reinterpret_cast<float*>(P.y) + (int64_t)r * P.max_cand;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (o0 + i >= n_out) break;
      y[o0 + i] = bad[i] ? __builtin_nanf("") : acc[i][0] * P.w_scale;
    }
    return;
  }
  const float rsc = P.row_scale ? P.row_scale[r] : 1.0f;
  float vo[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if constexpr (SILU) {
      float g = acc[i][0] * P.w_scale, u = acc[NP + i][0] * P.w_scale;
      if (P.row_scale) { g *= rsc; u *= rsc; }
      vo[i] = silu(g) * u;
    } else {
      vo[i] = acc[i][0] * P.w_scale;
      if (P.row_scale) vo[i] *= rsc;
    }
  }
  if constexpr (!SILU && NP % 2 == 0) {
    // rotary pairs: o0 is a multiple of 4 and rope_cols of the head width
    if (P.rope_cs && o0 < P.rope_cols) {
#pragma unroll
      for (int i = 0; i < NP; i += 2) rope_pair(P.rope_cs, P.rope_hd, r, o0 + i, vo[i], vo[i + 1]);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int o = o0 + i;
    if (o >= P.n_out) break;
    float v = vo[i];
    if constexpr (!SILU) {
      if (P.residual) v += P.residual[(int64_t)r * P.n_out + o];
    }
    if (P.y_bf16) reinterpret_cast<uint16_t*>(P.y)[(int64_t)r * P.y_stride + o] = (uint16_t)f32_to_bf16_bits(v);
    else reinterpret_cast<float*>(P.y)[(int64_t)r * P.y_stride + o] = v;
    if (P.y2) P.y2[(int64_t)r * P.n_out + o] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// Matrix-core products for bf16 activations with bf16 or fp8 weights.  A row
// group is 16 weight rows (SILU: 8 gate rows and their 8 up rows); one wave
// takes RB row groups and 16 activation rows (rows past the batch are zeros),
// one 16 x 16 x 32 product per row group and 32 k, the RB products sharing the
// activation operand.  The weights go straight from HBM into registers: lane
// (i, g) = (l % 16, l / 16) holds 8 elements of weight row i at k = 32 t + 8 g,
// so one wave load is 16 rows x 64 contiguous bytes (32 for fp8, widened
// exactly to bf16 in registers); the activations are the other operand in the
// same layout.  KS waves of a block (KS > 1: the block holds one wave's row
// groups) split the k-steps into contiguous ranges and add their partial sums
// through LDS in the order 0 .. KS - 1.  A product's column depends only on
// its own activation row and the split only on the matrix shape, so a row's
// result never depends on the batch.  This is the PKD_FAMILY_GEMV_MFMA family:
// the matrix cores keep it near the weight stream up to 16 activation rows per
// pass, where the vector-ALU form is bound by its multiply-adds from about 8,
// but its 64-byte weight runs stream below the vector form's 1 KiB runs at
// batch 1.
// GATHER: one activation row per block column (column 0 of the product), the
// 16 weight rows taken from its candidate list; everything else as dense.
template <int WT, bool SILU, int KS, bool GATHER, int RB>
__global__ __launch_bounds__(KS > 4 ? 64 * KS : 256) void gemv_mfma_kernel(GemvParams P) {
  static_assert(!(GATHER && SILU), "gathered rows: no silu pair");
  static_assert(!GATHER || RB == 1, "gathered rows: one row group per wave");
  constexpr int NW = KS > 4 ? KS : 4;  // waves per block
  constexpr int GPB = NW / KS;         // wave row slots per block
  constexpr int NP = SILU ? 8 : 16;    // outputs per row group
  const int wib = threadIdx.x >> 6, l = lane_id(), i = l & 15, g = l >> 4;
  const int kw = wib % KS;
  const int o0 = (blockIdx.x * GPB + wib / KS) * NP * RB;  // first output of row group 0 of this wave
  int n_out = P.n_out;
  if constexpr (GATHER) n_out = min(max(P.n_cand[blockIdx.y], 0), P.max_cand);
  if (o0 >= n_out) return;  // uniform over the block when KS > 1
  // weight row of lane i in row group b (rows past the end repeat the last one; not stored)
  int wr[RB];
  bool bad = false;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int ob = o0 + b * NP;
    if constexpr (GATHER) {
      const int j = P.cand[(int64_t)blockIdx.y * P.max_cand + min(ob + i, n_out - 1)];
      bad = j < 0 || j >= P.rows;
      wr[b] = bad ? 0 : j;
    } else if constexpr (SILU) {
      wr[b] = i < 8 ? min(ob + i, P.n_out - 1) : P.n_out + min(ob + i - 8, P.n_out - 1);
    } else {
      wr[b] = min(ob + i, P.rows - 1);
    }
  }
  // activation row of lane i (the product's column i)
  const int xr = GATHER ? (i == 0 ? (int)blockIdx.y : -1) : (blockIdx.y * 16 + i < P.n_rows ? blockIdx.y * 16 + i : -1);
  constexpr int WB = WT == 1 ? 16 : 8;  // weight bytes per lane and k-step
  const uint8_t* wp[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) wp[b] = P.W + (int64_t)wr[b] * P.cols * (WT == 1 ? 2 : 1) + WB * g;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(P.x) + (int64_t)(xr < 0 ? 0 : xr) * P.x_stride + 8 * g;
  const int nst = P.cols / 32;
  const int t0 = nst * kw / KS, t1 = nst * (kw + 1) / KS;
  f32x4_t acc[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // k-steps in flight per wave: 6 with two row groups keeps 104 VGPRs, four waves per SIMD
  constexpr int U = RB > 1 ? 6 : 8;
  for (int t = t0; t < t1; t += U) {
    u32x4 wv[U][RB], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u >= t1) break;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if constexpr (WT == 1) {
          wv[u][b] = *reinterpret_cast<const u32x4*>(wp[b] + 64 * (int64_t)(t + u));
        } else {
          const u32x2 c = *reinterpret_cast<const u32x2*>(wp[b] + 32 * (int64_t)(t + u));
          wv[u][b] = u32x4{c.x, c.y, 0u, 0u};
        }
      }
      xv[u] = xr >= 0 ? *reinterpret_cast<const u32x4*>(xp + 32 * (int64_t)(t + u)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u >= t1) break;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        u32x4 a = wv[u][b];
        if constexpr (WT == 2) {
          const u32x2 lo = fp8x4_to_bf16x4(wv[u][b].x), hi = fp8x4_to_bf16x4(wv[u][b].y);
          a = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x8_t, xv[u]), acc[b], 0, 0, 0);
      }
    }
  }
  if constexpr (KS > 1) {
    __shared__ f32x4_t part[KS][RB][64];
#pragma unroll
    for (int b = 0; b < RB; ++b) part[kw][b][l] = acc[b];
    __syncthreads();
    if (kw != 0) return;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      f32x4_t tsum = part[0][b][l];
#pragma unroll
      for (int w = 1; w < KS; ++w) tsum += part[w][b][l];
      acc[b] = tsum;
    }
  }
  // lane (rg, col) holds outputs o0 + NP b + 4 rg + v (v < 4) of activation column col
  const int col = l & 15, rg = l >> 4;
  if constexpr (GATHER) {
    bool bv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) bv[v] = __shfl((int)bad, 4 * rg + v, kWave) != 0;
    if (col != 0) return;
    float* y = reinterpret_cast<float*>(P.y) + (int64_t)blockIdx.y * P.max_cand;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int o = o0 + 4 * rg + v;
      if (o < n_out) y[o] = bv[v] ? __builtin_nanf("") : acc[0][v] * P.w_scale;
    }
    return;
  }
  const int r = blockIdx.y * 16 + col;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    float vo[4];
    int ob;  // first output of this lane in row group b
    if constexpr (SILU) {
      float up[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) up[v] = shfl_xor(acc[b][v], 32);
      if (rg >= 2 || r >= P.n_rows) continue;
      const float rsc = P.row_scale ? P.row_scale[r] : 1.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float gt = acc[b][v] * P.w_scale, u = up[v] * P.w_scale;
        if (P.row_scale) { gt *= rsc; u *= rsc; }
        vo[v] = silu(gt) * u;
      }
      ob = o0 + NP * b + 4 * rg;
    } else {
      if (r >= P.n_rows) continue;
      const float rsc = P.row_scale ? P.row_scale[r] : 1.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        vo[v] = acc[b][v] * P.w_scale;
        if (P.row_scale) vo[v] *= rsc;
      }
      ob = o0 + NP * b + 4 * rg;
      if (P.rope_cs && ob < P.rope_cols) {
        rope_pair(P.rope_cs, P.rope_hd, r, ob, vo[0], vo[1]);
        rope_pair(P.rope_cs, P.rope_hd, r, ob + 2, vo[2], vo[3]);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int o = ob + v;
      if (o >= P.n_out) break;
      float val = vo[v];
      if constexpr (!SILU) {
        if (P.residual) val += P.residual[(int64_t)r * P.n_out + o];
      }
      if (P.y_bf16) reinterpret_cast<uint16_t*>(P.y)[(int64_t)r * P.y_stride + o] = (uint16_t)f32_to_bf16_bits(val);
      else reinterpret_cast<float*>(P.y)[(int64_t)r * P.y_stride + o] = val;
      if (P.y2) P.y2[(int64_t)r * P.n_out + o] = (uint16_t)f32_to_bf16_bits(val);
    }
  }
}

// K split of the matrix-core form: a function of the weight-row count only
// (16-row groups), so a matrix and any gathered subset of its rows split alike.
static int gemv_mfma_k_split(int rows) {
  const int groups = (rows + 15) / 16;
  return groups < 1024 ? 8 : groups < 4096 ? 4 : 1;
}

template <int WT, bool SILU, bool GATHER>
static void launch_mfma(const GemvParams& P, int tiles_y, hipStream_t st) {
  constexpr int NP = SILU ? 8 : 16;
  const int groups = ((GATHER ? P.max_cand : P.n_out) + NP - 1) / NP;
  const int ks = gemv_mfma_k_split(P.rows);
  // Dense matrices with 1,024 or more row groups give each wave two row
  // groups, which share its activation loads.
  constexpr int RB = GATHER ? 1 : 2;
  if (ks == 8)
    hipLaunchKernelGGL((gemv_mfma_kernel<WT, SILU, 8, GATHER, 1>), dim3(groups, tiles_y), dim3(512), 0, st, P);
  else if (ks == 4)
    hipLaunchKernelGGL((gemv_mfma_kernel<WT, SILU, 4, GATHER, RB>), dim3((groups + RB - 1) / RB, tiles_y), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<WT, SILU, 1, GATHER, RB>), dim3((groups + 4 * RB - 1) / (4 * RB), tiles_y), dim3(256), 0, st, P);
}

// K split of a matrix: 4 when its row groups alone would give fewer than
// 8192 waves (a function of the shape, never of the batch).
static int gemv_k_split(int n_out, int np) { return (n_out + np - 1) / np < 8192 ? 4 : 1; }

template <int WT, int XT, int R, bool SILU>
static void launch_r(const GemvParams& P, hipStream_t st) {
  constexpr int NR = 4;
  constexpr int NP = SILU ? NR / 2 : NR;
  const int groups = (P.n_out + NP - 1) / NP;
  if (gemv_k_split(P.n_out, NP) > 1) {
    dim3 grid(groups, (P.n_rows + R - 1) / R);
    hipLaunchKernelGGL((gemv_kernel<WT, XT, R, NR, SILU, 4>), grid, dim3(256), 0, st, P);
  } else {
    dim3 grid((groups + 3) / 4, (P.n_rows + R - 1) / R);
    hipLaunchKernelGGL((gemv_kernel<WT, XT, R, NR, SILU, 1>), grid, dim3(256), 0, st, P);
  }
}

template <int WT, int XT, bool SILU>
static void launch_x(const GemvParams& P, hipStream_t st) {
  const int n = P.n_rows;
  if (n <= 1) launch_r<WT, XT, 1, SILU>(P, st);
  else if (n <= 2) launch_r<WT, XT, 2, SILU>(P, st);
  else if (n <= 4) launch_r<WT, XT, 4, SILU>(P, st);
  else if (n <= 8) launch_r<WT, XT, 8, SILU>(P, st);
  else launch_r<WT, XT, 16, SILU>(P, st);
}

template <int WT>
static void launch_w(const GemvParams& P, int xt, bool silu, hipStream_t st) {
  if (xt == PKD_F32) {
    if (silu) launch_x<WT, 0, true>(P, st); else launch_x<WT, 0, false>(P, st);
  } else if (xt == kXF32AsBf16) {
    if (silu) launch_x<WT, 3, true>(P, st); else launch_x<WT, 3, false>(P, st);
  } else {
    if (silu) launch_x<WT, 1, true>(P, st); else launch_x<WT, 1, false>(P, st);
  }
}

template <int WT, int XT>
static void launch_gather(const GemvParams& P, hipStream_t st) {
  constexpr int NR = 4;
  const int groups = (P.max_cand + NR - 1) / NR;
  // the dense head's K split for this shape, so each logit has its bits
  if (gemv_k_split(P.rows, NR) > 1) {
    hipLaunchKernelGGL((gemv_kernel<WT, XT, 1, NR, false, 4, true>), dim3(groups, P.n_rows), dim3(256), 0, st, P);
  } else {
    hipLaunchKernelGGL((gemv_kernel<WT, XT, 1, NR, false, 1, true>), dim3((groups + 3) / 4, P.n_rows), dim3(256), 0,
                       st, P);
  }
}

template <int WT>
static void launch_gather_w(const GemvParams& P, int xt, hipStream_t st) {
  if (xt == PKD_F32) launch_gather<WT, 0>(P, st);
  else launch_gather<WT, 1>(P, st);
}

pkd_status gemv_gather_launch(const pkd_matrix& W, const void* x, int32_t x_dtype, int32_t n_rows,
                              const int32_t* cand, const int32_t* n_cand, int32_t max_cand, float* y,
                              hipStream_t stream, pkd_error* err) {
  GemvParams P{};
  P.W = (const uint8_t*)W.data;
  P.rows = W.rows;
  P.cols = W.cols;
  P.w_scale = W.scale;
  P.x = (const uint8_t*)x;
  P.x_stride = W.cols;
  P.n_rows = n_rows;
  P.y = y;
  P.n_out = W.rows;
  P.y_stride = max_cand;
  P.cand = cand;
  P.n_cand = n_cand;
  P.max_cand = max_cand;
  if (W.family == PKD_FAMILY_GEMV_MFMA && W.dtype == PKD_BF16) launch_mfma<1, false, true>(P, n_rows, stream);
  else if (W.family == PKD_FAMILY_GEMV_MFMA) launch_mfma<2, false, true>(P, n_rows, stream);
  else if (W.dtype == PKD_F32) launch_gather_w<0>(P, x_dtype, stream);
  else if (W.dtype == PKD_BF16) launch_gather_w<1>(P, x_dtype, stream);
  else launch_gather_w<2>(P, x_dtype, stream);
  return check_launch(err, "gemv_gather_rows");
}

pkd_status gemv_launch(const ProjArgs& a, hipStream_t stream, pkd_error* err) {
  const pkd_matrix& W = *a.W;
  GemvParams P{};
  P.W = (const uint8_t*)W.data;
  P.rows = W.rows;
  P.cols = W.cols;
  P.w_scale = W.scale;
  P.x = (const uint8_t*)a.x;
  P.x_stride = W.cols;
  P.n_rows = a.n_rows;
  P.y = a.y;
  P.y_bf16 = a.out_dtype == PKD_BF16;
  P.n_out = a.silu_pair ? W.rows / 2 : W.rows;
  P.y_stride = P.n_out;
  P.residual = a.residual;
  P.y2 = (uint16_t*)a.y_bf16;
  P.row_scale = a.row_scale;
  P.rope_cs = a.rope_cs;
  P.rope_cols = a.rope_cols;
  P.rope_hd = a.rope_hd;
  const bool silu = a.silu_pair != 0;
  const int ty = (a.n_rows + 15) / 16;
  if (W.family == PKD_FAMILY_GEMV_MFMA && W.dtype == PKD_BF16) {
    if (silu) launch_mfma<1, true, false>(P, ty, stream); else launch_mfma<1, false, false>(P, ty, stream);
  } else if (W.family == PKD_FAMILY_GEMV_MFMA) {
    if (silu) launch_mfma<2, true, false>(P, ty, stream); else launch_mfma<2, false, false>(P, ty, stream);
  } else if (W.dtype == PKD_F32) {
    launch_w<0>(P, a.x_dtype, silu, stream);
  } else if (W.dtype == PKD_BF16) {
    launch_w<1>(P, a.x_dtype, silu, stream);
  } else {
    launch_w<2>(P, a.x_dtype, silu, stream);
  }
  return check_launch(err, "gemv_rows");
}

}  // namespace pkd
