// Batched projections on the matrix cores (bf16 and fp8 E4M3), fp32 accumulate.
//
// At large decode batches the projection stops being a matvec: the weights are
// read once for hundreds of rows, the step becomes a dense contraction, and it
// belongs on the matrix cores ("llm-rs", section 5: at large batch decode
// should run on the tensor-core GEMM that prefill uses; "Prefill: tensor
// cores, written by hand": bf16 inputs, fp32 accumulation).  The fp8 tier
// contracts fp8 weights with per-row fp8 activations ("Engines for the card you
// have", section "One checkpoint, many engines").
//
// Tile: 128 weight rows x 128 activation rows per 256-thread workgroup, k-tile
// of 128 bytes per row (64 bf16 or 128 fp8), double-buffered in LDS with an XOR
// swizzle of the 16-byte chunks so that matrix-core operand reads are free of
// bank conflicts.  Four waves, each 64 x 64, as 4 x 4 tiles of 16 x 16.  The
// k-loop order is fixed and a row's outputs never depend on which other rows
// share the tile, so results are batch invariant.  Tiles are assigned so that
// consecutive tiles of one weight block land on the same XCD (shared L2).

#include "common.h"

namespace pkd {

struct GemmParams {
  const uint8_t* W;  // [N][K] codes
  const uint8_t* X;  // [M][K] codes (bf16 or fp8)
  const float* x_scale;  // fp8: [M] per-row scales
  float w_scale;
  int32_t N;  // weight rows
  int32_t M;  // activation rows
  int32_t K;
  int32_t silu;  // W = [W_gate; W_up], N = 2F
  void* y;
  int32_t y_bf16;
  int64_t y_stride;  // elements (outputs per row)
  const float* residual;
  uint16_t* y2;
  int32_t n_out;
  int32_t tiles_n;
  int32_t tiles_m;
};

constexpr int TN = 128, TM = 128, TKB = 128;  // tile rows, k-tile bytes per row
constexpr int TILE_BYTES = TN * TKB;          // one operand tile in LDS

__device__ __forceinline__ int swz(int row, int chunk) { return row * TKB + ((chunk ^ (row & 7)) << 4); }

// Global row of LDS weight-tile row rho (silu: 32 gate rows then the 32 matching
// up rows for each 64-row half).
__device__ __forceinline__ int w_row(const GemmParams& P, int n0, int rho) {
  if (!P.silu) return n0 + rho;
  const int F = P.N / 2, j0 = n0 / 2, wn = rho >> 6, q = rho & 63;
  return q < 32 ? j0 + 32 * wn + q : F + j0 + 32 * wn + (q - 32);
}

// MODE 0: bf16 x bf16.  MODE 1: fp8 codes decoded exactly to bf16 while staged
// into LDS, contracted on the bf16 matrix core (fp32-accurate sums).  MODE 2:
// fp8 codes contracted by the native fp8 matrix-core instruction, whose
// internal sum of each 128 products carries ~17 significant bits.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams P) {
  constexpr bool FP8 = MODE != 0;          // operands stored as fp8 codes
  constexpr bool NATIVE8 = MODE == 2;      // fp8 matrix-core instruction
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // buffer b: weight tile at 2b * TILE_BYTES, activation tile right after it
  // XCD-aware tile order: hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous run of tiles (m fastest, so one weight tile is
  // reused from that XCD's L2).
  const int nt = P.tiles_n * P.tiles_m;
  const int b = blockIdx.x;
  const int tile = (nt % 8 == 0) ? (b % 8) * (nt / 8) + b / 8 : b;
  const int tn = tile / P.tiles_m, tm = tile % P.tiles_m;
  const int n0 = tn * TN, m0 = tm * TM;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, grp = l >> 4, i16 = l & 15;
  const int wn = wave >> 1, wm = wave & 1;
  const int64_t kbytes = FP8 ? P.K : 2 * (int64_t)P.K;  // bytes per operand row in HBM
  // k-tile: 128 bytes per row in LDS = 64 bf16 (modes 0, 1) or 128 fp8 (mode 2)
  const int nk = MODE == 1 ? P.K / 64 : (int)(kbytes / TKB);

  // global -> register staging.  Modes 0 and 2: thread t moves the 16-byte
  // chunk (t % 8) of rows t / 8 + 32 j (j < 4).  Mode 1: the k-tile is 64 fp8
  // bytes per row; thread t moves chunk (t % 4) of rows t / 4 + 64 j (j < 2)
  // and widens it to two bf16 chunks.
  constexpr int NJ = MODE == 1 ? 2 : 4;
  constexpr int RSTEP = MODE == 1 ? 64 : 32;
  constexpr int KT_BYTES = MODE == 1 ? 64 : TKB;  // HBM bytes per row per k-tile
  const int gc = MODE == 1 ? (t & 3) : (t & 7), gr = MODE == 1 ? (t >> 2) : (t >> 3);
  const uint8_t* wsrc[NJ];
  const uint8_t* xsrc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int rho = gr + RSTEP * j;
    wsrc[j] = P.W + (int64_t)w_row(P, n0, rho) * kbytes + 16 * gc;
    const int mr = min(m0 + rho, P.M - 1);
    xsrc[j] = P.X + (int64_t)mr * kbytes + 16 * gc;
  }
  u32x4 rw[NJ], rx[NJ];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      rw[j] = *reinterpret_cast<const u32x4*>(wsrc[j] + (int64_t)kt * KT_BYTES);
      rx[j] = *reinterpret_cast<const u32x4*>(xsrc[j] + (int64_t)kt * KT_BYTES);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sw = smem + 2 * buf * TILE_BYTES;
    uint8_t* sx = sw + TILE_BYTES;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rho = gr + RSTEP * j;
      if constexpr (MODE == 1) {
        const u32x2 w0 = fp8x4_to_bf16x4(rw[j].x), w1 = fp8x4_to_bf16x4(rw[j].y);
        const u32x2 w2 = fp8x4_to_bf16x4(rw[j].z), w3 = fp8x4_to_bf16x4(rw[j].w);
        const u32x2 x0 = fp8x4_to_bf16x4(rx[j].x), x1 = fp8x4_to_bf16x4(rx[j].y);
        const u32x2 x2 = fp8x4_to_bf16x4(rx[j].z), x3 = fp8x4_to_bf16x4(rx[j].w);
        *reinterpret_cast<u32x4*>(sw + swz(rho, 2 * gc)) = u32x4{w0.x, w0.y, w1.x, w1.y};
        *reinterpret_cast<u32x4*>(sw + swz(rho, 2 * gc + 1)) = u32x4{w2.x, w2.y, w3.x, w3.y};
        *reinterpret_cast<u32x4*>(sx + swz(rho, 2 * gc)) = u32x4{x0.x, x0.y, x1.x, x1.y};
        *reinterpret_cast<u32x4*>(sx + swz(rho, 2 * gc + 1)) = u32x4{x2.x, x2.y, x3.x, x3.y};
      } else {
        *reinterpret_cast<u32x4*>(sw + swz(rho, gc)) = rw[j];
        *reinterpret_cast<u32x4*>(sx + swz(rho, gc)) = rx[j];
      }
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* w = smem + 2 * buf * TILE_BYTES;
    const uint8_t* x = w + TILE_BYTES;
    if constexpr (!NATIVE8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t wo[4], xo[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
          wo[a] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(w + swz(wn * 64 + 16 * a + i16, 4 * s + grp)));
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xo[c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(x + swz(wm * 64 + 16 * c + i16, 4 * s + grp)));
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wo[a], xo[c], acc[a][c], 0, 0, 0);
      }
    } else {
      i32x8_t wo[4], xo[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int row = wn * 64 + 16 * a + i16;
        u32x4 lo = *reinterpret_cast<const u32x4*>(w + swz(row, 2 * grp));
        u32x4 hi = *reinterpret_cast<const u32x4*>(w + swz(row, 2 * grp + 1));
        wo[a] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = wm * 64 + 16 * c + i16;
        u32x4 lo = *reinterpret_cast<const u32x4*>(x + swz(row, 2 * grp));
        u32x4 hi = *reinterpret_cast<const u32x4*>(x + swz(row, 2 * grp + 1));
        xo[c] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wo[a], xo[c], acc[a][c], 0, 0, 0, 127, 0, 127);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds outputs n = wn*64 + 16a + 4grp + i of activation row m = wm*64 + 16c + i16
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int m = m0 + wm * 64 + 16 * c + i16;
    if (m >= P.M) continue;
    const float rs = FP8 ? P.x_scale[m] * P.w_scale : P.w_scale;
    if (!P.silu) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * 64 + 16 * a + 4 * grp;
        f32x4_t v = acc[a][c] * rs;
        if (P.residual) v += *reinterpret_cast<const f32x4_t*>(P.residual + (int64_t)m * P.n_out + n);
        if (P.y_bf16) {
          uint16_t* o = reinterpret_cast<uint16_t*>(P.y) + (int64_t)m * P.y_stride + n;
          *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        } else {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(P.y) + (int64_t)m * P.y_stride + n) = v;
        }
        if (P.y2)
          *reinterpret_cast<u32x2*>(P.y2 + (int64_t)m * P.n_out + n) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int j = n0 / 2 + wn * 32 + 16 * a + 4 * grp;
        f32x4_t g = acc[a][c] * rs, u = acc[a + 2][c] * rs;
        f32x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = g[i] / (1.0f + __expf(-g[i])) * u[i];
        if (P.y_bf16) {
          uint16_t* o = reinterpret_cast<uint16_t*>(P.y) + (int64_t)m * P.y_stride + j;
          *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        } else {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(P.y) + (int64_t)m * P.y_stride + j) = v;
        }
        if (P.y2)
          *reinterpret_cast<u32x2*>(P.y2 + (int64_t)m * P.n_out + j) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
  }
}

// Per-row fp8 quantisation of a projection input: s = max|x| / 448 (fp32
// division; 1 for an all-zero row), codes = E4M3 RNE(x / s), saturating.
template <int XT>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* x, int K, uint8_t* codes, float* scales) {
  __shared__ float red[4];
  const int r = blockIdx.x, t = threadIdx.x;
  auto val = [&](int k) -> float {
    if constexpr (XT == 0) return reinterpret_cast<const float*>(x)[(int64_t)r * K + k];
    else return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[(int64_t)r * K + k]);
  };
  float m = 0.f;
  for (int k = t; k < K; k += 256) m = fmaxf(m, fabsf(val(k)));
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m > 0.f ? m / 448.0f : 1.0f;
  if (t == 0) scales[r] = s;
  for (int k = 2 * t; k < K; k += 512) {
    const unsigned c = f32x2_to_fp8x2(val(k) / s, val(k + 1) / s);
    *reinterpret_cast<uint16_t*>(codes + (int64_t)r * K + k) = (uint16_t)c;
  }
}

size_t proj_workspace_bytes(const pkd_matrix* W, int32_t max_rows) {
  if (!W || max_rows <= 0) return 0;
  if (W->family != PKD_FAMILY_GEMV && W->dtype == PKD_FP8_E4M3)
    return align256((size_t)max_rows * W->cols) + align256(sizeof(float) * (size_t)max_rows);
  return 0;
}

pkd_status gemv_launch(const ProjArgs& a, hipStream_t stream, pkd_error* err);

pkd_status proj_launch(const ProjArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err) {
  const pkd_matrix& W = *a.W;
  if (a.n_rows == 0) return ok(err);
  if (W.family == PKD_FAMILY_GEMV) return gemv_launch(a, stream, err);
  GemmParams P{};
  P.W = (const uint8_t*)W.data;
  P.w_scale = W.scale;
  P.N = W.rows;
  P.M = a.n_rows;
  P.K = W.cols;
  P.silu = a.silu_pair;
  P.y = a.y;
  P.y_bf16 = a.out_dtype == PKD_BF16;
  P.n_out = a.silu_pair ? W.rows / 2 : W.rows;
  P.y_stride = P.n_out;
  P.residual = a.residual;
  P.y2 = (uint16_t*)a.y_bf16;
  P.tiles_n = W.rows / TN;
  P.tiles_m = (a.n_rows + TM - 1) / TM;
  const bool fp8 = W.dtype == PKD_FP8_E4M3;
  const int mode = !fp8 ? 0 : (W.family == PKD_FAMILY_MFMA_FP8 ? 2 : 1);
  if (fp8) {
    const size_t need = proj_workspace_bytes(a.W, a.n_rows);
    if (!ws || ws_bytes < need)
      return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)(ws ? ws_bytes : 0),
                  "fp8 projection workspace too small: need %zu bytes", need);
    uint8_t* codes = (uint8_t*)ws;
    float* scales = (float*)((uint8_t*)ws + align256((size_t)a.n_rows * W.cols));
    if (a.x_dtype == PKD_F32)
      hipLaunchKernelGGL(act_quant_kernel<0>, dim3(a.n_rows), dim3(256), 0, stream, a.x, W.cols, codes, scales);
    else
      hipLaunchKernelGGL(act_quant_kernel<1>, dim3(a.n_rows), dim3(256), 0, stream, a.x, W.cols, codes, scales);
    P.X = codes;
    P.x_scale = scales;
  } else {
    P.X = (const uint8_t*)a.x;
  }
  const int grid = P.tiles_n * P.tiles_m;
  const size_t lds = 4 * TILE_BYTES;
  if (mode == 0) hipLaunchKernelGGL(gemm_kernel<0>, dim3(grid), dim3(256), lds, stream, P);
  else if (mode == 1) hipLaunchKernelGGL(gemm_kernel<1>, dim3(grid), dim3(256), lds, stream, P);
  else hipLaunchKernelGGL(gemm_kernel<2>, dim3(grid), dim3(256), lds, stream, P);
  return check_launch(err, "matrix-core projection");
}

}  // namespace pkd
