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
// Workgroup tile: 256 weight rows x 128 activation rows, eight waves of
// 64 x 64 (4 x 4 matrix-core tiles of 16 x 16; two waves per SIMD so that one
// wave's LDS and memory waits overlap the other's products), k-tile of 128
// bytes per row.
// LDS holds [256 weight rows; 128 activation rows] x 128 bytes per stage with
// an XOR swizzle of the 16-byte chunks (row r, chunk c at c ^ (r & 7)), so the
// operand reads of a wave hit distinct banks.
//   mode 0 (bf16) and mode 2 (native fp8): three stages fed by direct
//     global-to-LDS loads (global_load_lds_dwordx4), waited on explicitly;
//   mode 1 (fp8 decoded to bf16): the codes pass through registers, are widened
//     exactly to bf16 and stored; two stages.
// The k-loop order is fixed; a row's outputs never depend on which rows share
// its tile.  With k_splits S > 1 each tile's K range is cut into S fixed parts
// whose fp32 partial sums a second kernel adds in ascending order, so results
// depend on S (a per-matrix constant) but never on the batch.  Work items are
// dealt so that an XCD runs a contiguous run of tiles sharing a weight block.

#include "common.h"

namespace pkd {

struct GemmParams {
  const uint8_t* W;      // [N][K] codes
  const uint8_t* X;      // [M][K] codes (bf16 or fp8)
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
  int32_t splits;
  float* partial;  // splits > 1: [splits][M][N] raw fp32 sums
};

constexpr int TN = 256, TM = 128, TKB = 128;   // tile rows, k-tile bytes per LDS row
constexpr int ROWS = TN + TM;                  // LDS rows per stage
constexpr int STAGE_BYTES = ROWS * TKB;        // 48 KiB
constexpr int NWAVES = 8;
constexpr int DMA_PER_WAVE = STAGE_BYTES / 1024 / NWAVES;  // 6 wave loads of 1 KiB each

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
#define PKD_VMCNT(n) (0x0F70 | ((n) & 0xF) | (((n) & 0x30) << 10))

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// 16 bytes land at lds + 16 l (lds is wave-uniform).  The host compilation
// pass never sees the device builtin.
__device__ __forceinline__ void lds_dma16(const void* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#else
  (void)g;
  (void)lds;
#endif
}

// Workgroup barrier that no memory access may cross in either direction (the
// compiler cannot see the LDS writes of the direct loads, so an intrinsic
// barrier alone would let it hoist LDS reads above it).  It waits for nothing
// by itself: the vmcnt / lgkmcnt waits around it are explicit.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int swz(int row, int chunk) { return row * TKB + ((chunk ^ (row & 7)) << 4); }

// Global weight row of LDS tile row rho (< TN).  silu: each 64-row quarter of
// the tile (one wave's rows) is 32 gate rows followed by the 32 matching up rows.
__device__ __forceinline__ int w_row(const GemmParams& P, int n0, int rho) {
  if (!P.silu) return min(n0 + rho, P.N - 1);
  const int F = P.N / 2, j0 = n0 / 2, wn = rho >> 6, q = rho & 63;
  const int j = min(j0 + 32 * wn + (q & 31), F - 1);
  return q < 32 ? j : F + j;
}

__device__ __forceinline__ const uint8_t* row_ptr(const GemmParams& P, int n0, int m0, int rho, int64_t kbytes) {
  if (rho < TN) return P.W + (int64_t)w_row(P, n0, rho) * kbytes;
  return P.X + (int64_t)min(m0 + rho - TN, P.M - 1) * kbytes;
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool NATIVE8 = MODE == 2;
  constexpr int STAGES = MODE == 1 ? 2 : 3;
  // work item -> (tile n, split, tile m), dealt contiguously per XCD
  const int items = P.tiles_n * P.splits * P.tiles_m;
  const int b = blockIdx.x;
  const int item = (items % 8 == 0) ? (b % 8) * (items / 8) + b / 8 : b;
  const int tm = item % P.tiles_m;
  const int sp = (item / P.tiles_m) % P.splits;
  const int tn = item / (P.tiles_m * P.splits);
  const int n0 = tn * TN, m0 = tm * TM;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, grp = l >> 4, i16 = l & 15;
  const int wn = wave >> 1, wm = wave & 1;  // wn 0..3 (64 weight rows), wm 0..1 (64 activation rows)
  const int64_t kbytes = MODE == 0 ? 2 * (int64_t)P.K : P.K;  // HBM bytes per operand row
  const int nk_all = MODE == 2 ? P.K / 128 : P.K / 64;       // k-tiles over the whole K
  const int kt0 = (int)((int64_t)nk_all * sp / P.splits), kt1 = (int)((int64_t)nk_all * (sp + 1) / P.splits);
  const int nk = kt1 - kt0;
  constexpr int KT_BYTES = MODE == 1 ? 64 : TKB;  // HBM bytes per row per k-tile

  // ---- loaders
  // DMA (modes 0, 2): wave w loads 1 KiB blocks 6w .. 6w + 5 of the stage;
  // lane l lands at block + 16 l = row 8 * block + l / 8, swizzled chunk l % 8,
  // so it reads global chunk (l % 8) ^ (l / 8) of that row.
  const uint8_t* dsrc[MODE == 1 ? 1 : DMA_PER_WAVE];
  // register path (mode 1): thread t moves fp8 chunks q = t + 512 j (j < 3),
  // row q / 4, 16-byte chunk q % 4 of the 64-byte k-tile.
  constexpr int NR = 3;
  const uint8_t* rsrc[MODE == 1 ? NR : 1];
  if constexpr (MODE != 1) {
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int rho = 8 * (DMA_PER_WAVE * wave + i) + (l >> 3);
      const int c = (l & 7) ^ (l >> 3);
      dsrc[i] = row_ptr(P, n0, m0, rho, kbytes) + (int64_t)kt0 * KT_BYTES + 16 * c;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int q = t + 512 * j;
      rsrc[j] = row_ptr(P, n0, m0, q >> 2, kbytes) + (int64_t)kt0 * KT_BYTES + 16 * (q & 3);
    }
  }
  auto dma_issue = [&](int kt) {  // stage kt (local index) into buffer kt % STAGES
    uint8_t* base = smem + (kt % STAGES) * STAGE_BYTES + DMA_PER_WAVE * 1024 * wave;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      lds_dma16(dsrc[i] + (int64_t)kt * KT_BYTES, base + 1024 * i);
  };
  u32x4 rr[NR];
  auto reg_load = [&](int kt) {
#pragma unroll
    for (int j = 0; j < NR; ++j) rr[j] = *reinterpret_cast<const u32x4*>(rsrc[j] + (int64_t)kt * KT_BYTES);
  };
  auto reg_store = [&](int buf) {
    uint8_t* s = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int q = t + 512 * j, rho = q >> 2, c = q & 3;
      const u32x2 a0 = fp8x4_to_bf16x4(rr[j].x), a1 = fp8x4_to_bf16x4(rr[j].y);
      const u32x2 a2 = fp8x4_to_bf16x4(rr[j].z), a3 = fp8x4_to_bf16x4(rr[j].w);
      *reinterpret_cast<u32x4*>(s + swz(rho, 2 * c)) = u32x4{a0.x, a0.y, a1.x, a1.y};
      *reinterpret_cast<u32x4*>(s + swz(rho, 2 * c + 1)) = u32x4{a2.x, a2.y, a3.x, a3.y};
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Operands of one k-tile in two halves.  bf16: half h = k-step h (4 weight
  // and 4 activation tiles).  Native fp8 (one 128-wide k-step): half 0 = the 4
  // activation tiles and weight tiles 0..1, half 1 = weight tiles 2..3.
  // Registers: ob[h][0..3] weight operands, ob[h][4..7] activation operands.
  u32x4 ob[2][8];
  u32x4 oc[2][8];  // second dword-quad of each native fp8 operand (32 bytes per lane)
  auto read_half = [&](const uint8_t* s, int h) {
    const uint8_t* w = s;
    const uint8_t* x = s + TN * TKB;
    if constexpr (!NATIVE8) {
#pragma unroll
      for (int a = 0; a < 4; ++a) ob[h][a] = *reinterpret_cast<const u32x4*>(w + swz(wn * 64 + 16 * a + i16, 4 * h + grp));
#pragma unroll
      for (int c = 0; c < 4; ++c) ob[h][4 + c] = *reinterpret_cast<const u32x4*>(x + swz(wm * 64 + 16 * c + i16, 4 * h + grp));
    } else {
      if (h == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int row = wm * 64 + 16 * c + i16;
          ob[0][4 + c] = *reinterpret_cast<const u32x4*>(x + swz(row, 2 * grp));
          oc[0][4 + c] = *reinterpret_cast<const u32x4*>(x + swz(row, 2 * grp + 1));
        }
      } else {
        // half 1 keeps its own copy of the tile's activation operands: the
        // next tile's half-0 reads overwrite ob[0] before half 1 runs
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ob[1][4 + c] = ob[0][4 + c];
          oc[1][4 + c] = oc[0][4 + c];
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int row = wn * 64 + 16 * (2 * h + a) + i16;
        ob[h][a] = *reinterpret_cast<const u32x4*>(w + swz(row, 2 * grp));
        oc[h][a] = *reinterpret_cast<const u32x4*>(w + swz(row, 2 * grp + 1));
      }
    }
  };
  auto mfma_half = [&](int h) {
    if constexpr (!NATIVE8) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ob[h][a]),
                                                              __builtin_bit_cast(bf16x8_t, ob[h][4 + c]), acc[a][c], 0, 0, 0);
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 wl = ob[h][a], wh = oc[h][a], xl = ob[h][4 + c], xh = oc[h][4 + c];
          const i32x8_t wo = {(int)wl.x, (int)wl.y, (int)wl.z, (int)wl.w, (int)wh.x, (int)wh.y, (int)wh.z, (int)wh.w};
          const i32x8_t xo = {(int)xl.x, (int)xl.y, (int)xl.z, (int)xl.w, (int)xh.x, (int)xh.y, (int)xh.z, (int)xh.w};
          acc[2 * h + a][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wo, xo, acc[2 * h + a][c], 0, 0, 0, 127, 0, 127);
        }
    }
  };

  // mode 1 keeps a single-phase compute over the LDS stage
  auto compute_simple = [&](const uint8_t* s) {
    read_half(s, 0);
    read_half(s, 1);
    mfma_half(0);
    mfma_half(1);
  };

  if constexpr (MODE != 1) {
    const int pre = nk < STAGES ? nk : STAGES;
    for (int kt = 0; kt < pre; ++kt) dma_issue(kt);
    // stage 0 landed: at most the loads of stages 1 .. pre - 1 remain
    if (pre == 3) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(2 * DMA_PER_WAVE));
    else if (pre == 2) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(DMA_PER_WAVE));
    else __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
    lds_barrier();
    if (nk > 0) read_half(smem, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* cur = smem + (kt % STAGES) * STAGE_BYTES;
      const uint8_t* nxt = smem + ((kt + 1) % STAGES) * STAGE_BYTES;
      // [A] second-half reads of tile kt under the first-half products
      read_half(cur, 1);
      mfma_half(0);
      // [B] this wave's reads of tile kt are done and tile kt + 1 has landed
      wait_lds_reads();
      if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(DMA_PER_WAVE));
      else __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
      lds_barrier();
      // [C] refill the buffer of tile kt with tile kt + 3
      if (kt + 3 < nk) dma_issue(kt + 3);
      // [D] first-half reads of tile kt + 1 under the second-half products of tile kt
      read_half(nxt, 0);
      mfma_half(1);
      // keep the prefetched operands in registers across the loop edge (the
      // compiler would otherwise re-read them after the next barrier)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        asm volatile("" : "+v"(ob[0][i]));
        if constexpr (NATIVE8) asm volatile("" : "+v"(oc[0][i]));
      }
    }
  } else {
    if (nk > 0) {
      reg_load(0);
      reg_store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) reg_load(kt + 1);
      compute_simple(smem + (kt & 1) * STAGE_BYTES);
      if (kt + 1 < nk) reg_store((kt + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds outputs n = n0 + wn*64 + 16a + 4grp + i of activation row
  // m = m0 + wm*64 + 16c + i16
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int m = m0 + wm * 64 + 16 * c + i16;
    if (m >= P.M) continue;
    if (P.splits > 1) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (!P.silu) {
          const int n = n0 + wn * 64 + 16 * a + 4 * grp;
          if (n < P.N) *reinterpret_cast<f32x4_t*>(P.partial + ((int64_t)sp * P.M + m) * P.N + n) = acc[a][c];
        } else {
          // raw gate / up sums at their weight rows j and F + j
          const int F = P.N / 2;
          const int j = n0 / 2 + wn * 32 + 16 * (a & 1) + 4 * grp;
          if (j < F) {
            const int nn = a < 2 ? j : F + j;
            *reinterpret_cast<f32x4_t*>(P.partial + ((int64_t)sp * P.M + m) * P.N + nn) = acc[a][c];
          }
        }
      }
      continue;
    }
    const float rs = MODE != 0 ? P.x_scale[m] * P.w_scale : P.w_scale;
    if (!P.silu) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * 64 + 16 * a + 4 * grp;
        if (n >= P.N) continue;
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
        if (j >= P.n_out) continue;
        const f32x4_t g = acc[a][c] * rs, u = acc[a + 2][c] * rs;
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

// Split-K finish: adds the S partial sums of each output in ascending split
// order, then applies the same epilogue as the single-pass kernel.  One thread
// per 4 consecutive outputs.
template <bool FP8IN>
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmParams P) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 4 outputs
  const int64_t groups = (int64_t)P.M * (P.n_out / 4);
  if (q >= groups) return;
  const int m = (int)(q / (P.n_out / 4));
  const int n = (int)(q % (P.n_out / 4)) * 4;
  const float rs = FP8IN ? P.x_scale[m] * P.w_scale : P.w_scale;
  const int F = P.N / 2;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < P.splits; ++sp) {
    const float* base = P.partial + ((int64_t)sp * P.M + m) * P.N;
    s += *reinterpret_cast<const f32x4_t*>(base + n);
    if (P.silu) su += *reinterpret_cast<const f32x4_t*>(base + F + n);
  }
  f32x4_t v;
  if (P.silu) {
    const f32x4_t g = s * rs, u = su * rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = g[i] / (1.0f + __expf(-g[i])) * u[i];
  } else {
    v = s * rs;
    if (P.residual) v += *reinterpret_cast<const f32x4_t*>(P.residual + (int64_t)m * P.n_out + n);
  }
  if (P.y_bf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(P.y) + (int64_t)m * P.y_stride + n;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(P.y) + (int64_t)m * P.y_stride + n) = v;
  }
  if (P.y2) *reinterpret_cast<u32x2*>(P.y2 + (int64_t)m * P.n_out + n) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
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

static int splits_of(const pkd_matrix* W) { return W->k_splits > 1 ? W->k_splits : 1; }

size_t proj_workspace_bytes(const pkd_matrix* W, int32_t max_rows) {
  if (!W || max_rows <= 0 || W->family == PKD_FAMILY_GEMV) return 0;
  size_t b = 0;
  if (W->dtype == PKD_FP8_E4M3) b += align256((size_t)max_rows * W->cols) + align256(sizeof(float) * (size_t)max_rows);
  if (splits_of(W) > 1) b += align256(sizeof(float) * (size_t)splits_of(W) * max_rows * W->rows);
  return b;
}

pkd_status gemv_launch(const ProjArgs& a, hipStream_t stream, pkd_error* err);

static bool lds_ready = false;

pkd_status proj_launch(const ProjArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err) {
  const pkd_matrix& W = *a.W;
  if (a.n_rows == 0) return ok(err);
  if (W.family == PKD_FAMILY_GEMV) return gemv_launch(a, stream, err);
  const size_t need = proj_workspace_bytes(a.W, a.n_rows);
  if (need && (!ws || ws_bytes < need))
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)(ws ? ws_bytes : 0),
                "projection workspace too small: need %zu bytes", need);
  if (need && ((uintptr_t)ws & 255)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "workspace must be 256-byte aligned");
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
  P.tiles_n = (W.rows + TN - 1) / TN;
  P.tiles_m = (a.n_rows + TM - 1) / TM;
  P.splits = splits_of(a.W);
  const bool fp8 = W.dtype == PKD_FP8_E4M3;
  const int mode = !fp8 ? 0 : (W.family == PKD_FAMILY_MFMA_FP8 ? 2 : 1);
  uint8_t* wsp = (uint8_t*)ws;
  if (fp8) {
    uint8_t* codes = wsp;
    float* scales = (float*)(wsp + align256((size_t)a.n_rows * W.cols));
    wsp += align256((size_t)a.n_rows * W.cols) + align256(sizeof(float) * (size_t)a.n_rows);
    if (a.x_dtype == PKD_F32)
      hipLaunchKernelGGL(act_quant_kernel<0>, dim3(a.n_rows), dim3(256), 0, stream, a.x, W.cols, codes, scales);
    else
      hipLaunchKernelGGL(act_quant_kernel<1>, dim3(a.n_rows), dim3(256), 0, stream, a.x, W.cols, codes, scales);
    P.X = codes;
    P.x_scale = scales;
  } else {
    P.X = (const uint8_t*)a.x;
  }
  P.partial = P.splits > 1 ? (float*)wsp : nullptr;
  if (!lds_ready) {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 3 * STAGE_BYTES);
    (void)hipFuncSetAttribute((const void*)gemm_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE_BYTES);
    (void)hipFuncSetAttribute((const void*)gemm_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, 3 * STAGE_BYTES);
    lds_ready = true;
  }
  const int grid = P.tiles_n * P.splits * P.tiles_m;
  if (mode == 0) hipLaunchKernelGGL(gemm_kernel<0>, dim3(grid), dim3(64 * NWAVES), 3 * STAGE_BYTES, stream, P);
  else if (mode == 1) hipLaunchKernelGGL(gemm_kernel<1>, dim3(grid), dim3(64 * NWAVES), 2 * STAGE_BYTES, stream, P);
  else hipLaunchKernelGGL(gemm_kernel<2>, dim3(grid), dim3(64 * NWAVES), 3 * STAGE_BYTES, stream, P);
  if (P.splits > 1) {
    const int64_t groups = (int64_t)P.M * (P.n_out / 4);
    const unsigned blocks = (unsigned)((groups + 255) / 256);
    if (fp8) hipLaunchKernelGGL(splitk_finish_kernel<true>, dim3(blocks), dim3(256), 0, stream, P);
    else hipLaunchKernelGGL(splitk_finish_kernel<false>, dim3(blocks), dim3(256), 0, stream, P);
  }
  return check_launch(err, "matrix-core projection");
}

}  // namespace pkd
