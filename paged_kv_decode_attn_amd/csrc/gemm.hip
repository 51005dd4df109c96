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
// Workgroup tile: TN = 256 weight rows x TM = 128 or 256 activation rows, k-tile
// of 128 bytes per row, eight waves (two per SIMD, so that one wave's LDS and
// memory waits overlap the other's products).  TM = 256: waves of 128 x 64
// (8 x 4 matrix-core tiles of 16 x 16); bf16 stages in a ring of three 32 KiB
// weight and two 32 KiB activation buffers, native fp8 in two stages of 64
// KiB; TM = 128: waves of 64 x 64, three stages of 48 KiB.  The taller tile
// halves the bytes each CU pulls from L2 per product; the shorter one keeps
// small batches busy.  LDS rows hold 128 bytes with an XOR swizzle of the
// 16-byte chunks (swz), so the operand reads of a wave hit distinct banks.
//   mode 0 (bf16) and mode 2 (native fp8): stages fed by buffer loads that
//     write LDS directly (buffer_load_dwordx4 ... lds), waited on explicitly;
//   mode 1 (fp8 decoded to bf16): the codes pass through registers, are widened
//     exactly to bf16 and stored; two stages.
// The k-loop order is fixed; a row's outputs never depend on which rows share
// its tile.  With k_splits S > 1 each tile's K range is cut into S fixed parts
// whose fp32 partial sums a second kernel adds in ascending order, so results
// depend on S (a per-matrix constant) but never on the batch.  Work items are
// dealt so that an XCD runs a contiguous run of tiles sharing weight blocks
// (in windows of 4 weight units x 8 activation tiles when there are 8 or more).

#include <atomic>

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
  const float* row_scale;  // optional per-row factor (a norm's 1/rms)
  const float* rope_cs;    // optional rotary table [M][rope_hd / 2][2]
  int32_t rope_cols;
  int32_t rope_hd;
};

// Epilogue shared by the single-pass kernel and the split-K finish: scale,
// per-row factor, and (ROPE) rotary pairs on four consecutive outputs
// n .. n + 3, n a multiple of 4.
template <bool ROPE>
__device__ __forceinline__ f32x4_t proj_scale4(const GemmParams& P, f32x4_t acc, float rs, int m, int n) {
  f32x4_t v = acc * rs;
  if (P.row_scale) v *= P.row_scale[m];
  if (ROPE && P.rope_cs && n < P.rope_cols) {
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    rope_pair(P.rope_cs, P.rope_hd, m, n, a0, a1);
    rope_pair(P.rope_cs, P.rope_hd, m, n + 2, a2, a3);
    v = f32x4_t{a0, a1, a2, a3};
  }
  return v;
}

constexpr int TN = 256;  // weight rows per tile
constexpr int NWAVES = 8;
template <int MODE, int TM>
struct Tile {
  // LDS bytes per row and stage: two 32-wide bf16 k-steps (modes 0, 1; mode 1
  // widened from fp8), one 128-wide fp8 k-step (mode 2)
  static constexpr int KB = 128;
  static constexpr int STAGE_BYTES = (TN + TM) * KB;
  static constexpr int STAGES = MODE == 1 ? 2 : (TM == 256 ? 2 : 3);
  // TM = 256 (bf16 and native fp8): the weight part of a stage has three
  // buffers and the activation part two (the weights are requested two stages
  // ahead), 160 KiB, under the two-group schedule.
  static constexpr bool WRING = MODE != 1 && TM == 256;
  static constexpr int LDS_BYTES = WRING ? 3 * TN * KB + 2 * TM * KB : STAGES * STAGE_BYTES;
  static constexpr int DPW = STAGE_BYTES / 1024 / NWAVES;            // 1 KiB wave loads per stage
  static constexpr int RPB = 1024 / KB;                              // LDS rows per 1 KiB block
  static constexpr int MW = TM / 64;                                 // waves along the activation rows
  static constexpr int WN = TN / (NWAVES / MW);                      // weight rows per wave: 128 or 64
  static constexpr int WA = WN / 16;                                 // weight tiles per wave
};

// Byte offset of 16-byte chunk `chunk` of LDS row `row` (rows of KB bytes).
// The XOR spreads the rows that one matrix-core operand read touches over the
// 64 banks: 128-byte rows use row & 7, 64-byte rows (four per 256 bytes) use
// (row >> 2) & 3.  Measured on the card (SQ_LDS_BANK_CONFLICT), a 16-byte
// read serves lanes {0-7, 16-23}, {8-15, 24-31}, {32-39, 48-55} and {40-47,
// 56-63} together.  The bf16 operand reads (lane group g at chunk c + g) are
// conflict-free with row & 7; the native fp8 reads (group g at chunks 2g and
// 2g + 1) were 2-way conflicted with it and are conflict-free with F8: rows
// r and chunks two apart then never share a bank group (the XOR values of
// the four rows of one parity are {0, 1, 4, 5}).
template <int KB, bool F8 = false>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (KB == 128 && F8) return row * 128 + ((chunk ^ ((row & 4) | ((row >> 1) & 1))) << 4);
  else if constexpr (KB == 128) return row * 128 + ((chunk ^ (row & 7)) << 4);
  else return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Global weight row of LDS tile row rho (< TN).  silu: each wave's slab of WN
// rows is WN / 2 gate rows followed by the WN / 2 matching up rows.
template <int WN>
__device__ __forceinline__ int w_row(const GemmParams& P, int n0, int rho) {
  if (!P.silu) return min(n0 + rho, P.N - 1);
  const int F = P.N / 2, j0 = n0 / 2, wn = rho / WN, q = rho % WN;
  const int j = min(j0 + (WN / 2) * wn + q % (WN / 2), F - 1);
  return q < WN / 2 ? j : F + j;
}

template <int WN, int TM>
__device__ __forceinline__ const uint8_t* row_ptr(const GemmParams& P, int n0, int m0, int rho, int64_t kbytes) {
  if (rho < TN) return P.W + (int64_t)w_row<WN>(P, n0, rho) * kbytes;
  return P.X + (int64_t)min(m0 + rho - TN, P.M - 1) * kbytes;
}

template <int MODE, int TM>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmParams P) {
  using T = Tile<MODE, TM>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool NATIVE8 = MODE == 2;
  constexpr int STAGES = T::STAGES, KB = T::KB, RPB = T::RPB;
  constexpr int SB = T::STAGE_BYTES, DPW = T::DPW, WN = T::WN, WA = T::WA;
  // work item -> (tile n, split, tile m), dealt contiguously per XCD
  const int items = P.tiles_n * P.splits * P.tiles_m;
  const int b = blockIdx.x;
  // blocks go to the 8 XCDs round-robin (XCD b % 8); XCD x takes the
  // contiguous items [x base + min(x, rem), ...), one extra for x < rem
  const int base8 = items / 8, rem8 = items % 8, xcd = b % 8;
  const int item = xcd * base8 + min(xcd, rem8) + b / 8;
  // items in order: groups of g weight units u = tn S + sp (the last group
  // possibly shorter), each group's tiles with the unit varying fastest, so
  // that with 8 or more activation tiles the 32 workgroups an XCD runs at once
  // are 4 weight units x 8 activation tiles (12 operand streams, not 18)
  const int units = P.tiles_n * P.splits, g = P.tiles_m >= 8 ? 4 : 1;
  const int grp_i = item / (g * P.tiles_m), r = item % (g * P.tiles_m);
  const int u0 = grp_i * g, gs = min(g, units - u0);
  const int tm = r / gs, u = u0 + r % gs;
  const int sp = u % P.splits;
  const int tn = u / P.splits;
  const int n0 = tn * TN, m0 = tm * TM;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, grp = l >> 4, i16 = l & 15;
  const int wn = wave / T::MW, wm = wave % T::MW;  // weight slab of WN rows, activation slab of 64 rows
  const int64_t kbytes = MODE == 0 ? 2 * (int64_t)P.K : P.K;  // HBM bytes per operand row
  constexpr int KT_BYTES = MODE == 1 ? 64 : KB;             // HBM bytes per row per k-tile
  const int nk_all = (int)(kbytes / KT_BYTES);               // k-tiles over the whole K
  const int kt0 = (int)((int64_t)nk_all * sp / P.splits), kt1 = (int)((int64_t)nk_all * (sp + 1) / P.splits);
  const int nk = kt1 - kt0;

  // ---- loaders
  // LDS buffer loads (modes 0, 2): wave w fills 1 KiB blocks b = DPW w + i of
  // the stage, block b being LDS rows RPB b .. RPB b + RPB - 1; lane l lands
  // at block + 16 l = row RPB b + l / CPR, swizzled chunk l % CPR, so it reads
  // the global chunk that the swizzle puts there.  The lane part of the
  // address is one VGPR; the block's first global row and the k offset are
  // wave-uniform.
  constexpr int CPR = KB / 16;  // 16-byte chunks per LDS row
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = l / CPR, lch = l % CPR;
  const int gch = KB != 128 ? (lch ^ ((lrow >> 2) & 3)) : NATIVE8 ? (lch ^ ((lrow & 4) | ((lrow >> 1) & 1))) : (lch ^ (lrow & 7));
  const uint32_t voff = (uint32_t)(lrow * kbytes + 16 * gch);
  const __amdgpu_buffer_rsrc_t wview = operand_view(P.W, (uint32_t)(P.N * kbytes));
  const __amdgpu_buffer_rsrc_t xview = operand_view(P.X, (uint32_t)(P.M * kbytes));
  // first global row of LDS block b (weight rows below TN, then activation rows)
  auto block_row = [&](int b) -> int {
    const int rho0 = RPB * b;
    if (rho0 >= TN) return m0 + rho0 - TN;
    if (!P.silu) return n0 + rho0;
    const int slab = rho0 / WN, q0 = rho0 % WN;
    const int j = n0 / 2 + (WN / 2) * slab + q0 % (WN / 2);
    return q0 < WN / 2 ? j : P.N / 2 + j;
  };
  // stage kt (local index) into buffer kt % STAGES: this wave's loads i0 .. i1 - 1
  auto dma_part = [&](int kt, int i0, int i1) {
    uint8_t* base = smem + (kt % STAGES) * SB + DPW * 1024 * wave_u;
    const uint32_t koff = (uint32_t)(kt0 + kt) * KT_BYTES;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int b = DPW * wave_u + i;
      const uint32_t soff = (uint32_t)block_row(b) * (uint32_t)kbytes + koff;
      lds_load16(RPB * b < TN ? wview : xview, voff, soff, base + 1024 * i);
    }
  };
  auto dma_issue = [&](int kt) { dma_part(kt, 0, DPW); };
  // register path (mode 1): thread t moves fp8 chunks q = t + 512 j (j < NR),
  // row q / 4, 16-byte chunk q % 4 of the 64-byte k-tile.
  constexpr int NR = (TN + TM) / 128;
  const uint8_t* rsrc[MODE == 1 ? NR : 1];
  if constexpr (MODE == 1) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int q = t + 512 * j;
      rsrc[j] = row_ptr<WN, TM>(P, n0, m0, q >> 2, kbytes) + (int64_t)kt0 * KT_BYTES + 16 * (q & 3);
    }
  }
  u32x4 rr[NR];
  auto reg_load = [&](int kt) {
#pragma unroll
    for (int j = 0; j < NR; ++j) rr[j] = *reinterpret_cast<const u32x4*>(rsrc[j] + (int64_t)kt * KT_BYTES);
  };
  auto reg_store = [&](int buf) {
    uint8_t* s = smem + buf * SB;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int q = t + 512 * j, rho = q >> 2, c = q & 3;
      const u32x2 a0 = fp8x4_to_bf16x4(rr[j].x), a1 = fp8x4_to_bf16x4(rr[j].y);
      const u32x2 a2 = fp8x4_to_bf16x4(rr[j].z), a3 = fp8x4_to_bf16x4(rr[j].w);
      *reinterpret_cast<u32x4*>(s + swz<KB>(rho, 2 * c)) = u32x4{a0.x, a0.y, a1.x, a1.y};
      *reinterpret_cast<u32x4*>(s + swz<KB>(rho, 2 * c + 1)) = u32x4{a2.x, a2.y, a3.x, a3.y};
    }
  };

  f32x4_t acc[WA][4];
#pragma unroll
  for (int a = 0; a < WA; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // bf16 operands of k-step h (of two 32-wide steps per stage): the wave's WA
  // weight tiles and 4 activation tiles, row i16 of each 16-row tile, 16 bytes
  // at k-chunk 4 h + grp.
  auto read_ops2 = [&](const uint8_t* w, const uint8_t* x, int h, u32x4(&wo)[WA], u32x4(&xo)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) xo[c] = *reinterpret_cast<const u32x4*>(x + swz<KB>(wm * 64 + 16 * c + i16, 4 * h + grp));
#pragma unroll
    for (int a = 0; a < WA; ++a) wo[a] = *reinterpret_cast<const u32x4*>(w + swz<KB>(wn * WN + 16 * a + i16, 4 * h + grp));
  };
  // a stage whose activation rows follow its weight rows
  auto read_ops = [&](const uint8_t* s, int h, u32x4(&wo)[WA], u32x4(&xo)[4]) { read_ops2(s, s + TN * KB, h, wo, xo); };
  auto mma = [&](const u32x4(&wo)[WA], const u32x4(&xo)[4]) {
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wo[a]),
                                                            __builtin_bit_cast(bf16x8_t, xo[c]), acc[a][c], 0, 0, 0);
  };
  // Products of one whole LDS stage (the fp8 paths).  Native fp8: one k-step of
  // 128, 32 bytes per lane (k-chunks 2 grp, 2 grp + 1), weight operands taken
  // in two halves to bound the live registers.
  auto compute2 = [&](const uint8_t* w, const uint8_t* x) {
    if constexpr (!NATIVE8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 wo[WA], xo[4];
        read_ops2(w, x, h, wo, xo);
        mma(wo, xo);
      }
    } else {
      i32x8_t xo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = wm * 64 + 16 * c + i16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(x + swz<KB, true>(row, 2 * grp));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(x + swz<KB, true>(row, 2 * grp + 1));
        xo[c] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x8_t wo[WA / 2];
#pragma unroll
        for (int a = 0; a < WA / 2; ++a) {
          const int row = wn * WN + 16 * (h * WA / 2 + a) + i16;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(w + swz<KB, true>(row, 2 * grp));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(w + swz<KB, true>(row, 2 * grp + 1));
          wo[a] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int a = 0; a < WA / 2; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[h * WA / 2 + a][c] =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wo[a], xo[c], acc[h * WA / 2 + a][c], 0, 0, 0, 127, 0, 127);
      }
    }
  };
  auto compute = [&](const uint8_t* s) { compute2(s, s + TN * KB); };

  // wait until at most n later stages' loads of this wave are outstanding
  auto wait_stages = [&](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(PKD_VMCNT(DPW)); break;
      case 2: __builtin_amdgcn_s_waitcnt(PKD_VMCNT(2 * DPW)); break;
      case 3: __builtin_amdgcn_s_waitcnt(PKD_VMCNT(3 * DPW)); break;
      default: __builtin_amdgcn_s_waitcnt(PKD_VMCNT(4 * DPW)); break;
    }
  };

  if constexpr (MODE != 1 && TM == 256) {
    // Two groups of four waves (A = waves 0..3, B = waves 4..7; one of each
    // per SIMD) run half a stage apart: while one wave of a SIMD issues the 64
    // products of a stage back to back, the other reads its operands of the
    // stage from LDS, and at each barrier they swap.  B starts one barrier
    // late; every barrier is shared by both groups.
    //   A: M0 | C0 | M1 | C1 ...      B: - | M0 | C0 | M1 ...
    // M(t) reads stage t into registers; C(t) runs its products (bf16: two
    // 32-wide k-steps; native fp8: one 128-wide k-step).  The weight
    // half of stage t sits in weight buffer t % 3, the activation half in
    // activation buffer t % 2 (3 x 32 + 2 x 32 KiB = 160 KiB).
    // Each wave loads one 64-row quarter of one operand (8 wave loads per
    // stage), at the start of its M phase: A waves the activations of stage
    // t + 1 at M(t), B waves the weights of stage t + 2 at their M(t), each
    // into the buffer of stage t - 1, which both groups finished reading
    // before.  A wave's M phase then issues 8 loads besides its 24 LDS reads,
    // about as long as the other group's products (issuing all 16 loads of a
    // wave in one M phase made that phase the longer one: measured 1,550-1,650
    // clocks against 1,160 for the products).  Activations have two phases to
    // land (A waits at the end of its C(t)); weights, the operand that misses
    // L2, three (B waits for stage t + 1's at the end of its M(t)).
    static_assert(STAGES == 2 && DPW == 8 && T::WRING, "weight ring of three, activation ring of two");
    const bool grp_b = wave_u >= 4;
    const bool w_loader = grp_b;
    const int quarter = wave_u & 3;
    u32x4 wo0[WA], xo0[4], wo1[WA], xo1[4];
    i32x8_t wo8[NATIVE8 ? WA : 1], xo8[NATIVE8 ? 4 : 1];
    constexpr int WBUF = TN * KB, XBUF = TM * KB;
    uint8_t* const wring = smem;
    uint8_t* const xring = smem + 3 * WBUF;
    // A wave's quarter is LDS rows 64 q .. 64 q + 63 of its operand: one run of
    // 64 consecutive global rows (under silu, 64 gate or 64 up rows of a slab)
    // starting at a wave-uniform row.
    const uint32_t run = (uint32_t)block_row(w_loader ? 8 * quarter : TN / RPB + 8 * quarter) * (uint32_t)kbytes;
    const uint32_t blk_stride = 8 * (uint32_t)kbytes;
    const __amdgpu_buffer_rsrc_t aview = w_loader ? wview : xview;
    auto dma_q = [&](int kt) {
      uint8_t* base = (w_loader ? wring + (kt % 3) * WBUF : xring + (kt % 2) * XBUF) + 8 * 1024 * quarter;
      const uint32_t koff = (uint32_t)(kt0 + kt) * KT_BYTES;
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_load16(aview, voff, run + (uint32_t)i * blk_stride + koff, base + 1024 * i);
    };
    // operands of k-step h of stage kt, from the two rings
    auto read_ring = [&](int kt, int h, u32x4(&wo)[WA], u32x4(&xo)[4]) {
      read_ops2(wring + (kt % 3) * WBUF, xring + (kt % 2) * XBUF, h, wo, xo);
    };
    // native fp8: the stage's one 128-wide k-step, 32 bytes per lane and tile
    auto read_ring8 = [&](int kt) {
      const uint8_t* w = wring + (kt % 3) * WBUF;
      const uint8_t* x = xring + (kt % 2) * XBUF;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = wm * 64 + 16 * c + i16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(x + swz<KB, true>(row, 2 * grp));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(x + swz<KB, true>(row, 2 * grp + 1));
        xo8[c] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int a = 0; a < WA; ++a) {
        const int row = wn * WN + 16 * a + i16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(w + swz<KB, true>(row, 2 * grp));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(w + swz<KB, true>(row, 2 * grp + 1));
        wo8[a] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    };
    auto mma8 = [&]() {
#pragma unroll
      for (int a = 0; a < WA; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wo8[a], xo8[c], acc[a][c], 0, 0, 0, 127, 0, 127);
    };
    if (nk > 0) {
      dma_q(0);
      if (w_loader && nk > 1) {
        dma_q(1);
        __builtin_amdgcn_s_waitcnt(PKD_VMCNT(8));
      } else {
        __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
      }
    }
    lds_barrier();
    if (grp_b) lds_barrier();
    // (An L2 prefetch of the weight lines six stages ahead, one dword per lane
    // of each weight loader's run, had made gate/up 3-9% faster while group A
    // issued every load; with the loads split over both groups it made gate/up
    // 4-6% slower at batches 768 and 4,096 and was removed.)
    for (int kt = 0; kt < nk; ++kt) {
      // M(kt)
      const int ahead = w_loader ? kt + 2 : kt + 1;
      const bool issued = ahead < nk;
      if (issued) dma_q(ahead);
      if constexpr (NATIVE8) {
        read_ring8(kt);
      } else {
        read_ring(kt, 0, wo0, xo0);
        read_ring(kt, 1, wo1, xo1);
      }
      wait_lds_reads();
      // B: the weights of stage kt + 1 have landed (stage kt + 2's 8 loads may
      // still be in flight)
      if (w_loader) {
        if (issued) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(8));
        else __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // C(kt)
      if constexpr (NATIVE8) {
        mma8();
      } else {
        mma(wo0, xo0);
        mma(wo1, xo1);
      }
      // A: the activations of stage kt + 1 have landed
      if (!w_loader) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!grp_b) lds_barrier();
  } else if constexpr (MODE == 0) {
    // Ping-pong over the KS = KB / 64 k-steps of each stage: the operands of
    // step g + 1 are read into one register set while the products of step g
    // run on the other, so the matrix core does not wait on LDS.  At a stage
    // boundary, once stage kt + 1 has landed everywhere (one barrier, which
    // also retires every wave's reads of stage kt), stage kt's buffer is
    // refilled with stage kt + STAGES.
    constexpr int KS = KB / 64;
    static_assert(STAGES - 2 <= 4, "wait_stages covers at most four later stages");
    u32x4 w0[WA], x0[4], w1[WA], x1[4];
    const int pre = nk < STAGES ? nk : STAGES;
    for (int kt = 0; kt < pre; ++kt) dma_issue(kt);
    wait_stages(pre - 1);
    lds_barrier();
    if (nk > 0) read_ops(smem, 0, w0, x0);
    const int steps = nk * KS;
    auto step = [&](int g, u32x4(&wc)[WA], u32x4(&xc)[4], u32x4(&wn_)[WA], u32x4(&xn)[4]) {
      const int kt = g / KS, h = g % KS;
      bool refill = false;
      if (h + 1 < KS) {
        read_ops(smem + (kt % STAGES) * SB, h + 1, wn_, xn);
      } else if (kt + 1 < nk) {
        const int later = nk - 2 - kt;
        wait_stages(later < STAGES - 2 ? later : STAGES - 2);
        wait_lds_reads();
        lds_barrier();
        read_ops(smem + ((kt + 1) % STAGES) * SB, 0, wn_, xn);
        refill = kt + STAGES < nk;
      }
      mma(wc, xc);
      // The refill of stage kt's buffer is issued behind the products, half
      // after this boundary step's and half after the next step's (a load
      // issue can stall while the memory pipeline is full; issued before the
      // products, measured 560-870 clocks per stage boundary with the matrix
      // core idle).  Stage order is kept, so the waits above still count
      // whole later stages.
      if (refill) dma_part(kt + STAGES, 0, DPW / 2);
      if (h == 0 && kt > 0 && kt - 1 + STAGES < nk) dma_part(kt - 1 + STAGES, DPW / 2, DPW);
#pragma unroll
      for (int a = 0; a < WA; ++a) asm volatile("" : "+v"(wn_[a]));
#pragma unroll
      for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(xn[c]));
    };
    for (int g = 0; g < steps; g += 2) {
      step(g, w0, x0, w1, x1);
      if (g + 1 < steps) step(g + 1, w1, x1, w0, x0);
    }
  } else if constexpr (MODE == 2) {
    // (128-row fp8 tile) Stages kt .. kt + STAGES - 2 are in flight when tile
    // kt's products start;
    // one barrier per k-tile both publishes tile kt and retires every wave's
    // reads of the buffer that the next load overwrites.
    const int pre = nk < STAGES - 1 ? nk : STAGES - 1;
    for (int kt = 0; kt < pre; ++kt) dma_issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
      // this wave's loads of tile kt are done; later tiles may still be in flight
      if (STAGES == 3 && kt + 1 < nk) __builtin_amdgcn_s_waitcnt(PKD_VMCNT(DPW));
      else __builtin_amdgcn_s_waitcnt(PKD_VMCNT(0));
      wait_lds_reads();
      lds_barrier();
      if (kt + STAGES - 1 < nk) dma_issue(kt + STAGES - 1);
      compute(smem + (kt % STAGES) * SB);
    }
  } else {
    if (nk > 0) {
      reg_load(0);
      reg_store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) reg_load(kt + 1);
      compute(smem + (kt & 1) * SB);
      if (kt + 1 < nk) reg_store((kt + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds outputs n = n0 + wn WN + 16a + 4grp + i of
  // activation row m = m0 + wm 64 + 16c + i16.  silu: weight tiles a < WA / 2
  // are gate rows j = n0 / 2 + wn WN / 2 + 16a + 4grp + i, tile a + WA / 2 the
  // matching up rows.
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int m = m0 + wm * 64 + 16 * c + i16;
    if (m >= P.M) continue;
    if (P.splits > 1) {
#pragma unroll
      for (int a = 0; a < WA; ++a) {
        if (!P.silu) {
          const int n = n0 + wn * WN + 16 * a + 4 * grp;
          if (n < P.N) *reinterpret_cast<f32x4_t*>(P.partial + ((int64_t)sp * P.M + m) * P.N + n) = acc[a][c];
        } else {
          // raw gate / up sums at their weight rows j and F + j
          const int F = P.N / 2;
          const int j = n0 / 2 + wn * (WN / 2) + 16 * (a % (WA / 2)) + 4 * grp;
          if (j < F) {
            const int nn = a < WA / 2 ? j : F + j;
            *reinterpret_cast<f32x4_t*>(P.partial + ((int64_t)sp * P.M + m) * P.N + nn) = acc[a][c];
          }
        }
      }
      continue;
    }
    const float rs = MODE != 0 ? P.x_scale[m] * P.w_scale : P.w_scale;
    if (!P.silu) {
#pragma unroll
      for (int a = 0; a < WA; ++a) {
        const int n = n0 + wn * WN + 16 * a + 4 * grp;
        if (n >= P.N) continue;
        f32x4_t v = proj_scale4<true>(P, acc[a][c], rs, m, n);
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
      for (int a = 0; a < WA / 2; ++a) {
        const int j = n0 / 2 + wn * (WN / 2) + 16 * a + 4 * grp;
        if (j >= P.n_out) continue;
        const f32x4_t g = proj_scale4<false>(P, acc[a][c], rs, m, 0),
                      u = proj_scale4<false>(P, acc[a + WA / 2][c], rs, m, 0);
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
    const f32x4_t g = proj_scale4<false>(P, s, rs, m, 0), u = proj_scale4<false>(P, su, rs, m, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = g[i] / (1.0f + __expf(-g[i])) * u[i];
  } else {
    v = proj_scale4<true>(P, s, rs, m, n);
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
// Each thread takes groups of 8 consecutive elements (K is a multiple of 64),
// four groups in flight: a group index past the row is clamped to its last
// group, whose values the maximum already holds and whose codes another
// thread writes with the same bytes, so no load or store is conditional (a
// condition between the loads and their use let the compiler wait for each
// load in turn).
template <int XT>
__device__ __forceinline__ void load8(const void* x, int64_t off, float (&v)[8]) {
  if constexpr (XT == 0) {
    const float* p = reinterpret_cast<const float*>(x) + off;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3]; v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
    const unsigned d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16lo(d[j]);
      v[2 * j + 1] = bf16hi(d[j]);
    }
  }
}

template <int XT>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* x, int K, uint8_t* codes, float* scales) {
  __shared__ float red[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const int ng = K / 8;
  constexpr int U = 4;
  float m = 0.f;
  for (int g0 = t; g0 < ng; g0 += 256 * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load8<XT>(x, (int64_t)r * K + 8 * min(g0 + 256 * u, ng - 1), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
  }
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m > 0.f ? m / 448.0f : 1.0f;
  if (t == 0) scales[r] = s;
  for (int g0 = t; g0 < ng; g0 += 256 * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load8<XT>(x, (int64_t)r * K + 8 * min(g0 + 256 * u, ng - 1), v[u]);
    __builtin_amdgcn_sched_barrier(0);  // all four loads issue before the divisions
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unsigned c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = f32x2_to_fp8x2(v[u][2 * j] / s, v[u][2 * j + 1] / s);
      *reinterpret_cast<u32x2*>(codes + (int64_t)r * K + 8 * min(g0 + 256 * u, ng - 1)) =
          u32x2{c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
    }
  }
}

static int splits_of(const pkd_matrix* W) { return W->k_splits > 1 ? W->k_splits : 1; }

size_t proj_workspace_bytes(const pkd_matrix* W, int32_t max_rows) {
  if (!W || max_rows <= 0 || !tiled_family(W->family)) return 0;
  size_t b = 0;
  if (W->dtype == PKD_FP8_E4M3) b += align256((size_t)max_rows * W->cols) + align256(sizeof(float) * (size_t)max_rows);
  if (splits_of(W) > 1) b += align256(sizeof(float) * (size_t)splits_of(W) * max_rows * W->rows);
  return b;
}

pkd_status gemv_launch(const ProjArgs& a, hipStream_t stream, pkd_error* err);

template <int MODE, int TM>
static void launch_tile(const GemmParams& P, int grid, hipStream_t stream) {
  constexpr int lds = Tile<MODE, TM>::LDS_BYTES;
  // dynamic LDS above 64 KiB must be enabled once per kernel and device; two
  // threads may both enable it, which is harmless
  static std::atomic<uint64_t> enabled{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = 1ull << (dev & 63);
  if (!(enabled.load(std::memory_order_acquire) & bit)) {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<MODE, TM>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    enabled.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((gemm_kernel<MODE, TM>), dim3(grid), dim3(64 * NWAVES), lds, stream, P);
}

// Measured per-CU rates of the two tile heights at the 7B shapes: the 256-row
// tile pulls fewer operand bytes per product (131 against 87 flop per byte)
// and runs at about 4.7 TFLOP/s per CU, the 128-row tile at about 3.5.
constexpr double kRate256 = 4.7e12, kRate128 = 3.5e12;

// Activation tile height: the one whose rounds of workgroups over the 256 CUs
// take less time at those rates (a tile's time is proportional to its height
// over its rate).  Either height runs the same k-loop per output, so the
// choice never changes a result.
static int tile_m_for(int tiles_n, int splits, int M) {
  const long i256 = (long)tiles_n * splits * ((M + 255) / 256);
  const long i128 = (long)tiles_n * splits * ((M + 127) / 128);
  const double t256 = (double)((i256 + 255) / 256) * 256.0 / kRate256;
  const double t128 = (double)((i128 + 255) / 256) * 128.0 / kRate128;
  return t256 <= t128 ? 256 : 128;
}


// Estimated time of a split, in microseconds: rounds of workgroups over the
// 256 CUs times the time of one workgroup (tile height x 256 weight rows x its
// share of K, at the measured rate of that tile height), plus the partial sums
// of S > 1, written once and read once by the finish pass (at about 5 TB/s).
// A larger S must beat the best so far by 5%.  With these terms the model
// picks the measured best S at the 7B shapes at batch 768 (qkv 2, W_o 3,
// gate/up 1, down 6 on the 256-row tile: 115 us against 130 at S = 3) and at
// batch 256 (qkv 6, W_o 6, gate/up 1, down 8).
int suggest_k_splits(int rows, int cols, int family, int typical_rows) {
  if (!tiled_family(family) || rows <= 0 || cols <= 0 || typical_rows <= 0) return 1;
  constexpr double kPartialBytesPerS = 5e12;
  const int tiles_n = (rows + TN - 1) / TN;
  int best = 1;
  double best_cost = 0;
  for (int s : {1, 2, 3, 4, 6, 8}) {
    if (s > 1 && cols / s < 512) break;
    const int tm = tile_m_for(tiles_n, s, typical_rows);
    const long items = (long)tiles_n * s * ((typical_rows + tm - 1) / tm);
    const double wg_us = 2.0 * tm * TN * ((cols + s - 1) / s) / (tm == 256 ? kRate256 : kRate128) * 1e6;
    const double partial_us = s > 1 ? 2.0 * s * rows * (double)typical_rows * 4 / kPartialBytesPerS * 1e6 : 0.0;
    const double cost = (double)((items + 255) / 256) * wg_us + partial_us;
    if (s == 1 || cost < 0.95 * best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

pkd_status proj_launch(const ProjArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err) {
  const pkd_matrix& W = *a.W;
  if (a.n_rows == 0) return ok(err);
  if (!tiled_family(W.family)) return gemv_launch(a, stream, err);
  const size_t need = proj_workspace_bytes(a.W, a.n_rows);
  if (need && (!ws || ws_bytes < need))
    return fail(err, PKD_ERR_OUT_OF_MEMORY, (int64_t)need, (int64_t)(ws ? ws_bytes : 0),
                "projection workspace too small: need %zu bytes", need);
  if (need && ((uintptr_t)ws & 255)) return fail(err, PKD_ERR_INVALID_ARG, 0, 0, "workspace must be 256-byte aligned");
  {
    // the tile loader addresses each operand with 32-bit byte offsets
    const int64_t row_bytes = W.dtype == PKD_BF16 ? 2 * (int64_t)W.cols : (int64_t)W.cols;
    if ((int64_t)(W.rows + 256) * row_bytes >= ((int64_t)1 << 31) ||
        (int64_t)(a.n_rows + 256) * row_bytes >= ((int64_t)1 << 31))
      return fail(err, PKD_ERR_UNSUPPORTED, (int64_t)W.rows, (int64_t)a.n_rows,
                  "matrix-core projection operands must each be below 2 GiB");
  }
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
  P.row_scale = a.row_scale;
  P.rope_cs = a.rope_cs;
  P.rope_cols = a.rope_cols;
  P.rope_hd = a.rope_hd;
  P.tiles_n = (W.rows + TN - 1) / TN;
  P.splits = splits_of(a.W);
  const int tile_m = tile_m_for(P.tiles_n, P.splits, a.n_rows);
  P.tiles_m = (a.n_rows + tile_m - 1) / tile_m;
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
  const int grid = P.tiles_n * P.splits * P.tiles_m;
  if (tile_m == 256) {
    if (mode == 0) launch_tile<0, 256>(P, grid, stream);
    else if (mode == 1) launch_tile<1, 256>(P, grid, stream);
    else launch_tile<2, 256>(P, grid, stream);
  } else {
    if (mode == 0) launch_tile<0, 128>(P, grid, stream);
    else if (mode == 1) launch_tile<1, 128>(P, grid, stream);
    else launch_tile<2, 128>(P, grid, stream);
  }
  if (P.splits > 1) {
    const int64_t groups = (int64_t)P.M * (P.n_out / 4);
    const unsigned blocks = (unsigned)((groups + 255) / 256);
    if (fp8) hipLaunchKernelGGL(splitk_finish_kernel<true>, dim3(blocks), dim3(256), 0, stream, P);
    else hipLaunchKernelGGL(splitk_finish_kernel<false>, dim3(blocks), dim3(256), 0, stream, P);
  }
  return check_launch(err, "matrix-core projection");
}

}  // namespace pkd
