// Grouped expert GEMMs on the gfx950 matrix cores, bf16 and E4M3.
//
// Each routed expert e owns rows offsets[e]..offsets[e+1]-1 of the dispatched order; the shared
// experts form one more group over all T tokens. One launch covers every group:
//   gate/up:  [g | v] = X W13^T, a = SiLU(g) * v        (X gathered from u through perm_src)
//   down:     y = a W2^T
// (DeepSeek Technical Report: MoE Architecture, 1.1 and 5.3 [1]; SwiGLU per the DeepSeek-V3
// walkthrough, "invariant core"). The E4M3 variant follows 3.6 of the same report: 1x128 activation
// scales, 128x128 weight scales, and every 128-element partial product multiplied by its two scales
// and added into an fp32 accumulator (promotion interval 128); the gate/up epilogue quantizes a
// again per row per 128 columns.
//
// Tile: 256 weight rows x 256 tokens, K streamed 128 bytes (128 E4M3 or 64 bf16 elements) per stage,
// so one stage moves 64 KB for 8.4 M multiply-adds. The product is formed transposed (weights as the
// MFMA A operand, tokens as B) so that each lane's accumulators belong to one token: the token's scale
// is one value per lane and the 1x128 requant reduces over channels held by one lane group. Eight waves
// (two per SIMD) each own 64 weight rows (gate/up: 32 gate channels and the same 32 up channels)
// against 128 tokens; the two waves of a SIMD share weight rows and split the tokens.
// Both operands move global -> LDS by the LDS-DMA loads, 8 lanes per 128-byte row so that every load
// instruction touches whole cache lines (gathering 16 rows x 64 B per instruction, the MFMA operand
// layout, runs the vector L1 at a third of that rate). The ring has two stages: one is multiplied while
// the next one loads. LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r sits at c ^ (r & 7))
// so that the MFMA operand reads are free of bank conflicts.
// Each block walks its tiles as one continuous stream of stages (the first stage of the next tile
// loads while the last stage of the current one is multiplied), and the epilogue stores straight from
// registers. Waves whose 128 tokens all lie past the tile's last row skip the multiply.
// The grid is persistent: blocks are split by XCD (block id mod 8) and each XCD walks one contiguous
// range of the tile list, in which neighbouring tiles share an expert's weight tile in that XCD's L2.
// Weights come either row-major or in the tiled layout of pack_weights below, where every 32 KB weight
// stage of a tile is contiguous in HBM and already in the MFMA operand order.
#include "common.h"
#include "kernels.h"

#include <atomic>
#include "tiles.h"

#include <utility>

namespace moe {

constexpr int kBM = 256;                         // tokens per tile
constexpr int kBW = 256;                         // weight rows per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStageB = 128;                     // K bytes per stage
constexpr int kTJ = 8;                           // 16-token MFMA tiles per wave (128 tokens)
constexpr int kChunks = kBW * 8 / kThreads;      // 16-byte chunks each thread moves per operand per stage
constexpr int kSlotA = kBW * kStageB;            // 32 KB of weight rows
constexpr int kSlotB = kBM * kStageB;            // 32 KB of token rows
constexpr int kSX = kSlotA + kSlotB;             // one E4M3 scale per token
constexpr int kWS = kSX + kBM * 4;               // the stage's two weight block scales
constexpr int kSlot = kWS + 16;
constexpr int kRed = 2 * kSlot;                  // epilogue exchange of row maxima [4][kBM] floats
constexpr int kTab = kRed + 4 * kBM * 4;         // copies of the tile prefix and group offsets
constexpr int kMaxGroups = 257;
constexpr int kIds = kTab + 2 * kMaxGroups * 4 + 8;   // ring of the block's next tile ids
constexpr int kLdsBytes = kIds + 16;
static_assert(kBW == kBM && kChunks == 4 && kLdsBytes <= 160 * 1024, "geometry");

// One K stage of one wave: its four 16-row weight tiles against its first JN 16-token tiles (the tiles of
// its 128 tokens that hold rows of the M tile, rounded up to an even count; the others are neither read
// nor multiplied). E4M3: every 16x16x128 product is a fresh partial sum, scaled by (token scale x weight
// block scale) and added into fp32 one MFMA after it is issued, so the matrix core and the vector ALU
// overlap.
template <bool FP8, bool GATEUP, bool PACKED, int JN>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[4][kTJ], const uint8_t* __restrict__ slot, int wn, int tok0,
                                          int tr, int g) {
  const uint8_t* A = slot;
  const uint8_t* B = slot + kSlotA;
  auto rd = [&](const uint8_t* base, int row, i32x4& lo, i32x4& hi) {
    lo = *reinterpret_cast<const i32x4*>(base + row * kStageB + ((g ^ (row & 7)) * 16));
    hi = *reinterpret_cast<const i32x4*>(base + row * kStageB + (((4 + g) ^ (row & 7)) * 16));
  };
  // weight rows of tile i: gate/up -> gate rows 32 wn + 16 i (i < 2) and the matching up rows 128 + ...;
  // down -> rows 64 wn + 16 i. In the tiled layout those are 16-row blocks 2 wn + i (+ 8 for up) or
  // 4 wn + i of the stage, each 2 KB in operand order: lane l's chunks g and 4 + g at 16 l and 1024 + 16 l.
  i32x4 a[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = GATEUP ? (i < 2 ? 0 : 8) + 2 * wn + (i & 1) : 4 * wn + i;
    if constexpr (PACKED) {
      const uint8_t* p = A + blk * 2048 + (16 * g + tr) * 16;
      a[i][0] = *reinterpret_cast<const i32x4*>(p);
      a[i][1] = *reinterpret_cast<const i32x4*>(p + 1024);
    } else {
      rd(A, 16 * blk + tr, a[i][0], a[i][1]);
    }
  }
  i32x4 b[2][2];
  rd(B, tok0 + tr, b[0][0], b[0][1]);
  if constexpr (FP8) {
    const float* SX = reinterpret_cast<const float*>(slot + kSX);
    const float* WSc = reinterpret_cast<const float*>(slot + kWS);
    const float ws0 = WSc[0], ws1 = WSc[1];
    float wsi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wsi[i] = GATEUP ? (i < 2 ? ws0 : ws1) : (wn < 2 ? ws0 : ws1);
    i32x8 aa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      aa[i] = i32x8{a[i][0][0], a[i][0][1], a[i][0][2], a[i][0][3], a[i][1][0], a[i][1][1], a[i][1][2], a[i][1][3]};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 p[2];
    float cs[4];
    float sxv[2];
    sxv[0] = SX[tok0 + tr];
    [&]<int... J>(std::integer_sequence<int, J...>) {
      ([&] {
        constexpr int j = J;
        if constexpr (j + 1 < JN) rd(B, tok0 + 16 * (j + 1) + tr, b[(j + 1) & 1][0], b[(j + 1) & 1][1]);
        const i32x4 b0 = b[j & 1][0], b1 = b[j & 1][1];
        const i32x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        // token scales are read one 16-token tile ahead, like the token operand
        if constexpr (j + 1 < JN) sxv[(j + 1) & 1] = SX[tok0 + 16 * (j + 1) + tr];
        const float sx = sxv[j & 1];
        [&]<int... I>(std::integer_sequence<int, I...>) {
          ([&] {
            constexpr int i = I;
            p[i & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aa[i], bb, zero, 0, 0, 0, 127, 0, 127);
            // the product issued one MFMA earlier: tile (i - 1, j), or (3, j - 1) for i = 0
            if constexpr (i > 0) acc[i - 1][j] += cs[i - 1] * p[(i - 1) & 1];
            else if constexpr (j > 0) acc[3][j - 1] += cs[3] * p[1];
            cs[i] = sx * wsi[i];
          }(), ...);
        }(std::make_integer_sequence<int, 4>{});
      }(), ...);
    }(std::make_integer_sequence<int, JN>{});
    acc[3][JN - 1] += cs[3] * p[1];
  } else {
    [&]<int... J>(std::integer_sequence<int, J...>) {
      ([&] {
        constexpr int j = J;
        if constexpr (j + 1 < JN) rd(B, tok0 + 16 * (j + 1) + tr, b[(j + 1) & 1][0], b[(j + 1) & 1][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][0]),
                                                              __builtin_bit_cast(bf16x8, b[j & 1][0]), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][1]),
                                                              __builtin_bit_cast(bf16x8, b[j & 1][1]), acc[i][j], 0, 0, 0);
        }
      }(), ...);
    }(std::make_integer_sequence<int, JN>{});
  }
}

// RAW: the accumulators are stored in fp32 as they are (gate/up: g and v, no SwiGLU; down: fp32 instead
// of bf16), for the input backward of the experts.
template <bool FP8, bool GATEUP, bool RAW, bool PACKED>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mfma(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wm = wave >> 2, tok0 = 128 * wm;
  const int tr = lane & 15, g = lane >> 4;
  constexpr int esz = FP8 ? 1 : 2;
  const int E = a.E;
  const int nt_r = GATEUP ? a.f / 128 : a.d / kBW;

  // the tile prefix and group offsets, copied once into LDS so that decoding a tile never waits on memory
  int32_t* mtp = reinterpret_cast<int32_t*>(lds + kTab);
  int32_t* goff = mtp + kMaxGroups;
  for (int i = tid; i <= E; i += kThreads) {
    mtp[i] = a.mt_prefix[i];
    goff[i] = a.offsets[i];
  }
  // This XCD's range of the tile list; its blocks take tiles in order from the XCD's counter. Tile k of
  // the block has id ids[k % 4]: the ring holds the next three, and one more request is in flight.
  const int xcd = blockIdx.x & 7;
  const int t_begin = a.xrange[xcd], t_end = a.xrange[xcd + 1];
  const int p_begin = a.xrange[8], n_tiles = a.xrange[9];
  // the next tile id for this block: from its XCD's range, then from the shared pool; n_tiles: none left
  auto claim = [&]() {
    const int id = t_begin + atomicAdd(a.xcount + xcd, 1);
    if (id < t_end) return id;
    const int p = p_begin + atomicAdd(a.xcount + 8, 1);
    return p < n_tiles ? p : n_tiles;
  };
  int32_t* ids = reinterpret_cast<int32_t*>(lds + kIds);
  int pending = 0;
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) ids[k] = claim();
    pending = claim();
  }
  barrier_lds();
  int id_l = __builtin_amdgcn_readfirstlane(ids[0]);
  if (id_l >= n_tiles) return;
  int ktile = 0;                           // tiles the loader has started, minus one
  auto next_id = [&](int k) { return __builtin_amdgcn_readfirstlane(ids[k & 3]); };
  const int nt_s = max(1, GATEUP ? a.fs / 128 : a.d / kBW);
  auto decode = [&](int id) { return decode_tile_lds<kBM>(id, mtp, goff, E, a.T, nt_r, nt_s); };

  // ---- loader geometry. Thread tid moves, per stage and operand, chunks id = 512 q + tid (q < 4): LDS
  // row id / 8 = 64 q + lrow, LDS position id % 8, which holds global chunk (id % 8) ^ (row & 7).
  const int lrow = tid >> 3;
  const int lchunk = ((tid & 7) ^ (lrow & 7)) * 16;
  // perm_src entries of the next tile's rows, loaded a tile early (always in bounds: every group's rows
  // lie below T*K). Rows 64 q + lrow for the token chunks, row tid for the token scales (waves 0-3).
  TileInfo tn = decode(id_l);
  int rawn[kChunks + 1];
  auto row_in_tile = [&](const TileInfo& t, int q) { return min(q < kChunks ? q * 64 + lrow : tid, t.nrows - 1); };
  auto fetch_rows = [&](const TileInfo& t) {
#pragma unroll
    for (int q = 0; q <= kChunks; ++q) rawn[q] = a.perm_src[t.rowbase + row_in_tile(t, q)];
  };
  fetch_rows(tn);

  TileInfo tl;
  const uint8_t* Wl = nullptr;
  const uint8_t* Xl = nullptr;
  const float* XSl = nullptr;
  const float* WSl = nullptr;
  int nst_l = 0, kl = 0, kblk_l = 0, kbytes_l = 0, fg_l = 0, started = 1;
  bool live = true;
  uint32_t boff[kChunks], sxoff = 0;
  int sxstep = 1;
  auto setup = [&]() {
    tl = tn;
    const bool shared = tl.group == E;
    fg_l = shared ? a.fs : a.f;
    const int kelems = GATEUP ? a.d : fg_l;
    kbytes_l = kelems * esz;
    kblk_l = kelems / 128;
    nst_l = kbytes_l / kStageB;
    const float* WS = nullptr;
    if (GATEUP) {
      Wl = shared ? a.w_shared : a.w_routed + (size_t)tl.group * (2 * (size_t)a.f) * a.d * esz;
      if (FP8) WS = shared ? a.ws_shared : a.ws_routed + (size_t)tl.group * (2 * a.f / 128) * (a.d / 128);
    } else {
      Wl = shared ? a.w_shared : a.w_routed + (size_t)tl.group * (size_t)a.d * a.f * esz;
      if (FP8) WS = shared ? a.ws_shared : a.ws_routed + (size_t)tl.group * (a.d / 128) * (a.f / 128);
    }
    Xl = shared ? a.x_shared : a.x_routed;
    if (FP8) XSl = shared ? a.xs_shared : a.xs_routed;
    const bool gather = GATEUP && !shared;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int r = gather ? rawn[q] : tl.rowbase + row_in_tile(tl, q);
      boff[q] = (uint32_t)r * kbytes_l + lchunk;
    }
    if (FP8) {
      const int r = gather ? rawn[kChunks] : tl.rowbase + row_in_tile(tl, kChunks);
      const int xs_ld = shared ? a.xs_ld_shared : a.xs_ld_routed;
      // block-major scales are read in the dispatched order (row rowbase + i), not through perm_src
      sxoff = xs_ld ? (uint32_t)(tl.rowbase + row_in_tile(tl, kChunks)) : (uint32_t)r * kblk_l;
      sxstep = xs_ld ? xs_ld : 1;
      // lane 0 of wave 4 copies the scale of block row c0 / 128 (gate, or the first 128 down rows),
      // lane 1 that of (fg + c0) / 128 (up) or c0 / 128 + 1 (the next 128 down rows)
      const int c0 = tl.n_tile * (GATEUP ? 128 : kBW);
      const int brow = lane == 0 ? c0 / 128 : (GATEUP ? (fg_l + c0) / 128 : c0 / 128 + 1);
      WSl = WS + (size_t)brow * kblk_l;
    }
    // the offsets are final before rawn is reloaded into the same registers
    asm volatile("" ::"v"(boff[0]), "v"(boff[1]), "v"(boff[2]), "v"(boff[3]), "v"(sxoff) : "memory");
    kl = 0;
  };
  setup();
  int id_n = next_id(1);
  if (id_n < n_tiles) {
    tn = decode(id_n);
    fetch_rows(tn);
  }

  // Issue the loader's next stage into ring slot `sl`. A block with no tile left re-reads stage 0 of
  // its last tile, so the loop stays uniform; that data is never multiplied.
  auto issue = [&](uint8_t* sl) {
    if (kl == nst_l && live) {
      ++ktile;
      id_l = next_id(ktile);
      if (id_l < n_tiles) {
        setup();
        ++started;
        id_n = next_id(ktile + 1);
        if (id_n < n_tiles) {
          tn = decode(id_n);
          fetch_rows(tn);
        }
        // the id of tile ktile + 2 arrived a tile ago; request the one after it
        if (tid == 0) {
          ids[(ktile + 2) & 3] = pending;
          pending = claim();
        }
      } else {
        live = false;
      }
    }
    const int kk = live ? kl : 0;
    ++kl;
    if constexpr (PACKED) {
      // the stage's 32 KB are contiguous and land in LDS as they are
      const uint8_t* Wk = Wl + ((size_t)(tl.n_tile * nst_l + kk) << 15) + tid * 16;
#pragma unroll
      for (int q = 0; q < kChunks; ++q) dma16(Wk + q * kThreads * 16, sl + (q * kThreads + wave * 64) * 16);
    } else {
      // weight rows: LDS row 64 q + lrow is W1 row c0 + 64 q + lrow (q < 2) or W3 row fg + c0 + 64 q - 128 +
      // lrow (gate/up, c0 = 128 n_tile); W2 row c0 + 64 q + lrow (down, c0 = 256 n_tile)
      const int c0 = tl.n_tile * (GATEUP ? 128 : kBW);
      const uint8_t* Wk = Wl + (size_t)kk * kStageB + lchunk;
#pragma unroll
      for (int q = 0; q < kChunks; ++q) {
        const int wrow = (GATEUP && q >= 2) ? fg_l + c0 + 64 * q - 128 : c0 + 64 * q;
        dma16(Wk + (size_t)(wrow + lrow) * kbytes_l, sl + (q * kThreads + wave * 64) * 16);
      }
    }
    const uint8_t* Xk = Xl + (size_t)kk * kStageB;
    // 64-row groups of the token tile past its last row are not copied: their LDS rows keep older data,
    // which only ever reaches the accumulators of padding tokens (a token's products use its own row
    // only), and those are never stored
#pragma unroll
    for (int q = 0; q < kChunks; ++q)
      if (q == 0 || 64 * q < tl.nrows) dma16(Xk + boff[q], sl + kSlotA + (q * kThreads + wave * 64) * 16);
    if (FP8 && wave < 4) dma4(XSl + sxoff + (size_t)kk * sxstep, sl + kSX + wave * 256);
    if (FP8 && wave == 4 && lane < 2) dma4(WSl + kk, sl + kWS);
  };

  // ---- compute: the tile being multiplied
  TileInfo tc = tl;
  int nst_c = nst_l, kb = 0, done = 0;
  f32x4 acc[4][kTJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(lds);
  int gs = 0;
  for (;;) {
    // the stages of tile tc, in a loop of their own for each count of live 16-token tiles of this wave
    // (so that each loop holds one fully unrolled multiply)
    auto stages = [&](auto jn) {
      constexpr int JN = decltype(jn)::value;
      for (; kb < nst_c; ++kb, ++gs) {
        uint8_t* cur = lds + (gs & 1) * kSlot;
        wait_vm0();       // this wave's copies of stage gs have landed
        barrier_lds();    // ... and every wave's; every wave is done with the other slot
        issue(lds + ((gs + 1) & 1) * kSlot);
        if constexpr (JN > 0) mma_stage<FP8, GATEUP, PACKED, JN>(acc, cur, wn, tok0, tr, g);
      }
    };
    const int live_rows = tc.nrows - tok0;
    if (live_rows > 96) stages(std::integral_constant<int, 8>{});
    else if (live_rows > 64) stages(std::integral_constant<int, 6>{});
    else if (live_rows > 32) stages(std::integral_constant<int, 4>{});
    else if (live_rows > 0) stages(std::integral_constant<int, 2>{});
    else stages(std::integral_constant<int, 0>{});

    // ---- epilogue of tile tc. Lane holds, for token tok0 + 16 j + tr, channels 4 g + r of each 16-row
    // weight tile i (gate/up: gate channels 32 wn + 16 i for i < 2, their up channels for i >= 2).
    const bool shared = tc.group == E;
    const int fg = shared ? a.fs : a.f;
    if constexpr (GATEUP && RAW) {
      // [g | v] in fp32, row stride 2 fg: gate channel c at column c, its up channel at fg + c
      const int c0 = tc.n_tile * 128;
      const size_t ostride = (size_t)2 * fg;
      float* OUTF = reinterpret_cast<float*>(shared ? a.out_shared : a.out_routed) + (size_t)tc.rowbase * ostride +
                    c0 + 32 * wn + 4 * g;
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        const int tok = tok0 + 16 * j + tr;
        if (tok < tc.nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(OUTF + (size_t)tok * ostride + 16 * (i & 1) + (i >= 2 ? fg : 0)) = acc[i][j];
        }
      }
    } else if constexpr (GATEUP) {
      const int c0 = tc.n_tile * 128;
      float av[2][kTJ][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) av[i][j][r] = silu(acc[i][j][r]) * acc[i + 2][j][r];
      const size_t out_stride = (size_t)fg * esz;
      uint8_t* OUT = (shared ? a.out_shared : a.out_routed) + (size_t)tc.rowbase * out_stride +
                     (size_t)(c0 + 32 * wn + 4 * g) * esz;
      if constexpr (FP8) {
        // 1x128 requant of a: a token's 128 channels of this tile are spread over the four wn waves
        float* red = reinterpret_cast<float*>(lds + kRed);
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          float m = 0.f;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(av[i][j][r]));
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          if (lane < 16) red[wn * kBM + tok0 + 16 * j + tr] = m;
        }
        barrier_lds();
        float* OS = shared ? a.out_scale_shared : a.out_scale_routed;
        // every exchange read comes before the first store: an LDS read placed after a global store waits
        // for that store to complete (the compiler guards LDS reads that may follow LDS-DMA copies with a
        // full vector-memory wait), which would put one store round trip per 16-token tile in the epilogue
        float sj[kTJ], ij[kTJ];
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int tok = tok0 + 16 * j + tr;
          const float m = fmaxf(fmaxf(red[tok], red[kBM + tok]), fmaxf(red[2 * kBM + tok], red[3 * kBM + tok]));
          e4m3_scales(m, sj[j], ij[j]);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int tok = tok0 + 16 * j + tr;
          const float s = sj[j], inv = ij[j];
          if (tok < tc.nrows) {
            if (wn == 0 && g == 0) {
              const int os_ld = shared ? a.os_ld_shared : a.os_ld_routed;
              OS[os_ld ? (size_t)tc.n_tile * os_ld + tc.rowbase + tok : (size_t)(tc.rowbase + tok) * (fg / 128) + tc.n_tile] = s;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
              *reinterpret_cast<uint32_t*>(OUT + (size_t)tok * out_stride + 16 * i) =
                  f32x4_to_e4m3x4(av[i][j][0] * inv, av[i][j][1] * inv, av[i][j][2] * inv, av[i][j][3] * inv);
          }
        }
        // `red` is written again only by the next epilogue, after at least one more barrier
      } else {
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int tok = tok0 + 16 * j + tr;
          if (tok < tc.nrows) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              uint2 v;
              v.x = uint32_t(f32_to_bf16(av[i][j][0])) | (uint32_t(f32_to_bf16(av[i][j][1])) << 16);
              v.y = uint32_t(f32_to_bf16(av[i][j][2])) | (uint32_t(f32_to_bf16(av[i][j][3])) << 16);
              *reinterpret_cast<uint2*>(OUT + (size_t)tok * out_stride + 16 * i * esz) = v;
            }
          }
        }
      }
    } else {
      const int c0 = tc.n_tile * kBW;
      constexpr int ysz = (FP8 && !RAW) ? 2 : 4;   // y in bf16 (the combine payload of the E4M3 path) or fp32
      const size_t out_stride = (size_t)a.d * ysz;
      uint8_t* OUT = (shared ? a.out_shared : a.out_routed) + (size_t)tc.rowbase * out_stride +
                     (size_t)(c0 + 64 * wn + 4 * g) * ysz;
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        const int tok = tok0 + 16 * j + tr;
        if (tok < tc.nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint8_t* o = OUT + (size_t)tok * out_stride + 16 * i * ysz;
            if constexpr (FP8 && !RAW) {
              uint2 v;
              v.x = uint32_t(f32_to_bf16(acc[i][j][0])) | (uint32_t(f32_to_bf16(acc[i][j][1])) << 16);
              v.y = uint32_t(f32_to_bf16(acc[i][j][2])) | (uint32_t(f32_to_bf16(acc[i][j][3])) << 16);
              *reinterpret_cast<uint2*>(o) = v;
            } else {
              *reinterpret_cast<f32x4*>(o) = acc[i][j];
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (++done == started && !live) break;
    // the loader moved to this tile while the last stage of the previous one was multiplied
    tc = tl;
    nst_c = nst_l;
    kb = 0;
  }
  wait_vm0();
}

int gemm_mfma_bm() { return kBM; }

template <bool FP8, bool GATEUP, bool RAW, bool PACKED>
hipError_t launch_variant(const GemmArgs& a, int grid, hipStream_t s) {
  static std::atomic<bool> attr_done{false};   // set once per kernel (setting it twice is harmless)
  const void* fn = (const void*)grouped_gemm_mfma<FP8, GATEUP, RAW, PACKED>;
  if (!attr_done.load(std::memory_order_relaxed)) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done.store(true, std::memory_order_relaxed);
  }
  grouped_gemm_mfma<FP8, GATEUP, RAW, PACKED><<<grid, kThreads, kLdsBytes, s>>>(a);
  return hipGetLastError();
}

template <bool PACKED>
hipError_t launch_layout(const GemmArgs& a, bool fp8, bool gateup, int grid, hipStream_t s, bool raw) {
  if (raw) return gateup ? launch_variant<true, true, true, PACKED>(a, grid, s) : launch_variant<true, false, true, PACKED>(a, grid, s);
  if (fp8) return gateup ? launch_variant<true, true, false, PACKED>(a, grid, s) : launch_variant<true, false, false, PACKED>(a, grid, s);
  return gateup ? launch_variant<false, true, false, PACKED>(a, grid, s) : launch_variant<false, false, false, PACKED>(a, grid, s);
}

hipError_t launch_gemm_mfma(const GemmArgs& a, bool fp8, bool gateup, int grid, hipStream_t s, bool raw) {
  if (raw && !fp8) return hipErrorInvalidValue;
  return a.packed ? launch_layout<true>(a, fp8, gateup, grid, s, raw) : launch_layout<false>(a, fp8, gateup, grid, s, raw);
}

// ---- the tiled weight layout. For each group (a routed expert, or the shared block), each N tile of 256
// weight rows (gate/up: W1 rows 128 n .. 128 n + 127 then the W3 rows f + 128 n ..; down: rows 256 n ..)
// and each 128-byte K stage k, 32 KB at ((n * stages + k) << 15): the tile's sixteen 16-row blocks, 2 KB
// each, and in a block the 16-byte chunk c (of 8) of row r (of 16) at byte 16 (64 (c / 4) + 16 (c % 4) + r),
// i.e. lane 16 (c % 4) + r of the MFMA operand, low half for c < 4, high half after 1 KB. One thread per
// 16-byte chunk of the output.
__global__ void pack_weights(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int rows, int row_bytes,
                             int gateup, long long per_group, long long total) {
  const int stages = row_bytes / kStageB;
  for (long long c = blockIdx.x * (long long)blockDim.x + threadIdx.x; c < total; c += (long long)gridDim.x * blockDim.x) {
    const long long grp = c / per_group;
    const long long r = c - grp * per_group;
    const int lane = (int)(r & 63), half = (int)((r >> 6) & 1), blk = (int)((r >> 7) & 15);
    const long long nk = r >> 11;
    const int n = (int)(nk / stages), k = (int)(nk - (long long)n * stages);
    const int row = (gateup ? (blk < 8 ? 128 * n + 16 * blk : rows / 2 + 128 * n + 16 * (blk - 8)) : 256 * n + 16 * blk) +
                    (lane & 15);
    const size_t so = (size_t)grp * rows * row_bytes + (size_t)row * row_bytes + (size_t)k * kStageB +
                      (4 * half + (lane >> 4)) * 16;
    *reinterpret_cast<i32x4*>(dst + c * 16) = *reinterpret_cast<const i32x4*>(src + so);
  }
}

hipError_t launch_pack_weights(const void* src, void* dst, int groups, int rows, int row_bytes, bool gateup,
                               hipStream_t s) {
  const long long per_group = (long long)rows * row_bytes / 16;
  const long long total = per_group * groups;
  if (total == 0) return hipSuccess;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  pack_weights<<<blocks, 256, 0, s>>>(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows, row_bytes,
                                      gateup ? 1 : 0, per_group, total);
  return hipGetLastError();
}

}  // namespace moe
