// Small-group 16-bit weight gradient on block-diagonal 16x16x32 MFMA (gfx950).
//
// Grouped convolutions with few channels per group (4 and 8 per group: the
// cpg4 / cpg8 cases of rocm-libraries PR #14157, "depthwise 7x7 and grouped
// cpg4/8 wgrad", section Technical Details) are computed as dense 16 x 16
// products over "super-groups" of 16 consecutive channels, keeping only the
// block-diagonal outputs where the output channel and the input channel belong
// to the same group.  The discarded products cost MFMA issue slots, which are
// plentiful here; the HBM bytes, the real bound, are each read once.
//
//   out[k][c] (tap r,s) += sum over 32 output pixels p of dY[p][k] * X[p + (r,s)][c]
//
// A workgroup owns 64 channels (4 waves x one super-group) and a slice of
// units; a unit is up to 4 output rows x 32 output pixels of one image.  The
// unit's dY pixels and the X pixels it needs (with zero padding) are staged in
// LDS in their NHWC order (64 channels per pixel, 160-byte pixel pitch).  The
// MFMA operands need 8 consecutive pixels of one channel per lane, which is a
// transpose of that layout; ds_read_b64_tr_b16 does it on the read: within a
// 16-lane group, lane j points at 4 channels of pixel j/4 and lane i receives
// channel i of 4 consecutive pixels.  One A operand (dY) per output row serves
// all R*S taps; each tap reads its B operand (X) at the tap's pixel offset.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kCh = 64;                 // channels per workgroup
constexpr int kPitchE = 80;             // 16-bit elements per staged pixel (64 + pad)
constexpr int kWoT = 32;                // output pixels per unit row (one MFMA k-step)
constexpr int kMaxRU = 4;               // output rows per unit
constexpr int kMaxXRows = 8;
constexpr int kMaxXPix = 40;
constexpr int kMaxTaps = 9;
constexpr int kDyPix = kMaxRU * kWoT;               // 128 staged dY pixels
constexpr int kXPix = kMaxXRows * kMaxXPix;          // 320 staged X pixels
constexpr int kLoaders = 256 / 8;                    // pixels per loader pass (8 x 16 B per pixel)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct G16Args {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;
  int32_t H, W, C, K, Ho, Wo, R, S, pad, dil, Cg, Kg, taps;
  int32_t ru, hblocks, wchunks, xrows, xpix;
  int32_t c_blocks, units, units_per_slice, ks_count;
  float* dbo;   // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

__device__ __forceinline__ s16x4 tr_read(const unsigned short* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <bool kBf16>
__device__ __forceinline__ f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// RT x ST: compile-time filter size (0 x 0 = runtime size, at most kMaxTaps taps).
template <bool kBf16, int RT, int ST>
__global__ __launch_bounds__(256, 2) void grouped16_kernel(G16Args a) {
  constexpr int kTaps = RT * ST > 0 ? RT * ST : kMaxTaps;
  const int taps = RT * ST > 0 ? RT * ST : a.taps;
  const int S = ST > 0 ? ST : a.S;
  __shared__ __attribute__((aligned(16))) unsigned short s_dy[kDyPix * kPitchE];
  __shared__ __attribute__((aligned(16))) unsigned short s_x[kXPix * kPitchE];
  const unsigned short* __restrict__ x = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ dy = static_cast<const unsigned short*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  const int cb = bid / a.ks_count;
  const int c0 = cb * kCh;
  const int u_begin = slice * a.units_per_slice;
  const int u_end = min(a.units, u_begin + a.units_per_slice);

  // Loader role: pixel slot tid/8 (+32 per pass), 16-byte chunk q of the 64 channels.
  const int q = tid & 7, pslot = tid >> 3;
  const bool ch_ok = c0 + 8 * q < a.C;  // C % 8 == 0: a chunk is all in or all out
  uint4 rdy[kDyPix / kLoaders];
  uint4 rx[kXPix / kLoaders];

  auto load_unit = [&](int u) {
    const int wc = u % a.wchunks;
    const int t = u / a.wchunks;
    const int hb = t % a.hblocks, n = t / a.hblocks;
    const int ho0 = hb * a.ru, wo0 = wc * kWoT;
#pragma unroll
    for (int i = 0; i < kDyPix / kLoaders; ++i) {
      const int pp = pslot + kLoaders * i;
      const int rho = pp / kWoT, p = pp % kWoT;
      const int ho = ho0 + rho, wo = wo0 + p;
      rdy[i] = uint4{0u, 0u, 0u, 0u};
      if (ch_ok && rho < a.ru && ho < a.Ho && wo < a.Wo)
        rdy[i] = *reinterpret_cast<const uint4*>(
            dy + ((int64_t)(n * a.Ho + ho) * a.Wo + wo) * a.K + c0 + 8 * q);
    }
    const int h0 = ho0 - a.pad, w0 = wo0 - a.pad;
#pragma unroll
    for (int i = 0; i < kXPix / kLoaders; ++i) {
      const int pp = pslot + kLoaders * i;
      const int xr = pp / kMaxXPix, xp = pp % kMaxXPix;
      const int h = h0 + xr, w = w0 + xp;
      rx[i] = uint4{0u, 0u, 0u, 0u};
      if (ch_ok && xr < a.xrows && xp < a.xpix && h >= 0 && h < a.H && w >= 0 && w < a.W)
        rx[i] = *reinterpret_cast<const uint4*>(
            x + (int64_t)n * a.x_img + ((int64_t)h * a.W + w) * a.C + c0 + 8 * q);
    }
  };
  // Bias-gradient partial of channels c0 + 8q .. + 7: every dY pixel of the
  // slice is staged once (pixels outside the output were loaded as zero).
  const bool want_db = a.dbo != nullptr;
  float dbp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto store_unit = [&]() {
#pragma unroll
    for (int i = 0; i < kDyPix / kLoaders; ++i) {
      *reinterpret_cast<uint4*>(&s_dy[(pslot + kLoaders * i) * kPitchE + 8 * q]) = rdy[i];
      if (want_db) add8<kBf16>(dbp, rdy[i]);
    }
#pragma unroll
    for (int i = 0; i < kXPix / kLoaders; ++i)
      *reinterpret_cast<uint4*>(&s_x[(pslot + kLoaders * i) * kPitchE + 8 * q]) = rx[i];
  };

  // Transposed-read addressing: in 16-lane group g, lane j points at pixel
  // 8g + (j >> 2) (+4 for the second half of the k-step) and channels
  // 16*wave + 4*(j & 3) .. +3.
  const int j = lane & 15, g = lane >> 4;
  const int pix_lane = 8 * g + (j >> 2);
  const int ch_lane = 16 * wave + 4 * (j & 3);
  int tap_off[kTaps];  // X pixel offset of tap t in the staged tile
#pragma unroll
  for (int t = 0; t < kTaps; ++t) {
    const int tt = t < taps ? t : 0;
    tap_off[t] = ((tt / S) * a.dil * kMaxXPix + (tt % S) * a.dil) * kPitchE;
  }

  f32x4 acc[kTaps];
#pragma unroll
  for (int t = 0; t < kTaps; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operands of one output row: A (dY) and the B (X) of every tap.  All reads
  // of a row are issued before its MFMAs, and the next row's reads before the
  // current row's MFMAs.
  s16x8 fa0, fa1, fb0[kTaps], fb1[kTaps];
  auto read_row = [&](int rho, s16x8& fa, s16x8 (&fb)[kTaps]) {
    const unsigned short* pa = s_dy + (rho * kWoT + pix_lane) * kPitchE + ch_lane;
    fa = __builtin_shufflevector(tr_read(pa), tr_read(pa + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
    const unsigned short* pb = s_x + (rho * kMaxXPix + pix_lane) * kPitchE + ch_lane;
#pragma unroll
    for (int t = 0; t < kTaps; ++t) {
      if (RT * ST > 0 || t < taps) {
        const unsigned short* pt = pb + tap_off[t];
        fb[t] = __builtin_shufflevector(tr_read(pt), tr_read(pt + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  auto mfma_row = [&](const s16x8& fa, const s16x8 (&fb)[kTaps]) {
#pragma unroll
    for (int t = 0; t < kTaps; ++t)
      if (RT * ST > 0 || t < taps) acc[t] = mfma16<kBf16>(fa, fb[t], acc[t]);
  };

  if (u_begin < u_end) load_unit(u_begin);
  for (int u = u_begin; u < u_end; ++u) {
    __syncthreads();  // previous unit's reads of the tiles are done
    store_unit();
    __syncthreads();
    if (u + 1 < u_end) load_unit(u + 1);
    read_row(0, fa0, fb0);
    for (int rho = 0; rho < a.ru; rho += 2) {
      if (rho + 1 < a.ru) read_row(rho + 1, fa1, fb1);
      mfma_row(fa0, fb0);
      if (rho + 1 < a.ru) {
        if (rho + 2 < a.ru) read_row(rho + 2, fa0, fb0);
        mfma_row(fa1, fb1);
      }
    }
  }

  if (want_db)
    block_sum64<32, 8>(reinterpret_cast<float*>(s_dy), pslot, 8 * q, dbp,
                       a.dbo + (int64_t)slice * a.slab_stride + c0, min(kCh, a.K - c0));

  // acc[t][v] = out[k = c0 + 16*wave + 4*g + v][c = c0 + 16*wave + j] for tap t;
  // only same-group pairs are outputs.
  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + j;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int k = c0 + 16 * wave + 4 * g + v;
    if (k < a.K && c < a.C && k / a.Kg == c / a.Cg) {
      float* o = out + (int64_t)k * taps * a.Cg + (c % a.Cg);
#pragma unroll
      for (int t = 0; t < kTaps; ++t)
        if (t < taps) o[t * a.Cg] = acc[t][v];
    }
  }
}

// Fast path for stride 1, dilation 1 and a compile-time R x S filter with 4
// output rows per unit.  The loop runs over the staged X rows instead of the
// output rows: X row t is read once per tap column s (S transposed reads) and
// multiplied with every dY row t - r that uses it, whose A operands stay in
// registers.  Per unit and wave: 4 A reads + (4 + R - 1) * S B reads for
// 4 * R * S MFMAs.  The LDS tiles are sized exactly (three workgroups per CU
// for 3 x 3).
template <bool kBf16, int R, int S>
__global__ __launch_bounds__(256, 3) void grouped16_win_kernel(G16Args a) {
  constexpr int RU = 4, XR = RU + R - 1, XP = kWoT + S - 1;
  constexpr int kDy = RU * kWoT, kX = XR * XP;
  __shared__ __attribute__((aligned(16))) unsigned short s_dy[kDy * kPitchE];
  __shared__ __attribute__((aligned(16))) unsigned short s_x[kX * kPitchE];
  const unsigned short* __restrict__ x = static_cast<const unsigned short*>(a.x);
  const unsigned short* __restrict__ dy = static_cast<const unsigned short*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int slice = bid % a.ks_count;
  const int c0 = (bid / a.ks_count) * kCh;
  const int u_begin = slice * a.units_per_slice;
  const int u_end = min(a.units, u_begin + a.units_per_slice);

  const int q = tid & 7, pslot = tid >> 3;
  const bool ch_ok = c0 + 8 * q < a.C;
  constexpr int kDyLoads = (kDy + kLoaders - 1) / kLoaders;
  constexpr int kXLoads = (kX + kLoaders - 1) / kLoaders;
  uint4 rdy[kDyLoads], rx[kXLoads];

  auto load_unit = [&](int u) {
    const int wc = u % a.wchunks;
    const int t = u / a.wchunks;
    const int hb = t % a.hblocks, n = t / a.hblocks;
    const int ho0 = hb * RU, wo0 = wc * kWoT;
#pragma unroll
    for (int i = 0; i < kDyLoads; ++i) {
      const int pp = pslot + kLoaders * i;
      const int rho = pp / kWoT, p = pp % kWoT;
      const int ho = ho0 + rho, wo = wo0 + p;
      rdy[i] = uint4{0u, 0u, 0u, 0u};
      if (ch_ok && pp < kDy && ho < a.Ho && wo < a.Wo)
        rdy[i] = *reinterpret_cast<const uint4*>(
            dy + ((int64_t)(n * a.Ho + ho) * a.Wo + wo) * a.K + c0 + 8 * q);
    }
    const int h0 = ho0 - a.pad, w0 = wo0 - a.pad;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int pp = pslot + kLoaders * i;
      const int xr = pp / XP, xp = pp % XP;
      const int h = h0 + xr, w = w0 + xp;
      rx[i] = uint4{0u, 0u, 0u, 0u};
      if (ch_ok && pp < kX && h >= 0 && h < a.H && w >= 0 && w < a.W)
        rx[i] = *reinterpret_cast<const uint4*>(
            x + (int64_t)n * a.x_img + ((int64_t)h * a.W + w) * a.C + c0 + 8 * q);
    }
  };
  const bool want_db = a.dbo != nullptr;
  float dbp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // bias partial, channels c0 + 8q ..
  auto store_unit = [&]() {
#pragma unroll
    for (int i = 0; i < kDyLoads; ++i)
      if (pslot + kLoaders * i < kDy) {
        *reinterpret_cast<uint4*>(&s_dy[(pslot + kLoaders * i) * kPitchE + 8 * q]) = rdy[i];
        if (want_db) add8<kBf16>(dbp, rdy[i]);
      }
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      if (pslot + kLoaders * i < kX)
        *reinterpret_cast<uint4*>(&s_x[(pslot + kLoaders * i) * kPitchE + 8 * q]) = rx[i];
  };

  const int j = lane & 15, g = lane >> 4;
  const int lane_off = (8 * g + (j >> 2)) * kPitchE + 16 * wave + 4 * (j & 3);
  auto tr8 = [&](const unsigned short* p) {
    return __builtin_shufflevector(tr_read(p), tr_read(p + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x4 acc[R * S];
#pragma unroll
  for (int t = 0; t < R * S; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (u_begin < u_end) load_unit(u_begin);
  for (int u = u_begin; u < u_end; ++u) {
    __syncthreads();
    store_unit();
    __syncthreads();
    if (u + 1 < u_end) load_unit(u + 1);
    s16x8 fa[RU];
#pragma unroll
    for (int t = 0; t < XR; ++t) {
      if (t < RU) fa[t] = tr8(s_dy + t * kWoT * kPitchE + lane_off);
      s16x8 fb[S];
#pragma unroll
      for (int s = 0; s < S; ++s) fb[s] = tr8(s_x + (t * XP + s) * kPitchE + lane_off);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rho = t - r;
        if (rho >= 0 && rho < RU) {
#pragma unroll
          for (int s = 0; s < S; ++s) acc[r * S + s] = mfma16<kBf16>(fa[rho], fb[s], acc[r * S + s]);
        }
      }
    }
  }

  if (want_db)
    block_sum64<32, 8>(reinterpret_cast<float*>(s_x), pslot, 8 * q, dbp,
                       a.dbo + (int64_t)slice * a.slab_stride + c0, min(kCh, a.K - c0));

  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + j;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int k = c0 + 16 * wave + 4 * g + v;
    if (k < a.K && c < a.C && k / a.Kg == c / a.Cg) {
      float* o = out + (int64_t)k * (R * S) * a.Cg + (c % a.Cg);
#pragma unroll
      for (int t = 0; t < R * S; ++t) o[t * a.Cg] = acc[t][v];
    }
  }
}

// Epilogue of the row-streaming grouped kernels: the bias partial (kDb) and the
// block-diagonal outputs.  acc[t][v] = out[k = c0 + 16*wave + 4*g + v]
// [c = c0 + 16*wave + j] for tap t; only same-group pairs are outputs.  With
// kStageOut they are gathered in `scratch` (LDS, free: every wave has passed
// the last barrier after its last tile read) in the [k][tap][c % Cg] order of
// the output, so that the workgroup writes its block of min(64, K - c0)
// output channels as whole 16-byte stores; otherwise they are stored directly.
template <int kTaps, bool kDb, bool kStageOut>
__device__ __forceinline__ void rows_epilogue(const G16Args& a, const f32x4 (&acc)[kTaps], f32x4 acc_db,
                                              int slice, int c0, float4* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  if constexpr (kDb) {
    // acc_db[v] = db partial of channel c0 + 16*wave + 4*g + v (the same in every column j).
    if (j == 0) {
      float* o = a.dbo + (int64_t)slice * a.slab_stride;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k = c0 + 16 * wave + 4 * g + v;
        if (k < a.K) o[k] = acc_db[v];
      }
    }
  }

  const int Cg = a.Cg;
  if constexpr (!kStageOut) {
    float* out = a.out + (int64_t)slice * a.slab_stride;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = c0 + 16 * wave + 4 * g + v;
      if (k < a.K && (4 * g + v) / Cg == j / Cg) {
        float* o = out + (int64_t)k * kTaps * Cg + j % Cg;
#pragma unroll
        for (int t = 0; t < kTaps; ++t) o[t * Cg] = acc[t][v];
      }
    }
    return;
  }
  float* s_out = reinterpret_cast<float*>(scratch);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int kl = 16 * wave + 4 * g + v;
    if ((4 * g + v) / Cg == j / Cg) {
#pragma unroll
      for (int t = 0; t < kTaps; ++t) s_out[(kl * kTaps + t) * Cg + j % Cg] = acc[t][v];
    }
  }
  __syncthreads();
  const int n4 = min(kCh, a.K - c0) * kTaps * Cg / 4;
  float4* out = reinterpret_cast<float4*>(a.out + (int64_t)slice * a.slab_stride + (int64_t)c0 * kTaps * Cg);
  for (int i = tid; i < n4; i += 256) out[i] = scratch[i];
}

// Row-streaming path for stride 1, dilation 1, Wo <= 64 and a compile-time
// R x S filter.  A workgroup owns 64 channels and a slice of output rows of
// one image at a time.  Each step brings kRows X rows (34 pixels with the
// padding columns) and kRows dY rows into LDS (double-buffered, one barrier
// per step) with 16-byte buffer loads that run kPf steps ahead; the buffer
// range of a row supplies its zero padding, and rows outside the image or the
// segment have an empty range.  The A operand of each dY row is read once and
// kept in registers for the R rows that use it; X row h is read at its S
// column offsets and multiplied with the A operands of output rows
// h + pad - r, so every staged element is read from HBM once per slice.
// kDb: also the bias gradient (a separate instantiation keeps the plain
// kernel's MFMA loop unchanged).  Only the W image pixels of an X row are
// loaded (one 16-byte chunk per lane, kNXL passes of 32 pixels, kWide when
// W > WT); they land at slot pad + w and the padding slots are zeroed once,
// so no load instruction is spent on padding columns.  Padding rows are not
// staged either: the steps cover only the X rows inside the image, and the
// up to R - 1 dY rows that pair with the padding rows above the first one
// are fetched with the segment's first loads and enter the A-operand shift
// register before its first step.
template <bool kBf16, int R, int S, bool kDb, int WT, bool kWide>
__global__ __launch_bounds__(256) void grouped16_rows_kernel(G16Args a) {
  constexpr int kXPixR = WT + S - 1;              // staged X pixels per row
  constexpr int kKs = WT / 32;                    // 32-pixel MFMA k-steps per row
  constexpr int kNXL = WT / 32 + (kWide ? 1 : 0); // X load passes per row (W <= 32 * kNXL)
  constexpr int kRows = 2;                        // rows per step (one barrier)
  constexpr int kPf = 2;                          // steps fetched ahead (even)
  // The output block (16 channels per group at most) is gathered in LDS when
  // it fits in the row tiles (1x1, 3x3); larger filters store it directly.
  constexpr int kPre = R - 1;                     // dY rows that enter before the first step
  struct Tiles {
    unsigned short x[2][kRows][kXPixR * kPitchE];
    unsigned short dy[2][kRows][WT * kPitchE];
    unsigned short pre[kPre > 0 ? kPre : 1][kPre > 0 ? WT * kPitchE : 8];
  };
  constexpr int kOut = kCh * R * S * 16;
  constexpr bool kStageOut = kOut * 4 <= (int)sizeof(Tiles);
  union Smem {
    Tiles t;
    float4 out[kStageOut ? kOut / 4 : 1];
  };
  static_assert(sizeof(Smem) == sizeof(Tiles), "the output block fits in the row tiles");
  __shared__ __attribute__((aligned(16))) Smem sm;
  auto& s_x = sm.t.x;
  auto& s_dy = sm.t.dy;
  auto& s_pre = sm.t.pre;
  const unsigned char* __restrict__ xg = static_cast<const unsigned char*>(a.x);
  const unsigned char* __restrict__ dyg = static_cast<const unsigned char*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Work item w = (slice, channel block), channel block fastest; the grid is
  // a multiple of 8 and block b runs on XCD b % 8, so XCD x takes the items
  // [x * per_xcd, (x + 1) * per_xcd): the channel blocks of a slice, which
  // read the same pixel rows at the same time, share one L2.
  const int work = a.c_blocks * a.ks_count;
  const int per_xcd = (work + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= work) return;
  const int cb = w % a.c_blocks;
  const int slice = w / a.c_blocks;
  const int c0 = cb * kCh;
  const int r_begin = slice * a.units_per_slice;
  const int r_end = min(a.units, r_begin + a.units_per_slice);   // units are output rows

  // Loader role: image pixels ps + 32 i of an X row (kNXL passes), dY pixels
  // ps + 32 i (kKs passes), 16-byte chunk q.
  const int q = tid & 7, ps = tid >> 3;
  const int x_row_bytes = (a.W * a.C - c0) * 2;
  const int dy_row_bytes = (a.Wo * a.K - c0) * 2;
  int ox[kNXL], ody[kKs];
#pragma unroll
  for (int i = 0; i < kNXL; ++i)   // offsets past the range read zero
    ox[i] = ps + 32 * i < a.W ? ((ps + 32 * i) * a.C + 8 * q) * 2 : 0x7fffffff;
#pragma unroll
  for (int i = 0; i < kKs; ++i) ody[i] = ((ps + 32 * i) * a.K + 8 * q) * 2;
  struct Row {
    uint4 x[kNXL], d[kKs];
  };
  struct Step {
    Row row[kRows];
  };
  // Segment: output rows [ho0, ho_hi) of image n.  Its X rows inside the
  // image are hx0 .. hx0 + ev - 1; row u of the segment is X row hx0 + u
  // (u < ev) and dY row hx0 + pad + u (the row that meets X row hx0 + u at
  // filter row 0; zero from ho_hi on).  Row ho = h + pad - r meets X row h at
  // filter row r, so the X rows below hx0 and from hx0 + ev on meet only
  // zero padding or rows outside the segment.
  int n = 0, ho0 = 0, ho_hi = 0, hx0 = 0, ev = 0;
  auto fetch_row = [&](int u, Row& st) {
    const int h = hx0 + u;
    const bool x_in = u < ev;
    const __amdgpu_buffer_rsrc_t rx =
        buf_rsrc(xg + 2 * ((int64_t)n * a.x_img + (int64_t)(x_in ? h : 0) * a.W * a.C + c0),
                 x_in ? x_row_bytes : 0);
#pragma unroll
    for (int i = 0; i < kNXL; ++i)
      st.x[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ox[i], 0, 0));
    const int ho = hx0 + a.pad + u;
    const bool d_in = ho < ho_hi;
    const __amdgpu_buffer_rsrc_t rd =
        buf_rsrc(dyg + 2 * (((int64_t)n * a.Ho + (d_in ? ho : ho0)) * a.Wo * a.K + c0),
                 d_in ? dy_row_bytes : 0);
#pragma unroll
    for (int i = 0; i < kKs; ++i)
      st.d[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, ody[i], 0, 0));
  };
  // dY rows hx0 + pad - 1 - i (i < R - 1): the rows that the shift register
  // holds at row 0 in its places 1 + i (zero outside the segment).
  uint4 pre[kPre > 0 ? kPre : 1][kKs];
  auto fetch_pre = [&]() {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int ho = hx0 + a.pad - 1 - i;
      const bool d_in = ho >= ho0 && ho < ho_hi;
      const __amdgpu_buffer_rsrc_t rd =
          buf_rsrc(dyg + 2 * (((int64_t)n * a.Ho + (d_in ? ho : ho0)) * a.Wo * a.K + c0),
                   d_in ? dy_row_bytes : 0);
#pragma unroll
      for (int k = 0; k < kKs; ++k)
        pre[i][k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, ody[k], 0, 0));
    }
  };
  auto fetch = [&](int t, Step& st) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) fetch_row(kRows * t + i, st.row[i]);
  };
  auto store = [&](int buf, const Step& st) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
#pragma unroll
      for (int x = 0; x < kNXL; ++x)
        if (ps + 32 * x < a.W)
          *reinterpret_cast<uint4*>(&s_x[buf][i][(ps + 32 * x + a.pad) * kPitchE + 8 * q]) = st.row[i].x[x];
#pragma unroll
      for (int x = 0; x < kKs; ++x)
        *reinterpret_cast<uint4*>(&s_dy[buf][i][(ps + 32 * x) * kPitchE + 8 * q]) = st.row[i].d[x];
    }
  };

  const int j = lane & 15, g = lane >> 4;
  const int lane_off = (8 * g + (j >> 2)) * kPitchE + 16 * wave + 4 * (j & 3);
  auto tr8 = [&](const unsigned short* p) {
    return __builtin_shufflevector(tr_read(p), tr_read(p + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x4 acc[R * S];
#pragma unroll
  for (int t = 0; t < R * S; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Bias gradient: each dY row's A operand (fa[0] when the row enters) times a
  // B operand of ones gives, in every column, the row's sum per output
  // channel; every dY row of a segment enters once, before the first step or
  // at its row (rows outside the segment are zero).
  f32x4 acc_db = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned short one = kBf16 ? 0x3f80 : 0x3c00;
  const s16x8 ones{(short)one, (short)one, (short)one, (short)one,
                   (short)one, (short)one, (short)one, (short)one};

  Step pf[kPf];
  int row = r_begin, seg = 0, steps = 0;
  // Sets up the segment that starts at output row `row` and issues its first
  // loads: the rows before its first step, then kPf steps.
  auto begin_segment = [&]() {
    n = row / a.Ho;
    ho0 = row % a.Ho;
    seg = min(r_end - row, a.Ho - ho0);
    ho_hi = ho0 + seg;
    hx0 = max(0, ho0 - a.pad);
    ev = min(a.H, ho_hi + R - 1 - a.pad) - hx0;   // >= 1 (pad < R, ho0 < Ho)
    steps = (ev + kRows - 1) / kRows;
    fetch_pre();
#pragma unroll
    for (int k = 0; k < kPf; ++k) fetch(k, pf[k]);
  };
  if (row < r_end) begin_segment();
  // X slots [0, pad) and [pad + W, kXPixR) of every row buffer hold the zero
  // padding; the stores below never touch them.  (Written while the first
  // loads are in flight; the barrier before the first step orders them.)
  for (int e = tid; e < 2 * kRows * kXPixR * 8; e += 256) {
    const int slot = (e >> 3) % kXPixR;
    if (slot < a.pad || slot >= a.pad + a.W)
      *reinterpret_cast<uint4*>(&s_x[e / (8 * kRows * kXPixR)][(e / (8 * kXPixR)) % kRows][slot * kPitchE + 8 * (e & 7)]) =
          uint4{0u, 0u, 0u, 0u};
  }
  while (row < r_end) {
    // A operands of dY rows hx0 + pad + u - r, r = 0..R-1, per k-step at row u.
    // Each row shifts the register up one place before its new row enters in
    // place 0, so the rows before the first step start in places 0..R-2.
    s16x8 fa[R][kKs];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int kk = 0; kk < kKs; ++kk) fa[r][kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (kPre > 0) {
#pragma unroll
      for (int i = 0; i < kPre; ++i)
#pragma unroll
        for (int x = 0; x < kKs; ++x)
          *reinterpret_cast<uint4*>(&s_pre[i][(ps + 32 * x) * kPitchE + 8 * q]) = pre[i][x];
      lds_barrier();
#pragma unroll
      for (int i = 0; i < kPre; ++i)
#pragma unroll
        for (int kk = 0; kk < kKs; ++kk) {
          fa[i][kk] = tr8(&s_pre[i][32 * kk * kPitchE + lane_off]);
          if constexpr (kDb) acc_db = mfma16<kBf16>(fa[i][kk], ones, acc_db);
        }
    }
    for (int t = 0; t < steps; t += kPf) {
#pragma unroll
      for (int k = 0; k < kPf; ++k) {
        const int tk = t + k;
        store(k & 1, pf[k]);
        fetch(tk + kPf, pf[k]);
        lds_barrier();
        if (tk < steps) {
          // Rows past the segment's ev rows hold zero X and dY.
#pragma unroll
          for (int i = 0; i < kRows; ++i) {
#pragma unroll
            for (int r = R - 1; r > 0; --r)
#pragma unroll
              for (int kk = 0; kk < kKs; ++kk) fa[r][kk] = fa[r - 1][kk];
#pragma unroll
            for (int kk = 0; kk < kKs; ++kk) {
              fa[0][kk] = tr8(&s_dy[k & 1][i][32 * kk * kPitchE + lane_off]);
              if constexpr (kDb) acc_db = mfma16<kBf16>(fa[0][kk], ones, acc_db);
              s16x8 fb[S];
#pragma unroll
              for (int s2 = 0; s2 < S; ++s2)
                fb[s2] = tr8(&s_x[k & 1][i][(32 * kk + s2) * kPitchE + lane_off]);
#pragma unroll
              for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s2 = 0; s2 < S; ++s2)
                  acc[r * S + s2] = mfma16<kBf16>(fa[r][kk], fb[s2], acc[r * S + s2]);
            }
          }
        }
      }
    }
    // The next segment restarts at buffer 0; all waves finish this one first.
    lds_barrier();
    row += seg;
    if (row < r_end) begin_segment();
  }

  constexpr int kTaps = R * S;
  rows_epilogue<kTaps, kDb, kStageOut>(a, acc, acc_db, slice, c0, reinterpret_cast<float4*>(&sm));
}


// Row-streaming path for stride 2 (dilation 1, Wo <= 32, compile-time R x S).
// Output row ho reads X rows 2 ho - pad + r, so each step brings two X rows
// and one dY row: X row 2t + i (i = 0, 1) of the segment meets the filter
// rows r with r = i mod 2, whose dY rows t - (r - i) / 2 have A operands in a
// shift register of (R + 1) / 2 rows.  Tap s reads X column 2 wo - pad + s:
// the X rows are staged de-interleaved (even and odd staged columns in two
// regions), so that the 32 pixels of one tap are consecutive in one region
// and the transposed reads work as for stride 1.
template <bool kBf16, int R, int S, bool kDb>
__global__ __launch_bounds__(256) void grouped16_rows_s2_kernel(G16Args a) {
  constexpr int kReg = kWoT + (S - 1) / 2;        // pixels per parity region
  constexpr int kXCols = 2 * kReg;                // staged X columns -pad .. -pad + kXCols - 1
  constexpr int kPf = 2;
  constexpr int kNA = (R + 1) / 2;                // dY rows in flight per X row pair
  struct Tiles {
    unsigned short x[2][2][kXCols * kPitchE];     // [buffer][row of the pair][region * kReg + index]
    unsigned short dy[2][kWoT * kPitchE];
  };
  constexpr int kOut = kCh * R * S * 16;
  constexpr bool kStageOut = kOut * 4 <= (int)sizeof(Tiles);
  __shared__ __attribute__((aligned(16))) Tiles sm;
  auto& s_x = sm.x;
  auto& s_dy = sm.dy;
  const unsigned char* __restrict__ xg = static_cast<const unsigned char*>(a.x);
  const unsigned char* __restrict__ dyg = static_cast<const unsigned char*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int work = a.c_blocks * a.ks_count;
  const int per_xcd = (work + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= work) return;
  const int cb = w % a.c_blocks;
  const int slice = w / a.c_blocks;
  const int c0 = cb * kCh;
  const int r_begin = slice * a.units_per_slice;
  const int r_end = min(a.units, r_begin + a.units_per_slice);   // units are output rows

  // Loader role: staged columns ps, ps + 32, ps + 64, 16-byte chunk q.
  const int q = tid & 7, ps = tid >> 3;
  const int x_row_bytes = (a.W * a.C - c0) * 2;
  const int dy_row_bytes = (a.Wo * a.K - c0) * 2;
  int ox[3];
#pragma unroll
  for (int i = 0; i < 3; ++i)
    ox[i] = ps + 32 * i < kXCols ? ((ps + 32 * i - a.pad) * a.C + 8 * q) * 2 : 0x7fffffff;
  const int ody = (ps * a.K + 8 * q) * 2;
  struct Step {
    uint4 x[2][3], d;
  };
  int n = 0, ho0 = 0, ho_hi = 0, rows_x = 0;
  // Step t: X rows 2 ho0 - pad + 2t + i of the segment, dY row ho0 + t.
  auto fetch = [&](int t, Step& st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 2 * t + i;
      const int h = 2 * ho0 - a.pad + u;
      const bool x_in = h >= 0 && h < a.H && u < rows_x;
      const __amdgpu_buffer_rsrc_t rx =
          buf_rsrc(xg + 2 * ((int64_t)n * a.x_img + (int64_t)(x_in ? h : 0) * a.W * a.C + c0),
                   x_in ? x_row_bytes : 0);
#pragma unroll
      for (int k = 0; k < 3; ++k)
        st.x[i][k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ox[k], 0, 0));
    }
    const int ho = ho0 + t;
    const bool d_in = ho < ho_hi;
    const __amdgpu_buffer_rsrc_t rd =
        buf_rsrc(dyg + 2 * (((int64_t)n * a.Ho + (d_in ? ho : ho0)) * a.Wo * a.K + c0),
                 d_in ? dy_row_bytes : 0);
    st.d = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, ody, 0, 0));
  };
  auto store = [&](int buf, const Step& st) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int col = ps + 32 * k;   // staged column: region col & 1, index col >> 1
        if (col < kXCols)
          *reinterpret_cast<uint4*>(&s_x[buf][i][((col & 1) * kReg + (col >> 1)) * kPitchE + 8 * q]) =
              st.x[i][k];
      }
    *reinterpret_cast<uint4*>(&s_dy[buf][ps * kPitchE + 8 * q]) = st.d;
  };

  const int j = lane & 15, g = lane >> 4;
  const int lane_off = (8 * g + (j >> 2)) * kPitchE + 16 * wave + 4 * (j & 3);
  auto tr8 = [&](const unsigned short* p) {
    return __builtin_shufflevector(tr_read(p), tr_read(p + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x4 acc[R * S];
#pragma unroll
  for (int t = 0; t < R * S; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc_db = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned short one = kBf16 ? 0x3f80 : 0x3c00;
  const s16x8 ones{(short)one, (short)one, (short)one, (short)one,
                   (short)one, (short)one, (short)one, (short)one};

  Step pf[kPf];
  int row = r_begin;
  while (row < r_end) {
    n = row / a.Ho;
    ho0 = row % a.Ho;
    const int seg = min(r_end - row, a.Ho - ho0);
    ho_hi = ho0 + seg;
    rows_x = 2 * (seg - 1) + R;   // X rows 2 ho0 - pad .. 2 (ho0 + seg - 1) - pad + R - 1
    const int steps = (rows_x + 1) / 2;
    // fa[m] = A operand of dY row ho0 + t - m (zero before the segment).
    s16x8 fa[kNA];
#pragma unroll
    for (int m = 0; m < kNA; ++m) fa[m] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kPf; ++k) fetch(k, pf[k]);
    for (int t = 0; t < steps; t += kPf) {
#pragma unroll
      for (int k = 0; k < kPf; ++k) {
        const int tk = t + k;
        store(k & 1, pf[k]);
        fetch(tk + kPf, pf[k]);
        lds_barrier();
        if (tk < steps) {
#pragma unroll
          for (int m = kNA - 1; m > 0; --m) fa[m] = fa[m - 1];
          fa[0] = tr8(&s_dy[k & 1][lane_off]);
          if constexpr (kDb) acc_db = mfma16<kBf16>(fa[0], ones, acc_db);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            s16x8 fb[S];
#pragma unroll
            for (int s2 = 0; s2 < S; ++s2)
              fb[s2] = tr8(&s_x[k & 1][i][((s2 & 1) * kReg + (s2 >> 1)) * kPitchE + lane_off]);
#pragma unroll
            for (int r = i; r < R; r += 2)
#pragma unroll
              for (int s2 = 0; s2 < S; ++s2)
                acc[r * S + s2] = mfma16<kBf16>(fa[(r - i) / 2], fb[s2], acc[r * S + s2]);
          }
        }
      }
    }
    lds_barrier();
    row += seg;
  }
  rows_epilogue<R * S, kDb, kStageOut>(a, acc, acc_db, slice, c0, reinterpret_cast<float4*>(&sm));
}

}  // namespace

hipError_t launch_grouped16(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                            hipStream_t stream) {
  const Problem& p = plan.p;
  G16Args a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo; a.R = (int32_t)p.R; a.S = (int32_t)p.S;
  a.pad = (int32_t)p.pad; a.dil = (int32_t)p.dil;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.taps = (int32_t)(p.R * p.S);
  a.ru = plan.ru;
  a.hblocks = plan.ru > 0 ? (int32_t)ceil_div(p.Ho, plan.ru) : 0;   // unit-row kernels only
  a.wchunks = (int32_t)ceil_div(p.Wo, kWoT);
  a.xrows = plan.xrows;
  a.xpix = plan.xspan;
  a.c_blocks = (int32_t)ceil_div(p.C, kCh);
  a.units = (int32_t)plan.pub.units;
  a.units_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.dbo = out.db;
  const dim3 grid((unsigned)plan.pub.grid), block(256);
  const bool bf = p.dtype == CONV_WGRAD_BF16;
  if (plan.pub.variant == kGrouped16Rows) {
    const dim3 xcd_grid((unsigned)(ceil_div(plan.pub.grid, 8) * 8));
    const bool db = a.dbo != nullptr;
    if (p.stride == 2) {
#define CW_G16S2(RR)                                                                                \
      if (p.R == RR) {                                                                              \
        if (db)                                                                                     \
          return bf ? launch_kernel(grouped16_rows_s2_kernel<true, RR, RR, true>, xcd_grid, block, a, stream)  \
                    : launch_kernel(grouped16_rows_s2_kernel<false, RR, RR, true>, xcd_grid, block, a, stream); \
        return bf ? launch_kernel(grouped16_rows_s2_kernel<true, RR, RR, false>, xcd_grid, block, a, stream)    \
                  : launch_kernel(grouped16_rows_s2_kernel<false, RR, RR, false>, xcd_grid, block, a, stream);  \
      }
      CW_G16S2(1)
      CW_G16S2(3)
      CW_G16S2(5)
      CW_G16S2(7)
#undef CW_G16S2
      return hipErrorInvalidValue;
    }
#define CW_G16R_W(RR, WW, XW)                                                                     \
    if (p.R == RR && wt == WW && wide == XW) {                                                   \
      if (db)                                                                                    \
        return bf ? launch_kernel(grouped16_rows_kernel<true, RR, RR, true, WW, XW>, xcd_grid, block, a, stream) \
                  : launch_kernel(grouped16_rows_kernel<false, RR, RR, true, WW, XW>, xcd_grid, block, a, stream); \
      return bf ? launch_kernel(grouped16_rows_kernel<true, RR, RR, false, WW, XW>, xcd_grid, block, a, stream)   \
                : launch_kernel(grouped16_rows_kernel<false, RR, RR, false, WW, XW>, xcd_grid, block, a, stream); \
    }
#define CW_G16R(RR) CW_G16R_W(RR, 32, false) CW_G16R_W(RR, 64, false) CW_G16R_W(RR, 32, true) CW_G16R_W(RR, 64, true)
    const int wt = p.Wo > 32 ? 64 : 32;
    const bool wide = p.W > wt;   // a row has more image pixels than one pass per k-step
    CW_G16R(1)
    CW_G16R(3)
    CW_G16R(5)
    CW_G16R(7)
#undef CW_G16R
#undef CW_G16R_W
    return hipErrorInvalidValue;
  }
  if (plan.ru == 4 && p.dil == 1 && p.R == 3 && p.S == 3)
    return bf ? launch_kernel(grouped16_win_kernel<true, 3, 3>, grid, block, a, stream)
              : launch_kernel(grouped16_win_kernel<false, 3, 3>, grid, block, a, stream);
  if (plan.ru == 4 && p.dil == 1 && p.R == 1 && p.S == 1)
    return bf ? launch_kernel(grouped16_win_kernel<true, 1, 1>, grid, block, a, stream)
              : launch_kernel(grouped16_win_kernel<false, 1, 1>, grid, block, a, stream);
  if (p.R == 3 && p.S == 3)
    return bf ? launch_kernel(grouped16_kernel<true, 3, 3>, grid, block, a, stream)
              : launch_kernel(grouped16_kernel<false, 3, 3>, grid, block, a, stream);
  if (p.R == 1 && p.S == 1)
    return bf ? launch_kernel(grouped16_kernel<true, 1, 1>, grid, block, a, stream)
              : launch_kernel(grouped16_kernel<false, 1, 1>, grid, block, a, stream);
  return bf ? launch_kernel(grouped16_kernel<true, 0, 0>, grid, block, a, stream)
            : launch_kernel(grouped16_kernel<false, 0, 0>, grid, block, a, stream);
}

}  // namespace cw
