// Dense implicit-GEMM weight gradient for 16-bit inputs on 16x16x32 MFMA (gfx950).
//
// The GEMM of the dense kernels (per group: M = Kg output channels,
// N = R*S*Cg columns, reduction over the output pixels), with bf16 / fp16
// operands on v_mfma_f32_16x16x32_{bf16,f16} and fp32 accumulation, for
// stride 1 and dilation 1:
//
//   * a reduction unit is a run of up to 64 output pixels of one output row;
//     a workgroup tile is (group, 64 output channels, filter row r, SB
//     consecutive taps, 64 input channels), as in the fp32 row kernel;
//   * the unit's 64 dY pixels and the 68 X pixels the taps need are staged in
//     LDS in their NHWC order (64 channels per pixel, 160-byte pixel pitch)
//     by 16-byte buffer loads whose range supplies the zero padding;
//   * the MFMA operands hold 8 consecutive pixels of one channel per lane, a
//     transpose of that layout, which ds_read_b64_tr_b16 does on the read:
//     within a 16-lane group lane j points at 4 channels of pixel j / 4 and
//     lane i receives channel i of 4 consecutive pixels.  Tap s's B operand is
//     the X segment read s pixels further on: an address offset;
//   * wave w owns input channels 16w .. 16w + 15 of the tile and all 64 output
//     channels: 4 A operands (dY) and SB B operands (X) per 32 pixels feed
//     4 * SB accumulators;
//   * two LDS buffers alternate: a unit is staged while the previous one is
//     computed, one barrier per unit;
//   * short rows (Wo + SB - 1 <= 32): a unit is ru = 64 / P consecutive output
//     rows staged at a pitch of P = Wo + SB - 1 pixels -- dY row j in slots
//     j*P .. j*P + Wo - 1 followed by zeros, its X segment in slots
//     j*P .. j*P + P - 1 -- so tap s is still the shift by s slots (a product
//     that crosses into the next row's segment meets a zero dY column), and a
//     14-pixel row no longer occupies a whole 64-pixel unit.
//
// BF16x3 mode (fp32 inputs, math = BF16X3; the gfx950 form of fp32 matrix
// work in rocm-libraries PR #14393, timeline, the TF32 entry): the loaders
// read fp32 and split every value v at staging into hi = bf16(v) and
// lo = bf16(v - hi) (both round-to-nearest-even, v - hi exact in fp32), kept
// in two LDS planes; each product is a_hi*b_hi + a_hi*b_lo + a_lo*b_hi, three
// bf16 MFMAs into the same fp32 accumulator.  The bias gradient is then summed
// from the fp32 values at staging (exact fp32 adds), not through the MFMA.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kPitchE = 80;      // 16-bit elements per staged pixel (64 channels + pad)
constexpr int kWt = 64;          // dY pixels staged per unit (two 32-pixel k-steps)
constexpr int kXUse = 68;        // X pixels a unit's MFMAs read (64 + up to 3 tap shifts)
constexpr int kDyChunks = kWt * 8 / 256;                  // 16-byte loads per lane for dY
constexpr int kXChunks = (kXUse * 8 + 255) / 256;         // and for X
constexpr int kXs = kXChunks * 32;                        // X pixel rows staged: every loader chunk has one

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct R16Args {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;   // H*W*C
  int32_t H, W, C, K, Ho, Wo, R, S, pad_h, pad_w;
  int32_t Cg, Kg, cols;
  int32_t m_tiles, c_tiles, s_blocks;
  int32_t wt, wchunks;
  int32_t ru, pitch, hblocks;   // output rows per unit, staging pitch, ceil(Ho / ru)
  int32_t units, units_per_slice, ks_count;
  int32_t tiles, work;
  float* dbo;      // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
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

// Split of 8 fp32 values into 8 bf16 high parts and 8 bf16 low parts
// (round-to-nearest-even; v - hi is exact in fp32).
__device__ __forceinline__ void split_bf16x8(uint4 v0, uint4 v1, uint4& hi, uint4& lo) {
  const float f[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z), __uint_as_float(v0.w),
                      __uint_as_float(v1.x), __uint_as_float(v1.y), __uint_as_float(v1.z), __uint_as_float(v1.w)};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h0 = (__bf16)f[2 * i], h1 = (__bf16)f[2 * i + 1];
    const __bf16 l0 = (__bf16)(f[2 * i] - (float)h0), l1 = (__bf16)(f[2 * i + 1] - (float)h1);
    h[i] = (uint32_t)__builtin_bit_cast(unsigned short, h0) | ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
    l[i] = (uint32_t)__builtin_bit_cast(unsigned short, l0) | ((uint32_t)__builtin_bit_cast(unsigned short, l1) << 16);
  }
  hi = uint4{h[0], h[1], h[2], h[3]};
  lo = uint4{l[0], l[1], l[2], l[3]};
}

// kDb: also the bias gradient (a separate instantiation).  kX3: fp32 inputs
// by BF16x3 (kBf16 is then true).  kMulti: units of several short rows.
// kSets: register sets of unit loads in flight.  The loop runs whole rounds
// of kSets units, each set with its own registers (no copies between sets),
// and every load is issued unconditionally -- units past the slice have empty
// buffer ranges and read zero, their MFMAs are skipped -- so the waits at a
// set's staging count only that set's loads.
template <bool kBf16, int SB, bool kDb, bool kX3, bool kMulti, int kSets>
__global__ __launch_bounds__(256) void dense16_rows_kernel(R16Args a) {
  constexpr int kEs = kX3 ? 4 : 2;          // bytes per input element
  constexpr int kLd = kX3 ? 2 : 1;          // 16-byte loads per 8-channel chunk
  constexpr int kPlanes = kX3 ? 2 : 1;      // hi (and lo) planes
  __shared__ __attribute__((aligned(16))) unsigned short s_dy[kPlanes][2][kWt * kPitchE];
  __shared__ __attribute__((aligned(16))) unsigned short s_x[kPlanes][2][kXs * kPitchE];
  const unsigned char* __restrict__ xg = static_cast<const unsigned char*>(a.x);
  const unsigned char* __restrict__ dyg = static_cast<const unsigned char*>(a.dy);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work item w = slice * tiles + tile; XCD x (block b runs on XCD b % 8)
  // takes a contiguous run of items, so the tiles of a slice share one L2.
  const int per_xcd = (a.work + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || w >= a.work) return;
  const int slice = w / a.tiles;
  int tile = w % a.tiles;
  const int ct = tile % a.c_tiles;
  tile /= a.c_tiles;
  const int sb = tile % a.s_blocks;
  tile /= a.s_blocks;
  const int r = tile % a.R;
  tile /= a.R;
  const int mt = tile % a.m_tiles;
  const int g = tile / a.m_tiles;
  const int m0 = mt * 64, c0 = ct * 64, s0 = sb * SB;
  const int u_begin = slice * a.units_per_slice;
  const int u_end = min(a.units, u_begin + a.units_per_slice);

  // Loader role: chunk t + 256 i = (pixel (t + 256 i) / 8, 8 channels at 8 * (t % 8)).
  const int q8 = tid & 7, px0 = tid >> 3;
  const int dy_col0 = g * a.Kg + m0;
  const int x_col0 = g * a.Cg + c0;
  const int x_row_bytes = (a.W * a.C - x_col0) * kEs;
  struct Set {
    uint4 dy[kDyChunks][kLd], x[kXChunks][kLd];
    int npix;   // output pixel slots the unit fills (0 past the slice)
  };
  // Multi-row units: slot p of a loader chunk is row p / pitch, column p % pitch.
  int dj[kDyChunks], dcol[kDyChunks], xj[kXChunks], xcol[kXChunks];
  if constexpr (kMulti) {
#pragma unroll
    for (int i = 0; i < kDyChunks; ++i) { dj[i] = (px0 + 32 * i) / a.pitch; dcol[i] = (px0 + 32 * i) % a.pitch; }
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) { xj[i] = (px0 + 32 * i) / a.pitch; xcol[i] = (px0 + 32 * i) % a.pitch; }
  }
  // The loads take the slice's units in order, so the next unit's coordinates
  // are a cursor advanced by one per load (no divisions in the loop):
  // multi-row units (n, row block cb), single-row units (n, ho, chunk wc).
  int cur_n, cur_ho = 0, cur_w = 0;
  if constexpr (kMulti) {
    cur_n = u_begin / a.hblocks;
    cur_ho = u_begin % a.hblocks;
  } else {
    cur_w = u_begin % a.wchunks;
    const int t0 = u_begin / a.wchunks;
    cur_ho = t0 % a.Ho;
    cur_n = t0 / a.Ho;
  }
  const int n_first = cur_n, ho_first = cur_ho, w_first = cur_w;
  auto advance = [&]() {
    if constexpr (kMulti) {
      if (++cur_ho == a.hblocks) { cur_ho = 0; ++cur_n; }
    } else {
      if (++cur_w == a.wchunks) {
        cur_w = 0;
        if (++cur_ho == a.Ho) { cur_ho = 0; ++cur_n; }
      }
    }
  };
  // Unit u of the slice (the cursor's) into set st; a unit past the slice
  // (u >= u_end) addresses the slice's first unit with empty ranges, so it
  // reads zero.
  auto load_unit = [&](int u, Set& st) {
    const bool live = u < u_end;
    const int un = live ? cur_n : n_first, uho = live ? cur_ho : ho_first, uw = live ? cur_w : w_first;
    if (live) advance();
    if constexpr (kMulti) {
      const int n = un, ho0 = uho * a.ru;
      const int rows = live ? min(a.ru, a.Ho - ho0) : 0;
      st.npix = live ? a.ru * a.pitch : 0;
      // dY rows ho0 .. ho0 + rows - 1 are contiguous; columns past Wo and rows
      // past the unit read zero.
      const unsigned char* dyp = dyg + kEs * (((int64_t)(n * a.Ho + ho0) * a.Wo) * a.K + dy_col0);
      const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dyp, rows > 0 ? (rows * a.Wo * a.K - dy_col0) * kEs : 0);
#pragma unroll
      for (int i = 0; i < kDyChunks; ++i) {
        const bool ok = dcol[i] < a.Wo && dj[i] < rows;
        const int off = ok ? ((dj[i] * a.Wo + dcol[i]) * a.K + 8 * q8) * kEs : 0x7fffffe0;
#pragma unroll
        for (int h = 0; h < kLd; ++h)
          st.dy[i][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, off + 16 * h, 0, 0));
      }
      // X rows h0 + j of the unit (filter row r), columns w0 .. w0 + pitch - 1;
      // rows and columns outside the image read zero.
      const int h0 = ho0 + r - a.pad_h;
      const int hb = max(h0, 0), he = min(h0 + rows, a.H);
      const int w0 = s0 - a.pad_w;
      const unsigned char* xp = xg + kEs * ((int64_t)n * a.x_img + (int64_t)hb * a.W * a.C + x_col0);
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(xp, he > hb ? ((he - hb) * a.W * a.C - x_col0) * kEs : 0);
#pragma unroll
      for (int i = 0; i < kXChunks; ++i) {
        const int h = h0 + xj[i], w = w0 + xcol[i];
        const bool ok = xj[i] < rows && h >= hb && h < he && w >= 0 && w < a.W;
        const int off = ok ? (((h - hb) * a.W + w) * a.C + 8 * q8) * kEs : 0x7fffffe0;
#pragma unroll
        for (int hh = 0; hh < kLd; ++hh)
          st.x[i][hh] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * hh, 0, 0));
      }
    } else {
      const int wc = uw, ho = uho, n = un;
      const int wo0 = wc * a.wt;
      const int npix = live ? min(a.wt, a.Wo - wo0) : 0;
      st.npix = npix;
      const unsigned char* dyp = dyg + kEs * (((int64_t)(n * a.Ho + ho) * a.Wo + wo0) * a.K + dy_col0);
      const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dyp, npix > 0 ? (npix * a.K - dy_col0) * kEs : 0);
#pragma unroll
      for (int i = 0; i < kDyChunks; ++i)
#pragma unroll
        for (int h = 0; h < kLd; ++h)
          st.dy[i][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rd, ((px0 + 32 * i) * a.K + 8 * q8) * kEs + 16 * h, 0, 0));
      const int h = ho + r - a.pad_h;
      const bool row_ok = live && h >= 0 && h < a.H;
      const unsigned char* xp = xg + kEs * ((int64_t)n * a.x_img + (int64_t)(row_ok ? h : 0) * a.W * a.C + x_col0);
      const int w0 = wo0 - a.pad_w + s0;   // first staged X column (negative: padding, reads zero)
      // The MFMAs use X columns up to w0 + npix + SB - 2; the loader chunks
      // past them (the rest of 96 staged slots) read zero instead of memory.
      const int x_used = (w0 + npix + SB - 1) * a.C * kEs;
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(xp, row_ok ? max(0, min(x_row_bytes, x_used)) : 0);
#pragma unroll
      for (int i = 0; i < kXChunks; ++i)
#pragma unroll
        for (int hh = 0; hh < kLd; ++hh)
          st.x[i][hh] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rs, ((w0 + px0 + 32 * i) * a.C + 8 * q8) * kEs + 16 * hh, 0, 0));
    }
  };
  // BF16x3: per-thread fp32 sums of the staged dY values (8 channels at 8 q8
  // for every loader pixel row), for the bias gradient.
  const bool db_x3 = kX3 && kDb && r == 0 && sb == 0 && ct == 0;
  float dbp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto store_unit = [&](int buf, const Set& st) {
#pragma unroll
    for (int i = 0; i < kDyChunks; ++i) {
      unsigned short* d = &s_dy[0][buf][(px0 + 32 * i) * kPitchE + 8 * q8];
      if constexpr (kX3) {
        uint4 hi, lo;
        split_bf16x8(st.dy[i][0], st.dy[i][kLd - 1], hi, lo);
        *reinterpret_cast<uint4*>(d) = hi;
        *reinterpret_cast<uint4*>(&s_dy[kPlanes - 1][buf][(px0 + 32 * i) * kPitchE + 8 * q8]) = lo;
        if (db_x3) {
          const uint32_t w[8] = {st.dy[i][0].x, st.dy[i][0].y, st.dy[i][0].z, st.dy[i][0].w,
                                 st.dy[i][kLd - 1].x, st.dy[i][kLd - 1].y, st.dy[i][kLd - 1].z,
                                 st.dy[i][kLd - 1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) dbp[e] += __uint_as_float(w[e]);
        }
      } else {
        *reinterpret_cast<uint4*>(d) = st.dy[i][0];
      }
    }
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      unsigned short* d = &s_x[0][buf][(px0 + 32 * i) * kPitchE + 8 * q8];
      if constexpr (kX3) {
        uint4 hi, lo;
        split_bf16x8(st.x[i][0], st.x[i][kLd - 1], hi, lo);
        *reinterpret_cast<uint4*>(d) = hi;
        *reinterpret_cast<uint4*>(&s_x[kPlanes - 1][buf][(px0 + 32 * i) * kPitchE + 8 * q8]) = lo;
      } else {
        *reinterpret_cast<uint4*>(d) = st.x[i][0];
      }
    }
  };

  // Transposed-read addressing: in 16-lane group gq, lane j points at pixel
  // 8 gq + j / 4 (+ 4 for the upper half of the k-step) and 4 channels at 4 (j % 4).
  const int j = lane & 15, gq = lane >> 4;
  const int lane_off = (8 * gq + (j >> 2)) * kPitchE + 4 * (j & 3);
  auto tr8 = [&](const unsigned short* p) {
    return __builtin_shufflevector(tr_read(p), tr_read(p + 4 * kPitchE), 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x4 acc[4][SB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < SB; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Bias gradient: in the tile with the first filter row, tap block and input
  // channel block, wave 0 multiplies each A operand by ones (every column of
  // the product is the per-channel sum of the operand's 32 pixels).
  const bool db_wave = kDb && !kX3 && r == 0 && sb == 0 && ct == 0 && wave == 0;
  f32x4 acc_db[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_db[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned short one = kBf16 ? 0x3f80 : 0x3c00;
  const s16x8 ones{(short)one, (short)one, (short)one, (short)one,
                   (short)one, (short)one, (short)one, (short)one};

  // One unit's MFMAs: per 32-pixel k-step, the A and B operands by
  // transposed LDS reads, then 4 * SB MFMAs (with BF16x3 the two cross terms,
  // small, before hi * hi).  npix is workgroup-uniform, so a unit of at most
  // 32 pixel slots skips the second k-step and a unit past the slice both.
  auto compute_unit = [&](int buf, int npix) {
    const unsigned short* ad = s_dy[0][buf] + lane_off;
    const unsigned short* bx = s_x[0][buf] + lane_off + 16 * wave;
    const unsigned short* ad_lo = s_dy[kPlanes - 1][buf] + lane_off;
    const unsigned short* bx_lo = s_x[kPlanes - 1][buf] + lane_off + 16 * wave;
#pragma unroll
    for (int ks = 0; ks < kWt / 32; ++ks) {
      if (32 * ks < npix) {
        s16x8 fa[4], fb[SB];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = tr8(ad + 32 * ks * kPitchE + 16 * i);
#pragma unroll
        for (int s = 0; s < SB; ++s) fb[s] = tr8(bx + (32 * ks + s) * kPitchE);
        if constexpr (kX3) {
          s16x8 fa_lo[4], fb_lo[SB];
#pragma unroll
          for (int i = 0; i < 4; ++i) fa_lo[i] = tr8(ad_lo + 32 * ks * kPitchE + 16 * i);
#pragma unroll
          for (int s = 0; s < SB; ++s) fb_lo[s] = tr8(bx_lo + (32 * ks + s) * kPitchE);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s = 0; s < SB; ++s) {
              acc[i][s] = mfma16<true>(fa_lo[i], fb[s], acc[i][s]);
              acc[i][s] = mfma16<true>(fa[i], fb_lo[s], acc[i][s]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int s = 0; s < SB; ++s) acc[i][s] = mfma16<kBf16>(fa[i], fb[s], acc[i][s]);
        if constexpr (kDb && !kX3) {
          if (db_wave) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_db[i] = mfma16<kBf16>(fa[i], ones, acc_db[i]);
          }
        }
      }
    }
  };

  // Whole rounds of kSets units; the prologue issues the sets in the order
  // the loop consumes them (pinned by scheduling barriers).
  const int rounds = (u_end - u_begin + kSets - 1) / kSets;
  Set sets[kSets];
#pragma unroll
  for (int p = 0; p < kSets; ++p) {
    load_unit(u_begin + p, sets[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int p = 0; p < kSets; ++p) {
      const int u = u_begin + it * kSets + p;
      const int buf = (it * kSets + p) & 1;
      const int npix = sets[p].npix;
      store_unit(buf, sets[p]);
      load_unit(u + kSets, sets[p]);
      // The unit is staged and every wave is done with the other buffer.  An
      // LDS-only barrier: the loads just issued stay in flight over the MFMAs
      // (__syncthreads would also wait for them).
      lds_barrier();
      compute_unit(buf, npix);
    }
  }

  // acc[i][s][v] = dW[g*Kg + m0 + 16 i + 4 gq + v][(r*S + s0 + s)*Cg + c0 + 16 wave + j].
  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + j;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 16 * i + 4 * gq + v;
      if (m < a.Kg && c < a.Cg) {
        float* o = out + ((int64_t)g * a.Kg + m) * a.cols + (int64_t)(r * a.S + s0) * a.Cg + c;
#pragma unroll
        for (int s = 0; s < SB; ++s)
          if (s0 + s < a.S) o[(int64_t)s * a.Cg] = acc[i][s][v];
      }
    }
  if constexpr (kX3 && kDb) {
    // 32 loader rows (px0) x 64 channels of per-thread sums, added in
    // ascending row order through LDS (the staging buffers are free now).
    if (db_x3)   // workgroup-uniform; block_sum64 has its own barriers
      block_sum64<32, 8>(reinterpret_cast<float*>(&s_x[0][0][0]), px0, 8 * q8, dbp,
                         a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                         min(64, a.Kg - m0));
  }
  if (db_wave && j == 0) {
    float* o = a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * gq + v;
        if (m < a.Kg) o[m] = acc_db[i][v];
      }
  }
}

constexpr int kSetsDefault = 2;

template <bool kBf16, int SB, bool kX3>
hipError_t launch_sb(const R16Args& args, int64_t grid, hipStream_t stream) {
  const dim3 xcd_grid((unsigned)((grid + 7) / 8 * 8)), block(256);   // whole rounds over the 8 XCDs
  constexpr int kS = kSetsDefault;
  if (args.ru > 1) {
    if (args.dbo) return launch_kernel(dense16_rows_kernel<kBf16, SB, true, kX3, true, kS>, xcd_grid, block, args, stream);
    return launch_kernel(dense16_rows_kernel<kBf16, SB, false, kX3, true, kS>, xcd_grid, block, args, stream);
  }
  if (args.dbo) return launch_kernel(dense16_rows_kernel<kBf16, SB, true, kX3, false, kS>, xcd_grid, block, args, stream);
  return launch_kernel(dense16_rows_kernel<kBf16, SB, false, kX3, false, kS>, xcd_grid, block, args, stream);
}

template <bool kBf16, bool kX3>
hipError_t launch_b(const Plan& plan, const R16Args& args, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  switch (plan.sb) {
    case 1: return launch_sb<kBf16, 1, kX3>(args, grid, stream);
    case 2: return launch_sb<kBf16, 2, kX3>(args, grid, stream);
    case 3: return launch_sb<kBf16, 3, kX3>(args, grid, stream);
    default: return launch_sb<kBf16, 4, kX3>(args, grid, stream);
  }
}

}  // namespace

hipError_t launch_dense16_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                               hipStream_t stream) {
  const Problem& p = plan.p;
  R16Args a;
  a.x = x;
  a.dy = dy;
  a.out = out.base;
  a.slab_stride = out.slab_stride;
  a.dbo = out.db;
  a.x_img = p.x_img;
  a.H = (int32_t)p.H; a.W = (int32_t)p.W; a.C = (int32_t)p.C; a.K = (int32_t)p.K;
  a.Ho = (int32_t)p.Ho; a.Wo = (int32_t)p.Wo;
  a.R = (int32_t)p.R; a.S = (int32_t)p.S;
  a.pad_h = (int32_t)p.pad_h; a.pad_w = (int32_t)p.pad_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.cols = (int32_t)p.cols;
  a.m_tiles = (int32_t)plan.m_tiles;
  a.c_tiles = (int32_t)plan.c_tiles;
  a.s_blocks = (int32_t)plan.s_blocks;
  a.wt = plan.wt;
  a.wchunks = (int32_t)plan.wchunks;
  a.ru = plan.ru > 1 ? plan.ru : 1;
  a.pitch = (int32_t)(p.Wo + plan.sb - 1);
  a.hblocks = (int32_t)ceil_div(p.Ho, a.ru);
  a.units = (int32_t)plan.pub.units;
  a.units_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.tiles = (int32_t)plan.pub.tiles;
  a.work = (int32_t)(plan.pub.tiles * plan.pub.ks_count);
  if (p.dtype == CONV_WGRAD_F32) return launch_b<true, true>(plan, a, stream);   // BF16x3
  if (p.dtype == CONV_WGRAD_BF16) return launch_b<true, false>(plan, a, stream);
  return launch_b<false, false>(plan, a, stream);
}

}  // namespace cw
