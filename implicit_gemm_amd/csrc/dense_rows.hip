// Dense implicit-GEMM weight gradient over output-row units (gfx950, f32 MFMA).
//
// Same GEMM as the general dense kernel (per group: M = Kg, N = R*S*Cg,
// reduction over output pixels), organised so that every staged element is
// reused by all the taps of one filter row:
//
//   * a reduction unit is a run of up to `wt` consecutive output pixels of one
//     output row (n, ho);
//   * a workgroup tile is (group, 64 output channels, filter row r, SB
//     consecutive taps s, 64 input channels), so its B operand for tap s is
//     the staged X row segment shifted by s*dil pixels -- an LDS address
//     offset, not another load;
//   * a unit's dY rows [wt][64] and X segment [xspan][64] are staged once in
//     LDS (widened to fp32); within a wave, 4*SB independent
//     v_mfma_f32_16x16x4_f32 accumulators (all 64 output channels x 16 input
//     channels) are fed per 4 reduction rows by one 16-byte read of 4 dY
//     channels and SB reads of X;
//   * two workgroup shapes keep the MFMA pipe busy while units are staged:
//     - 256 lanes (four waves, the planner's choice when the split gives at
//       least 1.5 workgroups per CU): two workgroups share a CU, each stages
//       a unit (the loads of the next one are issued right after), waits at a
//       barrier, computes it and waits again; the CU interleaves the two
//       workgroups, so one's staging and barriers overlap the other's MFMAs
//       and the two waves per SIMD hide each other's LDS reads;
//     - 512 lanes (one workgroup per CU): two halves of four waves (one wave
//       of each per SIMD) take alternate units of the slice, each with its own
//       LDS buffer.  Phases separated by workgroup barriers alternate the
//       roles, so while one half stages its next unit (global loads issued two
//       phases ahead, fp32 widening, LDS stores) the other half's MFMAs run on
//       the same SIMDs.  At the end the halves' accumulators are added (half 1
//       into half 0, a fixed order) and half 0 writes the slab.
//
// Three assignments of reduction rows to the MFMA k index:
//   * interleaved: lane group lg (lanes 16lg .. 16lg + 15) takes pixel 4k + lg
//     in k-step k, so each k-step reads SB X values (one per tap);
//   * quarters (stride 1, dilation 1, one unit per output row, 256 lanes,
//     rows the packed form below does not take):
//     lane group lg takes the contiguous pixels lg*Q .. lg*Q + Q - 1,
//     Q = ceil(Wo / 4), pixel lg*Q + k in k-step k.  Tap s then reads X slot
//     lg*Q + k + s, which tap s - 1 reads in k-step k + 1: each k-step reads
//     one new X value and keeps the last SB - 1 in registers.
// Staged pixel rows are P floats apart, chosen so that the 4 rows a wave reads
// per MFMA fall in disjoint bank groups (offsets 16 mod 32 and 16 or 48 mod
// 64 banks between lane groups): P = 80 for the interleaved form (rows 1
// apart) and for odd Q, 72 for Q = 2 mod 4 (rows Q apart); Q = 0 mod 4 has
// no such pitch and keeps the interleaved form.  The quarters form reads at
// most 64 dY and 64 X pixel rows, so two buffers fit beside the other
// workgroup on the CU: a unit is staged into the buffer the unit before last
// used, and one barrier per unit suffices.
//   * packed rows (stride 1, dilation 1, Wo <= 14 and Wo + SB - 1 <= 16 (the
//     16 columns the loader stages per row), 256 lanes): a unit is 4
//     consecutive output rows of one image and lane group lg takes row lg,
//     pixel k in k-step k.  dY row lg is staged at slots lg*QA .., its X
//     segment (Wo + SB - 1 pixels) at X slots lg*QB .., with QA >= Wo and
//     QB >= Wo + SB - 1 both 2 mod 4 under pitch 72 (lane groups in disjoint
//     banks); tap s reads X slot lg*QB + k + s, so the one-new-X-value window
//     of the quarters form applies, on 4x the pixels of a one-row unit.
//     Two buffers of 64 dY + 72 X pixel rows, one barrier per unit.
#include "device_common.h"
#include "kernels.h"

namespace cw {

namespace {

constexpr int kPitch = 80;      // floats per staged pixel row, interleaved form (64 channels + pad)
constexpr int kMaxWt = 64;      // output pixels per unit
constexpr int kMaxXSpan = 80;   // staged X pixels per unit
constexpr int kQuartersXSpan = 64;  // staged X pixels per unit, quarters form
constexpr int kPackedXSpan = 72;    // staged X pixel slots per unit, packed rows
constexpr int kPackedRows = 4;      // output rows per unit, packed rows

// Forms of the kernel (template argument kForm).
constexpr int kInterleaved = 0, kQuartersForm = 1, kPackedForm = 2;

// Calls f(integral_constant<K>) for K = 0, 1, ... while K < n (and K < N), as
// nested conditional blocks: step K is entered only from step K - 1, and the
// steps not taken all join once, after the last.  A flat unrolled loop of
// `if (k < n)` blocks joins after every step instead, and a wait inserted at
// such a join must cover the LDS reads in flight on any incoming path.
template <int K, int N, typename F>
__device__ __forceinline__ void steps_while(int n, F&& f) {
  if constexpr (K < N) {
    if (K < n) {
      f(std::integral_constant<int, K>{});
      steps_while<K + 1, N>(n, f);
    }
  }
}

struct RowsArgs {
  const void* x;
  const void* dy;
  float* out;
  int64_t slab_stride;
  int64_t x_img;  // H*W*C
  int32_t H, W, C, K, Ho, Wo;
  int32_t R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w;
  int32_t Cg, Kg, cols;
  int32_t m_tiles, c_tiles, s_blocks;
  int32_t wt, wchunks, xspan;
  int32_t units, units_per_slice, ks_count;
  int32_t tiles, work;   // tiles per slice, tiles * ks_count
  int32_t q;             // quarters: pixels per lane group; packed: dY slots between lane groups
  int32_t qb;            // X slots between lane groups (quarters: q)
  int32_t qk;            // k-steps per unit (quarters: q; packed: Wo)
  int32_t hunits;        // packed: units per image (ceil(Ho / 4))
  float* dbo;            // bias-gradient partial of slice 0 (slab_stride apart), or nullptr
};

// kUnit: column stride 1 and column dilation 1 are compile-time (every LDS offset of the
// MFMA loop is an immediate); otherwise they are read from the arguments.
// kSolo: the 256-lane form (no halves); otherwise 512 lanes in two halves.
// P: the staged pixel pitch in floats.  kForm: interleaved, quarters or
// packed rows (the last two: two buffers, one barrier per unit).
template <typename T, int SB, bool kUnit, bool kSolo, int P, int kForm>
__global__ __launch_bounds__(kSolo ? 256 : 512, kSolo ? 2 : 1) void dense_rows_kernel(RowsArgs a) {
  extern __shared__ float smem[];
  constexpr bool kQuarters = kForm != kInterleaved;   // quarters or packed: the window schedule
  constexpr bool kPacked = kForm == kPackedForm;
  static_assert(!kQuarters || (kUnit && kSolo), "quarters / packed: unit stride and dilation, 256 lanes");
  constexpr int kXSpan = kPacked ? kPackedXSpan : kQuarters ? kQuartersXSpan : kMaxXSpan;
  constexpr int kBuf = (kMaxWt + kXSpan) * P;  // floats per buffer
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ dy = static_cast<const T*>(a.dy);

  // The half index is wave-uniform; readfirstlane lets the compiler keep the
  // values derived from it (unit indices, buffer resources) in SGPRs.
  const int tid = threadIdx.x & 255;
  const int half = kSolo ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  // Work item w = slice * tiles + tile.  Workgroups are dispatched to the 8
  // XCDs round-robin (block i on XCD i % 8); each XCD takes a contiguous run
  // of items, so the tiles of one slice, which read the same dY rows and
  // overlapping X rows, run on one XCD and share its L2.
  const int per_xcd = (a.work + 7) >> 3;
  const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
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
  const int nu = min(a.units, u_begin + a.units_per_slice) - u_begin;   // units in the slice

  // Loader role within the half: pixel rows p0 + 16*i, channel quad q (4 channels).
  // Rows are fetched with buffer loads whose range ends at the valid data, so
  // pixels past the unit, columns outside the image and rows outside it read
  // zero; lane byte offsets are fixed per lane (plus the unit's first column).
  constexpr int kEs = sizeof(T);
  const int q = tid & 15, p0 = tid >> 4;
  const int dy_col0 = g * a.Kg + m0;         // first output channel of the tile
  const int x_col0 = g * a.Cg + c0;          // first input channel of the tile
  const int dh = r * a.dil_h - a.pad_h;
  const int xw_off = s0 * a.dil_w - a.pad_w;
  int oa[kMaxWt / 16], ob[kXSpan / 16];
#pragma unroll
  for (int i = 0; i < kMaxWt / 16; ++i) oa[i] = ((p0 + 16 * i) * a.K + 4 * q) * kEs;
#pragma unroll
  for (int i = 0; i < kXSpan / 16; ++i) ob[i] = ((p0 + 16 * i) * a.C + 4 * q) * kEs;
  const int x_row_bytes = (a.W * a.C - x_col0) * kEs;

  // Staged operands of one unit, as loaded.
  float ra[kMaxWt / 16][4];
  float rb[kXSpan / 16][4];
  int npix_reg = 0;

  // Packed rows: lane row p0 is the pixel column (16 per row), ra[i] / rb[i]
  // hold dY row ho0 + i and its X segment.
  auto load_packed = [&](int u) {
    const int n = u / a.hunits;
    const int ho0 = (u - n * a.hunits) * kPackedRows;
    npix_reg = a.Wo;
    const int da = (p0 * a.K + 4 * q) * kEs;
    const int xa = (p0 * a.C + 4 * q) * kEs + xw_off * a.C * kEs;
#pragma unroll
    for (int i = 0; i < kPackedRows; ++i) {
      const int ho = ho0 + i;
      const bool ok = ho < a.Ho;
      const T* dyp = dy + ((int64_t)n * a.Ho + (ok ? ho : 0)) * a.Wo * a.K + dy_col0;
      buf_load4(buf_rsrc(dyp, ok ? (a.Wo * a.K - dy_col0) * kEs : 0), da, dyp, ra[i]);
      const int h = ho * a.stride_h + dh;
      const bool xok = ok && h >= 0 && h < a.H;
      const T* xp = x + (int64_t)n * a.x_img + (int64_t)(xok ? h : 0) * a.W * a.C + x_col0;
      buf_load4(buf_rsrc(xp, xok ? x_row_bytes : 0), xa, xp, rb[i]);
    }
  };
  auto load_unit = [&](int u) {
    if constexpr (kPacked) {
      load_packed(u);
      return;
    }
    const int wc = u % a.wchunks;
    const int t = u / a.wchunks;
    const int ho = t % a.Ho, n = t / a.Ho;
    const int wo0 = wc * a.wt;
    const int npix = min(a.wt, a.Wo - wo0);
    npix_reg = npix;
    const T* dyp = dy + ((int64_t)(n * a.Ho + ho) * a.Wo + wo0) * a.K + dy_col0;
    const __amdgpu_buffer_rsrc_t rs_a = buf_rsrc(dyp, (npix * a.K - dy_col0) * kEs);
#pragma unroll
    for (int i = 0; i < kMaxWt / 16; ++i) buf_load4(rs_a, oa[i], dyp, ra[i]);
    const int h = ho * a.stride_h + dh;
    const bool row_ok = h >= 0 && h < a.H;
    const int w0 = wo0 * a.stride_w + xw_off;
    const T* xp = x + (int64_t)n * a.x_img + (int64_t)(row_ok ? h : 0) * a.W * a.C + x_col0;
    const __amdgpu_buffer_rsrc_t rs_b = buf_rsrc(xp, row_ok ? x_row_bytes : 0);
    const int wb = w0 * a.C * kEs;
#pragma unroll
    for (int i = 0; i < kXSpan / 16; ++i) buf_load4(rs_b, ob[i] + wb, xp, rb[i]);
  };

  // Bias gradient: the tile with the first filter row, tap block and input
  // channel block of its (group, output-channel block) adds up the dY rows it
  // stages (every output pixel of the slice once; pixels past a unit load as
  // zero), per thread for its 4 channels.
  const bool want_db = a.dbo != nullptr && r == 0 && sb == 0 && ct == 0;
  float dbp[4] = {0.f, 0.f, 0.f, 0.f};
  auto store_packed = [&](float* buf) {
    // Columns past a row's slots belong to the next row: dY columns from QA
    // and X columns from QB on are not stored (they would be zero or unread).
    float* xb = buf + kMaxWt * P;
#pragma unroll
    for (int i = 0; i < kPackedRows; ++i) {
      if (p0 < a.q)
        *reinterpret_cast<float4*>(&buf[(i * a.q + p0) * P + 4 * q]) =
            float4{ra[i][0], ra[i][1], ra[i][2], ra[i][3]};
      if (p0 < a.qb)
        *reinterpret_cast<float4*>(&xb[(i * a.qb + p0) * P + 4 * q]) =
            float4{rb[i][0], rb[i][1], rb[i][2], rb[i][3]};
      if (want_db) {   // dY pixels from Wo on loaded as zero
#pragma unroll
        for (int j = 0; j < 4; ++j) dbp[j] += ra[i][j];
      }
    }
  };
  auto store_unit = [&](float* buf) {
    if constexpr (kPacked) {
      store_packed(buf);
      return;
    }
#pragma unroll
    for (int i = 0; i < kMaxWt / 16; ++i) {
      *reinterpret_cast<float4*>(&buf[(p0 + 16 * i) * P + 4 * q]) =
          float4{ra[i][0], ra[i][1], ra[i][2], ra[i][3]};
      if (want_db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dbp[j] += ra[i][j];
      }
    }
    float* xb = buf + kMaxWt * P;
#pragma unroll
    for (int i = 0; i < kXSpan / 16; ++i)
      *reinterpret_cast<float4*>(&xb[(p0 + 16 * i) * P + 4 * q]) =
          float4{rb[i][0], rb[i][1], rb[i][2], rb[i][3]};
  };

  f32x4 acc[4][SB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < SB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int stride = kUnit ? 1 : a.stride_w;
  // Row li of M-block i is output channel m0 + 4*li + i, so a lane's four A
  // fragments are the 4 consecutive channels 4*li .. 4*li + 3 of its pixel
  // row: one 16-byte LDS read per k-step.
  const int row0 = kQuarters ? lg * a.q : lg;   // the lane group's first dY pixel slot
  const int xrow0 = kQuarters ? lg * a.qb : lg;  // ... and first X pixel slot
  float* const buf = smem + half * kBuf;         // the half's buffer (the first buffer)
  const float* const A0 = buf + row0 * P + 4 * li;
  const float* const B0 = buf + kMaxWt * P + xrow0 * stride * P + 16 * wave + li;
  const int b_kstep = (kQuarters ? 1 : 4) * stride * P;
  const int b_tap = (kUnit ? 1 : a.dil_w) * P;

  // One unit's MFMAs: up to kMaxWt / 4 k-steps, fully unrolled so that every
  // LDS offset is an immediate (no VALU work between the MFMAs).  Two operand
  // sets alternate: the fragments of k-step k + 1 are read before the MFMAs of
  // k-step k issue.
  auto compute_interleaved = [&](int npix) {
    const int nk = (npix + 3) >> 2;
    const float* const A = A0;
    const float* const B = B0;
    float fa[2][4], fb[2][SB];
    auto read_k = [&](int k, float (&ra_)[4], float (&rb_)[SB]) {
      const float4 av = *reinterpret_cast<const float4*>(A + 4 * k * P);
      ra_[0] = av.x; ra_[1] = av.y; ra_[2] = av.z; ra_[3] = av.w;
#pragma unroll
      for (int s = 0; s < SB; ++s) rb_[s] = B[k * b_kstep + s * b_tap];
      // Keep the scheduler from hoisting the following MFMAs above the reads.
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mfmas = [&](int k) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < SB; ++s)
          acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[k & 1][i], fb[k & 1][s], acc[i][s], 0, 0, 0);
    };
    if (nk > 0) read_k(0, fa[0], fb[0]);
    if constexpr (kUnit) {
      // Unit stride and dilation: the fragments one k-step past the last
      // (pixel rows up to 63, X slots up to 66) lie inside the buffer, so the
      // next step's reads need no condition and the steps nest.
      steps_while<0, kMaxWt / 4>(nk, [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k + 1 < kMaxWt / 4) read_k(k + 1, fa[(k + 1) & 1], fb[(k + 1) & 1]);
        mfmas(k);
      });
    } else {
      // Strided or dilated X slots one step past the last may lie past the
      // buffer: the reads stay conditional (a nested form with the last
      // step's MFMAs duplicated measured 14 % slower).
#pragma unroll
      for (int k = 0; k < kMaxWt / 4; ++k) {
        if (k < nk) {
          if (k + 1 < nk) read_k(k + 1, fa[(k + 1) & 1], fb[(k + 1) & 1]);
          mfmas(k);
        }
      }
    }
  };
  // Quarters form: k-step k reads the A fragments of pixel lg*Q + k + 1 and
  // the one X value of slot lg*Q + k + SB ahead of its MFMAs; xw[j] holds X
  // slot lg*Q + j (a register window of SB + 1 values once unrolled).  Every
  // lane group has a valid pixel in k-step k < min(Q, npix); slots past npix
  // hold zero dY.  The reads one step past the last (pixel row up to 4Q,
  // X slot up to 4Q + SB - 1, Q <= 15) lie inside the buffer and are issued
  // unconditionally, as in the interleaved form.  Packed rows: the same with
  // X slots lg*QB + k + s and nk = Wo (rows past the image hold zero dY);
  // the reads one step past the last reach dY slot 3 QA + Wo <= 56 and X
  // slot 3 QB + Wo + SB - 1 <= 71.
  auto compute_quarters = [&](int npix, int boff) {
    const int nk = min(a.qk, npix);
    const float* const A = A0 + boff;
    const float* const B = B0 + boff;
    float fa[2][4], xw[kMaxWt / 4 + SB];
    auto read_a = [&](int k, float (&ra_)[4]) {
      const float4 av = *reinterpret_cast<const float4*>(A + k * P);
      ra_[0] = av.x; ra_[1] = av.y; ra_[2] = av.z; ra_[3] = av.w;
    };
    if (nk > 0) {
      read_a(0, fa[0]);
#pragma unroll
      for (int s = 0; s < SB; ++s) xw[s] = B[s * P];
      __builtin_amdgcn_sched_barrier(0);
    }
    steps_while<0, kMaxWt / 4>(nk, [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k + 1 < kMaxWt / 4) {
        read_a(k + 1, fa[(k + 1) & 1]);
        xw[k + SB] = B[(k + SB) * P];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < SB; ++s)
          acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[k & 1][i], xw[k + s], acc[i][s], 0, 0, 0);
    });
  };

  if constexpr (kQuarters) {
    // Unit p is staged into buffer p & 1 (its loads were issued one unit
    // earlier), the next unit's loads are issued, and after one barrier it
    // is computed.  Buffer p & 1 was last read by unit p - 2, which every
    // wave finished before the barrier of unit p - 1.
    if (nu > 0) load_unit(u_begin);
    for (int p = 0; p < nu; ++p) {
      const int npix = npix_reg;
      const int boff = (p & 1) * kBuf;
      store_unit(smem + boff);
      if (p + 1 < nu) load_unit(u_begin + p + 1);
      lds_barrier();   // LDS only: the next unit's loads stay in flight
      compute_quarters(npix, boff);
    }
    if (want_db)   // block_sum64 begins with a barrier: every wave is past its last unit
      block_sum64<16, 4>(smem, p0, 4 * q, dbp,
                         a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                         min(64, a.Kg - m0));
  } else if constexpr (kSolo) {
    // Unit by unit: stage it (its loads were issued one unit earlier), issue
    // the next unit's loads, compute it; the second barrier keeps the next
    // staging off the buffer until every wave has read it.
    if (nu > 0) load_unit(u_begin);
    for (int p = 0; p < nu; ++p) {
      const int npix = npix_reg;
      store_unit(buf);
      if (p + 1 < nu) load_unit(u_begin + p + 1);
      // LDS-only barriers: the next unit's loads stay in flight over the
      // MFMAs (__syncthreads would also wait for them).
      lds_barrier();
      compute_interleaved(npix);
      lds_barrier();
    }
    if (want_db)   // 16 loader rows per channel quad
      block_sum64<16, 4>(smem, p0, 4 * q, dbp,
                         a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                         min(64, a.Kg - m0));
  } else {
    // Half h takes units h, h + 2, ... of the slice.  In phase p the half with
    // parity p stages unit p and the other half computes unit p - 1; a
    // workgroup barrier ends every phase.
    if (half < nu) load_unit(u_begin + half);
    int npix_cur = 0;
    for (int p = 0; p <= nu; ++p) {
      const bool stage = (p & 1) == half && p < nu;
      const bool comp = (p & 1) != half && p >= 1;
      if (stage) {
        npix_cur = npix_reg;
        store_unit(buf);
        if (p + 2 < nu) load_unit(u_begin + p + 2);
      }
      // Called on every phase (with no pixels when staging) so that the
      // accumulators take one path through the loop.
      compute_interleaved(comp ? npix_cur : 0);
      lds_barrier();   // LDS only: the loads issued two phases ahead stay in flight
    }

    // Bias partial: rows are the 16 loader rows of half 0, then those of half 1.
    if (want_db)
      block_sum64<32, 4>(smem, 16 * half + p0, 4 * q, dbp,
                         a.dbo + (int64_t)slice * a.slab_stride + (int64_t)g * a.Kg + m0,
                         min(64, a.Kg - m0));

    // Half 1 hands its accumulators to half 0 through LDS (both buffers are
    // free after the last barrier); half 0 adds them and writes the slab.
    float* xfer = smem + tid;
    if (half == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
          for (int v = 0; v < 4; ++v) xfer[((i * SB + s) * 4 + v) * 256] = acc[i][s][v];
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < SB; ++s)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][s][v] += xfer[((i * SB + s) * 4 + v) * 256];
  }

  float* out = a.out + (int64_t)slice * a.slab_stride;
  const int c = c0 + 16 * wave + li;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // acc[i][s][v] is D row 4*lg + v of M-block i: channel 4*(4*lg + v) + i.
        const int m = m0 + 16 * lg + 4 * v + i;
        const int sa = s0 + s;
        if (m < a.Kg && c < a.Cg && sa < a.S)
          out[((int64_t)g * a.Kg + m) * a.cols + (r * a.S + sa) * a.Cg + c] = acc[i][s][v];
      }
}

template <typename T, int SB, bool kUnit, bool kSolo, int P, int kForm>
hipError_t launch_p(const RowsArgs& args, int64_t grid, hipStream_t stream) {
  // One staging buffer (256 lanes), one per half (512 lanes), two of 128
  // pixel rows (quarters form: 73.7 or 80 KB) or two of 136 (packed rows:
  // 78.3 KB); two workgroups per CU in the 256-lane forms.
  constexpr size_t kLds = kForm == kPackedForm ? 2 * (kMaxWt + kPackedXSpan) * P * sizeof(float)
                          : kForm == kQuartersForm ? 2 * (kMaxWt + kQuartersXSpan) * P * sizeof(float)
                                                   : (kSolo ? 1 : 2) * (kMaxWt + kMaxXSpan) * P * sizeof(float);
  static_assert(2 * kLds <= 160 * 1024 || !kSolo, "two workgroups per CU");
  const void* fn = reinterpret_cast<const void*>(dense_rows_kernel<T, SB, kUnit, kSolo, P, kForm>);
  // More than 64 KB of dynamic LDS must be enabled per kernel (once).
  if (kLds > 64 * 1024) {
    static const hipError_t attr =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (attr != hipSuccess) return attr;
  }
  void* params[] = {const_cast<RowsArgs*>(&args)};
  const int64_t xcd_grid = (grid + 7) / 8 * 8;   // whole rounds over the 8 XCDs
  return launch_raw(fn, dim3((unsigned)xcd_grid), dim3(kSolo ? 256 : 512), params, kLds, stream);
}

// Packed rows when the plan has them (hunits > 0); else the quarters form
// when it applies (unit stride and dilation, 256 lanes, one unit per output
// row, Q = ceil(Wo / 4) not a multiple of 4); else interleaved.
template <typename T, int SB, bool kUnit, bool kSolo>
hipError_t launch_sb(const RowsArgs& args, int64_t grid, hipStream_t stream) {
  if constexpr (kUnit && kSolo) {
    if (args.hunits > 0) return launch_p<T, SB, kUnit, kSolo, 72, kPackedForm>(args, grid, stream);
    if (args.wchunks == 1 && args.q % 4 != 0) {
      if (args.q & 1) return launch_p<T, SB, kUnit, kSolo, 80, kQuartersForm>(args, grid, stream);
      return launch_p<T, SB, kUnit, kSolo, 72, kQuartersForm>(args, grid, stream);
    }
  }
  return launch_p<T, SB, kUnit, kSolo, kPitch, kInterleaved>(args, grid, stream);
}

template <typename T, bool kUnit, bool kSolo>
hipError_t launch_s(const Plan& plan, const RowsArgs& args, hipStream_t stream) {
  const int64_t grid = plan.pub.grid;
  switch (plan.sb) {
    case 1: return launch_sb<T, 1, kUnit, kSolo>(args, grid, stream);
    case 2: return launch_sb<T, 2, kUnit, kSolo>(args, grid, stream);
    case 3: return launch_sb<T, 3, kUnit, kSolo>(args, grid, stream);
    default: return launch_sb<T, 4, kUnit, kSolo>(args, grid, stream);
  }
}

template <typename T, bool kUnit>
hipError_t launch_u(const Plan& plan, const RowsArgs& args, hipStream_t stream) {
  if (plan.threads == 256) return launch_s<T, kUnit, true>(plan, args, stream);
  return launch_s<T, kUnit, false>(plan, args, stream);
}

template <typename T>
hipError_t launch_t(const Plan& plan, const RowsArgs& args, hipStream_t stream) {
  if (args.stride_w == 1 && args.dil_w == 1) return launch_u<T, true>(plan, args, stream);
  return launch_u<T, false>(plan, args, stream);
}

}  // namespace

hipError_t launch_dense_rows(const Plan& plan, const void* x, const void* dy, Stage1Out out,
                             hipStream_t stream) {
  const Problem& p = plan.p;
  RowsArgs a;
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
  a.stride_h = (int32_t)p.stride_h; a.stride_w = (int32_t)p.stride_w;
  a.dil_h = (int32_t)p.dil_h; a.dil_w = (int32_t)p.dil_w;
  a.Cg = (int32_t)p.Cg; a.Kg = (int32_t)p.Kg; a.cols = (int32_t)p.cols;
  a.m_tiles = (int32_t)plan.m_tiles;
  a.c_tiles = (int32_t)plan.c_tiles;
  a.s_blocks = (int32_t)plan.s_blocks;
  a.wt = plan.wt;
  a.wchunks = (int32_t)plan.wchunks;
  a.xspan = plan.xspan;
  a.units = (int32_t)plan.pub.units;
  a.units_per_slice = (int32_t)plan.pub.units_per_slice;
  a.ks_count = plan.pub.ks_count;
  a.tiles = (int32_t)plan.pub.tiles;
  a.work = (int32_t)plan.pub.grid;
  if (plan.ru > 1) {   // packed rows
    a.q = plan.qa;
    a.qb = plan.qb;
    a.qk = (int32_t)p.Wo;
    a.hunits = (int32_t)ceil_div(p.Ho, plan.ru);
  } else {
    a.q = a.qb = a.qk = (int32_t)((p.Wo + 3) / 4);
    a.hunits = 0;
  }
  switch (p.dtype) {
    case CONV_WGRAD_F32: return launch_t<float>(plan, a, stream);
    case CONV_WGRAD_BF16: return launch_t<Bf16>(plan, a, stream);
    default: return launch_t<F16>(plan, a, stream);
  }
}

}  // namespace cw
