// The dense GEMMs of a neural-processor layer around the contextualizer, on bf16 MFMA (gfx950):
//   enricher  Z = ReLU(X U + b)^2       U [d][m]: each token's d features up to m
//   fuser     Y = [Z_h || C] O + X      O [m_h + m_t][d]: the bypassed head of Z joined with the
//                                       contextualised tail C, projected back to d, plus the
//                                       layer's input
// (papernotes.org Avey-B note, 方法详解/整体框架; paperlayer.ai "Avey-B" summary, section 3 and
// appendix A for the squared ReLU.)
//
// Both are C^T[f][t] = sum_k W[k][f] A[t][k] with W = U or O row-major [K][F] and A the token
// rows: the structure of the persistent compression kernel (compress_bf16.hip) without the
// gather and the block weights. A unit is 256 output features x 256 tokens; W streams through
// LDS as 32-row chunks of 256 features (512-byte rows, read back with the LDS transpose read)
// and A as 256 token rows x 32 K-values (64 bytes) per chunk, through a 4-stage ring of 32 KiB
// direct-copy stages, one 8-wave workgroup per CU (2 x 4 waves of 128 features x 64 tokens;
// wave (wm, wn) holds features 128 wm .. +127, two whole 64-feature slices of its tokens).
//   * The fuser's A is two tensors along K: columns [0, m_h) of Z (its head), then C.
//   * The fuser's residual: 8 more chunks stage the unit's 256 token rows of X (256 features)
//     in the W part, with zeros in the A part; in the chunk holding a wave's token block, 8
//     MFMAs of those rows' transposed fragments against an identity operand add X[t][f] to
//     C^T[f][t] exactly (products with 1.0, fp32 accumulation).
//   * Epilogue through stage 3, each wave through its own 4 KiB of it (one barrier per unit), in
//     four rounds of 32 tokens x 64 features stored as whole 128-byte row pieces; the enricher
//     adds b[f] and squares the ReLU in fp32 before the single rounding to bf16.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int TF = 256;                 // output features per unit
constexpr int TT = 256;                 // tokens per unit
constexpr int KH = 32;                  // K per chunk
constexpr int XB = TF * 2;              // bytes per W row in LDS
constexpr int XS = KH * XB;             // W part of a stage (16 KiB)
constexpr int PB = KH * 2;              // bytes per A row in LDS
constexpr int STAGE = XS + TT * PB;     // 32 KiB
constexpr int kMaxF = 4096;             // features held in the LDS bias table

__device__ __forceinline__ uint32_t sw4(int r) { return (uint32_t)((r >> 2) & 3); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* base, uint32_t off) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

struct GemmParams {
  const uint16_t* W;       // [K][F], row stride ldw
  const uint16_t* A1;      // A columns [0, k1): [M][k1] rows of stride lda1
  const uint16_t* A2;      // A columns [k1, K): [M][K - k1] rows of stride lda2 (nullptr if k1 == K)
  const uint16_t* R;       // residual [M][F] (stride ldr) or nullptr
  uint16_t* C;             // [M][F], row stride ldc
  const float* bias;       // [F] or nullptr
  int64_t ldw, lda1, lda2, ldr, ldc, M, units;
  int F, K, k1, f_tiles, relu2;
};

#define WAIT_KEEP(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

template <int P>
using Pos = std::integral_constant<int, P>;

// kRelu2: the enricher (one A tensor, bias and squared ReLU in the epilogue); otherwise the
// fuser (A in two tensors along K, then the residual). Fixing each one's operands at compile
// time keeps the unused descriptors and their selects out of the K loop's scalar registers.
template <bool kRelu2>
__global__ void __launch_bounds__(512, 1) gemm_unit_kernel(GemmParams a) {
  __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  __shared__ __align__(16) float s_bias[kMaxF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 2, wn = wave & 3;

  // XCD x owns units [xs, xs + cnt) (consecutive units share a token tile); its workgroup l
  // takes every Gx-th of them from l.
  const int G = gridDim.x, wg = blockIdx.x, xcd = wg % NXCD, l = wg / NXCD;
  const int Gx = (G - xcd + NXCD - 1) / NXCD;
  const int64_t q8 = a.units / NXCD, r8 = a.units % NXCD;
  const int64_t xs = xcd * q8 + (xcd < r8 ? xcd : r8), cnt = q8 + (xcd < r8 ? 1 : 0);
  int64_t t = l;
  if (t >= cnt) return;

  for (int f = tid; f < kMaxF; f += 512) s_bias[f] = (a.bias && f < a.F) ? a.bias[f] : 0.f;
  lds_sync();   // the bias table is complete (its loads were waited for before the LDS writes)

  const int nreg = a.K / KH;                       // chunks of W x A
  constexpr bool kRes = !kRelu2;                   // the fuser adds its residual
  const int nk = nreg + (kRes ? TT / KH : 0);      // then the residual chunks
  const int nk4 = (nk + 3) / 4 * 4;                // padded with zero chunks to a multiple of 4
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.W, (uint32_t)((int64_t)a.K * a.ldw * 2));
  const __amdgpu_buffer_rsrc_t a1r = make_rsrc(a.A1, (uint32_t)(a.M * a.lda1 * 2));
  const __amdgpu_buffer_rsrc_t a2r = make_rsrc(kRes ? a.A2 : nullptr, kRes ? (uint32_t)(a.M * a.lda2 * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(kRes ? a.R : nullptr, kRes ? (uint32_t)(a.M * a.ldr * 2) : 0u);
  // the output; each wave's epilogue stores go through it, lanes out of range at OOB
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.C, (uint32_t)(a.M * a.ldc * 2));

  // ---- copy side: the unit whose chunks are being copied
  int64_t c_t0 = 0;
  int c_f0 = 0;
  // Enricher: each lane's copy offsets for the copy unit, less the chunk's K term, with bit 31
  // set where the lane is out of range (past F for W, past M for A); the K term rides in the
  // scalar offset, so that a copy costs no vector arithmetic. Copy n = 0, 1: W row
  // 4 w + 2 n + (lane >> 5) at the lane's feature; n = 2, 3: A row 32 w + 16 (n - 2) + (lane >> 2).
  uint32_t c_off[4] = {0u, 0u, 0u, 0u};
  uint32_t c_off2[2] = {0u, 0u};   // fuser: the A rows in its second A tensor
  auto set_copy_unit = [&](int64_t tl) {
    const int64_t L = xs + tl;
    c_f0 = (int)(L % a.f_tiles) * TF;
    c_t0 = (L / a.f_tiles) * TT;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tr = wave * 4 + n * 2 + (lane >> 5);
      const int p = lane & 31;
      const int fl = ((p >> 1) ^ (2 * (tr & 3))) * 16 + (p & 1) * 8;
      c_off[n] = ((uint32_t)tr * (uint32_t)a.ldw + (uint32_t)(c_f0 + fl)) * 2u |
                 ((uint32_t)!(fl < a.F - c_f0) << 31);
    }
#pragma unroll
    for (int n = 2; n < 4; ++n) {
      const int r0 = wave * 32 + (n - 2) * 16;
      const uint32_t tok = (uint32_t)c_t0 + (uint32_t)(r0 + (lane >> 2));
      const uint32_t piece = (uint32_t)((lane & 3) ^ (int)sw4(r0 + (lane >> 2)));
      const uint32_t oob = (uint32_t)!(tok < (uint32_t)a.M) << 31;
      c_off[n] = (tok * (uint32_t)a.lda1 * 2u + 16u * piece) | oob;
      if constexpr (!kRelu2) c_off2[n - 2] = (tok * (uint32_t)a.lda2 * 2u + 16u * piece) | oob;
    }
  };
  // Copy n of chunk kc into stage st: n = 0, 1 are W rows 4 w + 2 n, + 1 (1 KiB; in the
  // residual chunks the unit's token rows of R), n = 2, 3 are A rows 32 w + 16 (n - 2) .. + 15
  // (zeros in the residual chunks). Everything past M, F or K loads zeros. The source buffer is
  // selected per chunk without a branch (a control-flow join around a copy makes the compiler
  // drain every copy in flight).
  auto copy = [&](int kc, uint8_t* st, bool valid, int n, bool may_res = true) {
    // Held offsets: an invalid chunk takes scalar offset 0, so that bit 31 alone puts it out of
    // range. W copies that may be residual ones (the unit's rows of R; may_res is a constant at
    // every call) take the general path below, whose choice of source is a select: a branch
    // around a copy makes the compiler drain every copy in flight.
    const bool res_chunk = kRes && may_res && kc >= nreg;
    if (n < 2 && !(kRes && may_res)) {
      dma16(wr, st + (wave * 4 + n * 2) * XB, c_off[n] | (valid ? 0u : 0x80000000u),
            valid ? (uint32_t)(kc * KH) * (uint32_t)a.ldw * 2u : 0u);
      return;
    }
    if (n >= 2) {
      const int k0 = kc * KH;
      const bool first = !kRes || k0 < a.k1;
      const bool live = valid && !res_chunk;   // the residual chunks' A rows load zeros
      uint32_t vo = c_off[n];
      if constexpr (kRes) {
        uint32_t v2 = c_off2[n - 2];
        asm volatile("" : "+v"(v2));   // a select, not a branch on the uniform `first`
        vo = first ? vo : v2;
      }
      dma16(first ? a1r : a2r, st + XS + (wave * 32 + (n - 2) * 16) * PB, vo | (live ? 0u : 0x80000000u),
            live ? (uint32_t)(first ? k0 : k0 - a.k1) * 2u : 0u);
      return;
    }
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const bool res = kRes && may_res && kc >= nreg;
    // Offsets are 32-bit (every operand is below 2^31 bytes); a lane out of range gets the high
    // bit, past the descriptor's range, so that no branch is needed.
    if (n < 2) {
      const int tr = wave * 4 + n * 2 + (ln >> 5);
      const int p = ln & 31;
      const int c = (p >> 1) ^ (2 * (tr & 3));
      const int fl = c * 16 + (p & 1) * 8;                  // feature within the tile
      const uint32_t row = res ? (uint32_t)c_t0 + (uint32_t)((kc - nreg) * KH + tr) : (uint32_t)(kc * KH + tr);
      const uint32_t ld = res ? (uint32_t)a.ldr : (uint32_t)a.ldw;
      const bool ok = valid & (fl < a.F - c_f0) & (!res | (row < (uint32_t)a.M));
      const uint32_t off = (row * ld + (uint32_t)(c_f0 + fl)) * 2u;
      dma16(res ? rr : wr, st + (wave * 4 + n * 2) * XB, off | ((uint32_t)!ok << 31), 0);
    } else {
      const int r0 = wave * 32 + (n - 2) * 16;
      const uint32_t tok = (uint32_t)c_t0 + (uint32_t)(r0 + (ln >> 2));
      const uint32_t piece = (uint32_t)((ln & 3) ^ (int)sw4(r0 + (ln >> 2)));
      const int k0 = kc * KH;
      const bool first = !kRes || k0 < a.k1;
      const uint32_t ld = first ? (uint32_t)a.lda1 : (uint32_t)a.lda2;
      const int kk = first ? k0 : k0 - a.k1;
      const bool ok = valid & !res & (tok < (uint32_t)a.M);
      // the K offset rides in the (uniform) scalar offset
      dma16(first ? a1r : a2r, st + XS + r0 * PB, (tok * ld * 2u + 16u * piece) | ((uint32_t)!ok << 31),
            res ? 0u : (uint32_t)kk * 2u);
    }
  };
  auto dma = [&](int kc, uint8_t* st, bool valid) {
#pragma unroll
    for (int n = 0; n < 4; ++n) copy(kc, st, valid, n);
  };

  // ---- fragments: transposed W for the A operand (features 128 wm + 32 mb), A rows for B
  uint32_t offA[4];
  {
    const int s2 = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    const uint32_t row = (uint32_t)(8 * (lane >> 5) + ((lane & 15) >> 2)) * XB;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      offA[mb] = row + (uint32_t)((((8 * wm + 2 * mb) ^ (2 * s2)) + g1) << 5) + 8u * (lane & 3);
  }
  uint32_t offB[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rb = wn * 64 + (lane & 31);
    offB[ks] = (uint32_t)XS + (uint32_t)rb * PB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(rb)) << 4);
  }
  f32x16 acc[4][2];
  uint4 ra0[4], rb0[2], ra1[4], rb1[2];
  auto fetch = [&](const uint8_t* st, int ks, uint4 (&ra)[4], uint4 (&rb)[2]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint2 lo = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks) * XB);
      const uint2 hi = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks + 4) * XB);
      ra[mb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) rb[nb] = lds_read16(st, offB[ks] + nb * 32 * PB);
  };

  // Residual. Identity fragment of k-step ks: lane l (column l & 31) holds 1.0 at element
  // (l & 31) - 16 ks - 8 (l >> 5) when that lies in 0..7. Token block nb of this wave sits in
  // chunk nreg + 2 wn + nb; nreg is even (K % 64 == 0), so that chunk is at an odd pipeline
  // position exactly when nb = 1.
  // The fragment is built where it is used (from a laundered lane index), so that it does not
  // hold 8 registers across the main loop.
  auto id_frag = [&](int ks) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int j = (ln & 31) - 16 * ks - 8 * (ln >> 5);
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[q] = (j >> 1) == q ? ((j & 1) ? 0x3F800000u : 0x00003F80u) : 0u;
    return make_uint4(wv[0], wv[1], wv[2], wv[3]);
  };
  auto res_mfma = [&](auto POS, bool on, const uint4 (&ra)[4], int ks) {
    if (on) {
      const uint4 id = id_frag(ks);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][POS.value & 1] = mfma32(as_bf16x8(ra[mb]), as_bf16x8(id), acc[mb][POS.value & 1]);
    }
  };
  constexpr bool has_res = kRes;

  // One chunk c from stage st at pipeline position POS (k-step-0 fragments already in ra0 /
  // rb0); the 4 copies of chunk kc of the copy unit into dst go between the MFMA groups.
  const f32x16 zero16 = {};
  // FIRST: the unit's first chunk, whose k-step-0 MFMAs start the accumulators from zero (an
  // inline constant) instead of reading them, so that nothing has to clear them.
  // late: the previous unit's 16 epilogue stores were issued after the copies of the chunk that
  // `next` waits for, and may stay in flight as well.
  // next is nullptr for the unit's last chunk; its type decides at compile time (a run-time test
  // of the stage pointer, which the compiler cannot prove non-null, put a branch into every chunk).
  // RES (compile time): chunk c, or the chunk kc being copied, may be one of the residual
  // chunks; off in the main loop's groups that lie before them, so that neither the identity
  // MFMAs nor the copy's choice of source put a branch into those chunks.
  auto compute_pipe = [&](auto FIRST, auto POS, const uint8_t* st, int c, int kc, uint8_t* dst, bool valid,
                          auto next, bool late, auto RES) {
    constexpr bool kHasNext = !std::is_same_v<decltype(next), std::nullptr_t>;
    const bool ron = RES.value && has_res && (c == nreg + 2 * wn || c == nreg + 2 * wn + 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] =
            mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    fetch(st, 1, ra1, rb1);
    copy(kc, dst, valid, 0, RES.value);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] =
            mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    copy(kc, dst, valid, 1, RES.value);
    __builtin_amdgcn_sched_barrier(0);
    res_mfma(POS, ron, ra0, 0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(kc, dst, valid, 2, RES.value);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kHasNext) {
      // 3 of this chunk's copies and the 4 of the previous one may stay in flight
      if (late) WAIT_KEEP(23); else WAIT_KEEP(7);
      fetch(next, 0, ra0, rb0);
    }
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(kc, dst, valid, 3, RES.value);
    __builtin_amdgcn_sched_barrier(0);
    res_mfma(POS, ron, ra1, 1);
  };

  set_copy_unit(t);
  dma(0, st0, true);
  dma(1, st1, 1 < nk);
  dma(2, st2, 2 < nk);

  bool first_unit = true;
  const std::integral_constant<bool, true> kFirst;
  const std::integral_constant<bool, false> kNext;
  for (;;) {
    const bool has_next = t + Gx < cnt;
    const int64_t Lc = xs + t;
    const int f0 = (int)(Lc % a.f_tiles) * TF;
    const int64_t t0 = (Lc / a.f_tiles) * TT;
    // The unit's first chunk starts the accumulators (FIRST) when there are more than four
    // chunks; with four, the last group is the first one and they are cleared beforehand.
    if (nk4 == 4) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16;
    }

    // Every chunk is exactly 4 copies per wave, every copy is issued unconditionally and every
    // epilogue issues exactly 16 stores per wave, so the waits are exact: at a chunk boundary
    // the two newer chunks stay in flight, and after the first unit the previous epilogue's
    // stores too, until chunk 3 (issued after them) is awaited. The branches on `late` are
    // uniform.
    const bool late = !first_unit;
    if (late) WAIT_KEEP(24); else WAIT_KEEP(8);
    first_unit = false;
    fetch(st0, 0, ra0, rb0);
    const std::integral_constant<bool, true> kMayRes;
    const std::integral_constant<bool, false> kNoRes;
    if (nk4 > 4) {
      compute_pipe(kFirst, Pos<0>{}, st0, 0, 3, st3, 3 < nk, st1, late, kMayRes);
      compute_pipe(kNext, Pos<1>{}, st1, 1, 4, st0, 4 < nk, st2, late, kMayRes);
      compute_pipe(kNext, Pos<2>{}, st2, 2, 5, st1, 5 < nk, st3, false, kMayRes);
      compute_pipe(kNext, Pos<3>{}, st3, 3, 6, st2, 6 < nk, st0, false, kMayRes);
      int kc = 4;
      // groups whose chunks and copies (3 chunks ahead) all lie before the residual
      for (; kc + 4 < nk4 && (!kRes || kc + 6 < nreg); kc += 4) {
        compute_pipe(kNext, Pos<0>{}, st0, kc, kc + 3, st3, kc + 3 < nk, st1, false, kNoRes);
        compute_pipe(kNext, Pos<1>{}, st1, kc + 1, kc + 4, st0, kc + 4 < nk, st2, false, kNoRes);
        compute_pipe(kNext, Pos<2>{}, st2, kc + 2, kc + 5, st1, kc + 5 < nk, st3, false, kNoRes);
        compute_pipe(kNext, Pos<3>{}, st3, kc + 3, kc + 6, st2, kc + 6 < nk, st0, false, kNoRes);
      }
      if constexpr (kRes) {
        for (; kc + 4 < nk4; kc += 4) {
          compute_pipe(kNext, Pos<0>{}, st0, kc, kc + 3, st3, kc + 3 < nk, st1, false, kMayRes);
          compute_pipe(kNext, Pos<1>{}, st1, kc + 1, kc + 4, st0, kc + 4 < nk, st2, false, kMayRes);
          compute_pipe(kNext, Pos<2>{}, st2, kc + 2, kc + 5, st1, kc + 5 < nk, st3, false, kMayRes);
          compute_pipe(kNext, Pos<3>{}, st3, kc + 3, kc + 6, st2, kc + 6 < nk, st0, false, kMayRes);
        }
      }
    }
    {
      // last four chunks; the next unit's first three are copied meanwhile
      const int kc = nk4 - 4;
      const bool late4 = late && nk4 == 4;
      compute_pipe(kNext, Pos<0>{}, st0, kc, kc + 3, st3, kc + 3 < nk, st1, late4, kMayRes);
      if (has_next) set_copy_unit(t + Gx);
      compute_pipe(kNext, Pos<1>{}, st1, kc + 1, 0, st0, has_next, st2, late4, kMayRes);
      compute_pipe(kNext, Pos<2>{}, st2, kc + 2, 1, st1, has_next && 1 < nk, st3, false, kMayRes);
      compute_pipe(kNext, Pos<3>{}, st3, kc + 3, 2, st2, has_next && 2 < nk, nullptr, false, kMayRes);
    }

    // ---- epilogue through stage 3: wave w uses bytes 4096 w .. +4095, a [32 tokens][64
    // features] bf16 tile whose 16-byte piece c of row r sits at c ^ ((r >> 1) & 7). A wave
    // writes and reads back only its own tile, so after the first barrier (every wave is done
    // reading stage 3) it needs none. Round (nb, fh): token block nb, features 128 wm + 64 fh.
    lds_sync();
    uint8_t* const stg = st3 + wave * 4096;
    // write: row lane & 31, half lane >> 5, piece c at wofs ^ (c << 4); read: row 8 it + (lane >> 3),
    // piece lane & 7, at (rofs ^ ((it & 1) << 6)) + 1024 it (the row's swizzle is 4 (it & 1) + (lane >> 4))
    const uint32_t wofs = ((uint32_t)(lane & 31) * 128u + 8u * (uint32_t)(lane >> 5)) | ((uint32_t)((lane >> 1) & 7) << 4);
    const uint32_t rofs = (uint32_t)(lane >> 3) * 128u + ((uint32_t)((lane & 7) ^ (lane >> 4)) << 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
            if constexpr (kRelu2) {
              const int fl = wm * 128 + (2 * fh + h) * 32 + g * 8 + (lane >> 5) * 4;   // feature in the unit
              const float4 bq = *reinterpret_cast<const float4*>(&s_bias[(f0 + fl) & (kMaxF - 1)]);
              const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float r = fmaxf(acc[2 * fh + h][nb][g * 4 + e] + bb[e], 0.f);
                v[e] = r * r;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[2 * fh + h][nb][g * 4 + e];
            }
            *reinterpret_cast<uint2*>(stg + (wofs ^ ((uint32_t)(4 * h + g) << 4))) =
                make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
          }
        }
        const int f = f0 + wm * 128 + fh * 64 + (lane & 7) * 8;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint4 v = lds_read16(stg, (rofs ^ ((uint32_t)(it & 1) << 6)) + (uint32_t)it * 1024u);
          const int64_t tok = t0 + wn * 64 + nb * 32 + it * 8 + (lane >> 3);
          const bool ok = tok < a.M && f < a.F;
          buf_store16<2>(cr, ok ? (uint32_t)((tok * a.ldc + f) * 2) : OOB, 0, v);   // non-temporal
        }
      }
    }
    if (!has_next) break;
    t += Gx;
  }
  wait_vmem();   // the zero-filled copies issued past the last unit land before the exit
}

hipError_t launch_gemm(const GemmParams& p0, hipStream_t stream) {
  GemmParams p = p0;
  p.f_tiles = (p.F + TF - 1) / TF;
  p.units = (p.M + TT - 1) / TT * p.f_tiles;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t grid = p.units < cus ? p.units : cus;
  if (p.relu2) hipLaunchKernelGGL(gemm_unit_kernel<true>, dim3((unsigned)grid), dim3(512), 0, stream, p);
  else hipLaunchKernelGGL(gemm_unit_kernel<false>, dim3((unsigned)grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_enrich_bf16(const uint16_t* x, int64_t M, int d, int64_t ld_x, const uint16_t* U, int m,
                              const float* bias, uint16_t* z, int64_t ld_z, hipStream_t stream) {
  GemmParams p{};
  p.W = U; p.ldw = m;
  p.A1 = x; p.lda1 = ld_x; p.k1 = d;
  p.A2 = nullptr; p.lda2 = 0;
  p.R = nullptr; p.ldr = 0;
  p.C = z; p.ldc = ld_z;
  p.bias = bias; p.relu2 = 1;
  p.M = M; p.F = m; p.K = d;
  return launch_gemm(p, stream);
}

hipError_t launch_fuse_bf16(const uint16_t* z, int64_t M, int m_h, int64_t ld_z, const uint16_t* c, int m_t,
                            int64_t ld_c, const uint16_t* O, int d, const uint16_t* x_res, int64_t ld_res,
                            uint16_t* y, int64_t ld_y, hipStream_t stream) {
  GemmParams p{};
  p.W = O; p.ldw = d;
  p.A1 = z; p.lda1 = ld_z; p.k1 = m_h;
  p.A2 = c; p.lda2 = ld_c;
  p.R = x_res; p.ldr = ld_res;
  p.C = y; p.ldc = ld_y;
  p.bias = nullptr; p.relu2 = 0;
  p.M = M; p.F = d; p.K = m_h + m_t;
  return launch_gemm(p, stream);
}

}  // namespace avey
