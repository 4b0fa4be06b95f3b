// All-pairs split MaxSim on bf16 MFMA (gfx950).
//
// MaxSim relevance of candidate split j to target split i is the sum over the tokens t of i of
// the largest cosine between x_t and any token u of j (paperlayer.ai "Avey-B" summary,
// section 3; papernotes.org Avey-B note, 方法详解/整体框架). The operands are the L2-normalised
// tokens n_t = N(x_t) (papernotes.org Avey-B note, 关键设计 2), prepared once per call in a
// split-packed bf16 copy (prepare.hip), so that an MFMA tile C = N(X_i) N(X_j)^T holds the
// cosines themselves and both directions of the pair come from it:
//   score(i <- j) = sum_t max_u C_tu          (row direction)
//   score(j <- i) = sum_u max_t C_tu          (column direction)
// Each unordered pair i < j is computed once, and no token-by-token similarity leaves the chip.
//
// Units are 256 target rows x 256 candidate rows (one per pair at S = 256, four at S = 512).
// One workgroup of 8 waves per CU (2 per SIMD), in a 2 x 4 grid: each wave owns 128 x 64 of the
// fp32 accumulator (8 MFMA 32x32x16 blocks). Features stream through a 4-stage LDS ring in
// chunks of 32 by direct global -> LDS copies, three chunks in flight while one is multiplied
// (the copies of a chunk are issued between the MFMA groups of the chunk being multiplied, and
// the wait for the next chunk comes before the last group, whose MFMAs hide the next chunk's
// first fragment reads);
// the next unit's first three chunks are copied while the current one finishes and during its
// epilogue. The packed layout makes every copy instruction read 1 KiB of contiguous memory.
//
// Persistent grid: workgroups are dealt to the 8 XCDs round-robin; each XCD owns one contiguous
// range of pair tiles, walked in bands of 4 target splits, so that the target operands of the
// concurrently resident tiles stay in the XCD's L2 while candidates stream past.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int T = 256;    // rows per unit block (target and candidate)
constexpr int KH = 32;    // K elements per chunk
constexpr int RB = 64;    // bytes per LDS row (one chunk of one token)

// 16-byte piece c of LDS row r sits at position c ^ ((r >> 2) & 3): an MFMA fragment read (16
// consecutive rows, one piece each) then covers the 16 slots of a 256-byte bank window once.
__device__ __forceinline__ uint32_t sw4(int r) { return (uint32_t)((r >> 2) & 3); }

struct MaxsimParams {
  const uint16_t* xp;   // packed N(x): [B][n_s][d / 32][S][32] bf16, padding tokens zero
  int64_t N;
  int d, S, n_s;
  int q;                // 256-row blocks per split
  int pairs;            // unordered pairs per sequence
  int64_t tiles;        // B * pairs
  float* scores;
};

// Unordered pair p of one sequence -> (i, j), i < j. Pairs come in bands of 4 target splits:
// the 6 pairs inside the band, then the band x later-splits rectangle in candidate-major order.
// A full band I holds 4 n_s - 16 I - 10 pairs, so P(I) = I (4 n_s - 2) - 8 I^2 pairs precede it.
__device__ void decode_pair(int p, int n_s, int& i, int& j) {
  const int nfull = n_s / 4;
  auto P = [&](int I) -> long long { return (long long)I * (4LL * n_s - 2) - 8LL * I * I; };
  const long long pfull = P(nfull);
  int i0, h;
  long long rem;
  if (p < pfull) {
    const double bq = 4.0 * n_s - 2.0;
    int I = (int)((bq - sqrt(bq * bq - 32.0 * (double)p)) / 16.0);
    I = max(0, min(I, nfull - 1));
    while (I + 1 < nfull && P(I + 1) <= p) ++I;
    while (I > 0 && P(I) > p) --I;
    i0 = 4 * I;
    h = 4;
    rem = p - P(I);
  } else {
    i0 = 4 * nfull;
    h = n_s - i0;
    rem = p - pfull;
  }
  const int inband = h * (h - 1) / 2;
  if (rem < inband) {
    int r = (int)rem, s = 0;
    while (r >= h - 1 - s) {
      r -= h - 1 - s;
      ++s;
    }
    i = i0 + s;
    j = i + 1 + r;
  } else {
    const int r = (int)(rem - inband);
    j = i0 + h + r / h;
    i = i0 + r % h;
  }
}

struct Unit {
  int64_t b;
  int i, j, ua, ub;   // pair and the unit's target / candidate block
};

// This wave's copies except the newest n are complete, then a workgroup barrier: afterwards
// every wave's older copies have landed in LDS and every wave is done with the previous stage.
#define WAIT_KEEP(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

__global__ void __launch_bounds__(512, 1) maxsim_bf16_kernel(MaxsimParams a) {
  // One LDS object per stage (target block, then candidate block): the compiler tracks copies
  // per object, so reads of one stage do not wait for copies into another. Stage 3 doubles as
  // the epilogue's row-max scratch.
  __shared__ __align__(16) uint8_t st0[2 * T * RB], st1[2 * T * RB], st2[2 * T * RB], st3[2 * T * RB];
  __shared__ __align__(16) float s_biA[T];   // per target row: 0, or -inf for a padding token
  __shared__ float s_biB[T];                 // per candidate row
  __shared__ float s_cm[2][T];               // column maxima of the two row halves
  __shared__ float s_colmax[2 * T];          // running column maxima over target blocks (S = 512)
  __shared__ float s_red[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 2, wn = wave & 3;

  // ---- persistent work split: XCD x owns tiles [xs, xs + cnt); its workgroup l takes every
  // Gx-th of them starting at l.
  const int G = gridDim.x, wg = blockIdx.x, xcd = wg % NXCD, l = wg / NXCD;
  const int Gx = (G - xcd + NXCD - 1) / NXCD;
  const int64_t q8 = a.tiles / NXCD, r8 = a.tiles % NXCD;
  const int64_t xs = xcd * q8 + (xcd < r8 ? xcd : r8), cnt = q8 + (xcd < r8 ? 1 : 0);
  int64_t t = l;
  if (t >= cnt) return;

  const int nk = a.d / KH;
  uint32_t fa[2], fb[2];   // fragment offsets of the two k-steps of a chunk
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ra = wm * 128 + (lane & 31), rb = wn * 64 + (lane & 31);
    fa[ks] = (uint32_t)ra * RB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(ra)) << 4);
    fb[ks] = (uint32_t)rb * RB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(rb)) << 4);
  }

  auto tile_unit = [&](int64_t tl) {
    Unit u;
    const int64_t L = xs + tl;
    u.b = L / a.pairs;
    decode_pair((int)(L % a.pairs), a.n_s, u.i, u.j);
    u.ua = 0;
    u.ub = 0;
    return u;
  };

  // Copy addressing: a descriptor over the unit's sequence and the byte offsets of its two
  // blocks in chunk 0; chunk kc is kc * S * 64 bytes further.
  const uint16_t* xbase = a.xp;   // the copy unit's sequence
  uint32_t xbytes = 0;
  int limA = 0, limB = 0;      // valid (non-padding) rows of the unit's blocks
  uint32_t pbA = 0, pbB = 0;
  auto set_unit = [&](const Unit& u) {
    const int64_t seq = (int64_t)a.n_s * a.S * a.d;
    xbase = a.xp + u.b * seq;
    xbytes = (uint32_t)(seq * 2);
    limA = (int)min((int64_t)min(a.S - u.ua * T, T), a.N - ((int64_t)u.i * a.S + u.ua * T));
    limB = (int)min((int64_t)min(a.S - u.ub * T, T), a.N - ((int64_t)u.j * a.S + u.ub * T));
    pbA = (uint32_t)((int64_t)u.i * a.S * a.d * 2 + u.ua * T * RB);
    pbB = (uint32_t)((int64_t)u.j * a.S * a.d * 2 + u.ub * T * RB);
  };
  // Chunk kc of the current copy unit into stage st: wave w copies rows [32w, 32w + 32) of both
  // blocks, 16 rows (1 KiB) per instruction, 4 instructions. Lane l lands at LDS row l >> 2,
  // position l & 3, so it fetches the logical piece (l & 3) ^ sw4(row). Lane terms are
  // recomputed per copy (laundered through an empty asm so they are not hoisted into long-lived
  // registers). With valid == false every lane loads zeros.
  auto dma = [&](int kc, uint8_t* st, bool valid) {
    int sub = lane >> 2;
    asm volatile("" : "+v"(sub));
    const uint32_t kb = (uint32_t)kc * (uint32_t)a.S * RB;
    const uint32_t c = (uint32_t)sub * RB + 16u * (uint32_t)((lane & 3) ^ ((sub >> 2) & 3));
    const uint32_t laneA = pbA + c, laneB = pbB + c;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int r0 = wave * 32 + n * 16;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc_uniform(xbase, xbytes);
      dma16(xr, st + r0 * RB, valid ? laneA + (uint32_t)r0 * RB : OOB, kb);
      dma16(xr, st + T * RB + r0 * RB, valid ? laneB + (uint32_t)r0 * RB : OOB, kb);
    }
  };

  f32x16 acc[4][2];
  // Fragments of k-step 0 (ra0, rb0) and 1 (ra1, rb1) of the chunk being multiplied.
  uint4 ra0[4], rb0[2], ra1[4], rb1[2];
  auto fetch0 = [&](const uint8_t* st) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) ra0[mb] = lds_read16(st, fa[0] + mb * 32 * RB);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) rb0[nb] = lds_read16(st + T * RB, fb[0] + nb * 32 * RB);
  };
  auto fetch1 = [&](const uint8_t* st) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) ra1[mb] = lds_read16(st, fa[1] + mb * 32 * RB);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) rb1[nb] = lds_read16(st + T * RB, fb[1] + nb * 32 * RB);
  };
  // One chunk from stage st whose k-step-0 fragments are already in ra0 / rb0; the 4 copies of
  // chunk kc into dst go between the MFMA groups. With next != nullptr the next chunk's wait
  // and barrier come before the last MFMA group, and its k-step-0 fragments are read under it.
  // FIRST: the unit's first chunk, whose k-step-0 MFMAs start the accumulators from zero (an
  // inline constant) instead of reading them, so that nothing has to clear them.
  const f32x16 zero16 = {};
  auto compute_pipe = [&](auto FIRST, const uint8_t* st, int kc, uint8_t* dst, bool valid, const uint8_t* next) {
    int sub = lane >> 2;
    asm volatile("" : "+v"(sub));
    const uint32_t kb = (uint32_t)kc * (uint32_t)a.S * RB;
    const uint32_t c = (uint32_t)sub * RB + 16u * (uint32_t)((lane & 3) ^ ((sub >> 2) & 3));
    const uint32_t laneA = pbA + c, laneB = pbB + c;
    auto copy = [&](int ks, int h) {
      const int r0 = wave * 32 + ks * 16;
      // the descriptor is rebuilt from the first lane at each copy: carried across the loop it
      // is taken as per-lane, and every copy through it became a loop over distinct values
      const __amdgpu_buffer_rsrc_t xr = make_rsrc_uniform(xbase, xbytes);
      if (h == 0) dma16(xr, dst + r0 * RB, valid ? laneA + (uint32_t)r0 * RB : OOB, kb);
      else dma16(xr, dst + T * RB + r0 * RB, valid ? laneB + (uint32_t)r0 * RB : OOB, kb);
    };
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    fetch1(st);
    copy(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    copy(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (next) {
      // 3 of this chunk's copies and the 4 of the previous one may stay in flight
      WAIT_KEEP(7);
      fetch0(next);
    }
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(1, 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Thread tid < 256 owns target row tid of the unit, thread tid >= 256 candidate column
  // tid - 256; part accumulates its share of the pair's score.
  const bool is_row = tid < T;
  const int own = tid & (T - 1);
  float rmax = 0.f, part = 0.f;

  Unit cur = tile_unit(t);
  set_unit(cur);
  dma(0, st0, true);
  dma(1, st1, 1 < nk);
  dma(2, st2, 2 < nk);
  // Chunk count padded to a multiple of 4 with zero chunks so that every unit starts on stage 0.
  const int nk4 = (nk + 3) / 4 * 4;

  for (;;) {
    // ---- what comes after this unit: candidate blocks inner, target blocks outer, then tiles
    Unit nx = cur;
    bool has_next = true;
    if (cur.ub + 1 < a.q) {
      nx.ub = cur.ub + 1;
    } else if (cur.ua + 1 < a.q) {
      nx.ua = cur.ua + 1;
      nx.ub = 0;
    } else if (t + Gx < cnt) {
      nx = tile_unit(t + Gx);
    } else {
      has_next = false;
    }
    const int cLimA = limA, cLimB = limB;
    const bool valid = own < (is_row ? cLimA : cLimB);

    // ---- K loop. Every copy is issued unconditionally (a control-flow join around a copy
    // makes the compiler drain all copies before the next LDS read) and every chunk is exactly
    // 4 copies per wave, so WAIT_KEEP(8) at a chunk boundary (WAIT_KEEP(7) before the last MFMA
    // group, with 3 of the current chunk's copies issued) leaves exactly the newer copies in
    // flight.
    // The unit's first chunk starts the accumulators (FIRST) when there are more than four
    // chunks; with four, the last group is the first one and they are cleared beforehand.
    const std::integral_constant<bool, true> kFirst;
    const std::integral_constant<bool, false> kNext;
    if (nk4 == 4) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16;
    }
    WAIT_KEEP(8);
    fetch0(st0);
    if (nk4 > 4) {
      compute_pipe(kFirst, st0, 3, st3, 3 < nk, st1);
      compute_pipe(kNext, st1, 4, st0, 4 < nk, st2);
      compute_pipe(kNext, st2, 5, st1, 5 < nk, st3);
      compute_pipe(kNext, st3, 6, st2, 6 < nk, st0);
      for (int kc = 4; kc + 4 < nk4; kc += 4) {
        compute_pipe(kNext, st0, kc + 3, st3, kc + 3 < nk, st1);
        compute_pipe(kNext, st1, kc + 4, st0, kc + 4 < nk, st2);
        compute_pipe(kNext, st2, kc + 5, st1, kc + 5 < nk, st3);
        compute_pipe(kNext, st3, kc + 6, st2, kc + 6 < nk, st0);
      }
    }
    {
      // last four chunks; the next unit's first three are copied meanwhile
      const int kc = nk4 - 4;
      compute_pipe(kNext, st0, kc + 3, st3, kc + 3 < nk, st1);
      if (has_next) set_unit(nx);
      compute_pipe(kNext, st1, 0, st0, has_next, st2);
      compute_pipe(kNext, st2, 1, st1, has_next && 1 < nk, st3);
      compute_pipe(kNext, st3, 2, st2, has_next && 2 < nk, nullptr);
    }

    // ---- epilogue (the next unit's first three chunks are in flight into stages 0-2)
    const bool first_ub = cur.ub == 0, last_ub = cur.ub == a.q - 1;
    const bool first_ua = cur.ua == 0, last_ua = cur.ua == a.q - 1;
    const bool full = cLimA == T && cLimB == T;   // no padding token in this unit
    // (two stores to named arrays: a store through a selected pointer would make the compiler
    // wait for the copies in flight)
    if (is_row) s_biA[own] = valid ? 0.f : -INFINITY;
    else s_biB[own] = valid ? 0.f : -INFINITY;
    lds_sync();   // also: every wave is done reading stage 3

    // One pass over the accumulators, both directions:
    //   column u: max over this wave's 128 rows -> cm, then across the two row halves
    //   row t:    max over this wave's 64 columns -> scratch [128 rows][8 lane quads] per wave
    // A two-step transposing max across the 4 lanes of a quad leaves lane q with row e = q of
    // each group of 4 rows, so each lane stores one value per group.
    const int q = lane & 3, par = lane & 1, hi2 = (lane >> 1) & 1;
    float* const wscr = reinterpret_cast<float*>(st3) + wave * (128 * 8) + ((lane & 31) >> 2);
    float cm[2] = {-INFINITY, -INFINITY};
    auto reduce_store = [&](int mb, int g, const float (&m)[4]) {
      // step 1, lanes l and l ^ 1: the even lane keeps rows e = 0, 2, the odd lane e = 1, 3
      const float s0 = par ? m[0] : m[1], k0 = par ? m[1] : m[0];
      const float s1 = par ? m[2] : m[3], k1 = par ? m[3] : m[2];
      const float t0 = fmaxf(k0, __builtin_amdgcn_update_dpp(0.f, s0, 0xB1, 0xF, 0xF, false));
      const float t1 = fmaxf(k1, __builtin_amdgcn_update_dpp(0.f, s1, 0xB1, 0xF, 0xF, false));
      // step 2, lanes l and l ^ 2: keep row e = par (hi2 == 0) or e = par + 2 (hi2 == 1)
      const float s2 = hi2 ? t0 : t1, k2 = hi2 ? t1 : t0;
      const float f = fmaxf(k2, __builtin_amdgcn_update_dpp(0.f, s2, 0x4E, 0xF, 0xF, false));
      wscr[(mb * 32 + g * 8 + (lane >> 5) * 4 + q) * 8] = f;
    };
    // Accumulator element v of block (mb, nb) in lane l: row mb*32 + 8(v >> 2) + 4(l >> 5) + (v & 3)
    // of the wave's rows, column nb*32 + (l & 31) of its columns.
    if (full) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float m[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c0 = acc[mb][0][g * 4 + e], c1 = acc[mb][1][g * 4 + e];
            m[e] = fmaxf(c0, c1);
            cm[0] = fmaxf(cm[0], c0);
            cm[1] = fmaxf(cm[1], c1);
          }
          reduce_store(mb, g, m);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // padding tokens take part in neither the max nor the sum: bias them to -inf
      float cbi[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) cbi[nb] = s_biB[wn * 64 + nb * 32 + (lane & 31)];
      const float* biA_lane = s_biA + wm * 128 + (lane >> 5) * 4;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 rbi = *reinterpret_cast<const float4*>(biA_lane + mb * 32 + g * 8);
          const float rb4[4] = {rbi.x, rbi.y, rbi.z, rbi.w};
          float m[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c0 = acc[mb][0][g * 4 + e], c1 = acc[mb][1][g * 4 + e];
            m[e] = fmaxf(c0 + cbi[0], c1 + cbi[1]);
            cm[0] = fmaxf(cm[0], c0 + rb4[e]);
            cm[1] = fmaxf(cm[1], c1 + rb4[e]);
          }
          reduce_store(mb, g, m);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float m = fmaxf(cm[nb], __shfl_xor(cm[nb], 32));
      if (lane < 32) s_cm[wm][wn * 64 + nb * 32 + lane] = m;
    }
    lds_sync();
    if (is_row) {
      // target row own: 8 quad maxima from each of the 4 waves that hold its columns
      const int wr = own >> 7, rl = own & 127;
      const float* p = reinterpret_cast<const float*>(st3) + wr * (4 * 128 * 8) + rl * 8;
      float m = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int cc = ((c + (rl >> 3)) & 1) * 4;   // rotation: no bank conflicts
          const float4 u = *reinterpret_cast<const float4*>(p + w * (128 * 8) + cc);
          m = fmaxf(m, fmaxf(fmaxf(u.x, u.y), fmaxf(u.z, u.w)));
        }
      }
      rmax = first_ub ? m : fmaxf(rmax, m);
      if (last_ub && valid) part += rmax;
    } else {
      float cmv = fmaxf(s_cm[0][own], s_cm[1][own]);
      if (!first_ua) cmv = fmaxf(cmv, s_colmax[cur.ub * T + own]);
      if (!last_ua) s_colmax[cur.ub * T + own] = cmv;
      else if (valid) part += cmv;
    }

    if (last_ua && last_ub) {
      // ---- scores of the pair; fixed reduction order (bitwise reproducible)
      float r = part;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) r += __shfl_xor(r, o);
      if (lane == 0) s_red[wave] = r;
      lds_sync();
      if (tid == 0) {
        const float tr = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
        const float tc = ((s_red[4] + s_red[5]) + s_red[6]) + s_red[7];
        float* sb = a.scores + cur.b * (int64_t)a.n_s * a.n_s;
        sb[(int64_t)cur.i * a.n_s + cur.j] = tr;
        sb[(int64_t)cur.j * a.n_s + cur.i] = tc;
        if (cur.j == cur.i + 1) {
          sb[(int64_t)cur.i * a.n_s + cur.i] = -INFINITY;
          if (cur.j == a.n_s - 1) sb[(int64_t)cur.j * a.n_s + cur.j] = -INFINITY;
        }
      }
      part = 0.f;
    }

    if (!has_next) break;
    if (nx.ua == 0 && nx.ub == 0) t += Gx;
    cur = nx;
    lds_sync();   // this epilogue's LDS reads are done before stage 3 is refilled
  }
  wait_vmem();    // the zero-filled copies issued past the last unit land before the exit
}

}  // namespace

hipError_t launch_maxsim_bf16(const uint16_t* xp, int64_t B, int64_t N, int d, int S, float* scores,
                              hipStream_t stream) {
  MaxsimParams p;
  p.xp = xp;
  p.N = N;
  p.d = d;
  p.S = S;
  p.n_s = (int)((N + S - 1) / S);
  p.q = (S + T - 1) / T;
  p.pairs = (int)((int64_t)p.n_s * (p.n_s - 1) / 2);
  p.tiles = B * (int64_t)p.pairs;
  p.scores = scores;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t grid = p.tiles < cus ? p.tiles : cus;
  hipLaunchKernelGGL(maxsim_bf16_kernel, dim3((unsigned)grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
