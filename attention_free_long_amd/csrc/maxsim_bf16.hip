// All-pairs split MaxSim on bf16 MFMA (gfx950).
//
// MaxSim relevance of candidate split j to target split i is the sum over the tokens t of i of
// the largest cosine between x_t and any token u of j (paperlayer.ai "Avey-B" summary,
// section 3; papernotes.org Avey-B note, 方法详解/整体框架). Both directions of a split pair
// come from the same dot-product tile C = X_i X_j^T:
//   score(i <- j) = sum_t rn_t * max_u (C_tu * rn_u)      (row direction)
//   score(j <- i) = sum_u rn_u * max_t (C_tu * rn_t)      (column direction)
// with rn = 1 / |x| (0 for a zero vector; precomputed once per token), because rn_t >= 0
// factors out of the max. So each unordered pair i < j is computed once for both directions,
// and no token-by-token similarity ever leaves the chip.
//
// Persistent grid, one workgroup per CU. Workgroups are dealt to the 8 XCDs round-robin; each
// XCD owns one contiguous range of pair tiles, and its 32 workgroups walk that range 32 tiles at
// a time, so concurrently resident tiles span about 4 target x 8 candidate splits and share
// operands in the XCD's L2.
//
// A pair is processed in units of 256 target rows x 128 candidate rows (2 units per pair at
// S = 256, 8 at S = 512); row maxima run across the units of a pair, column maxima across its
// target blocks. Workgroup: 256 threads = 4 waves in a 2 x 2 grid, each wave owning 128 x 64 of
// the fp32 accumulator (8 MFMA 32x32x16 blocks, 128 accumulator registers). Features stream
// through LDS in chunks of 64 by direct global -> LDS copies, double-buffered; the next unit's
// first chunk is copied during the current unit's last chunk.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int TA = 256;   // target rows per unit
constexpr int TB = 128;   // candidate rows per unit

struct MaxsimParams {
  const uint16_t* x;
  const float* rn;
  int64_t N, ld_x;
  int d, S, n_s;
  int qa, qb;      // 256-row target blocks and 128-row candidate blocks per split
  int pairs;       // unordered pairs per sequence
  int64_t tiles;   // B * pairs
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

__global__ void __launch_bounds__(256, 1) maxsim_bf16_kernel(MaxsimParams a) {
  // Named stage buffers: separate LDS objects let the compiler see that reads of one stage do not
  // depend on copies in flight into the other. sA1 doubles as the epilogue's row-max scratch.
  __shared__ __align__(16) uint8_t sA0[TA * ROWB], sB0[TB * ROWB], sA1[TA * ROWB], sB1[TB * ROWB];
  __shared__ __align__(16) float2 s_sbA[TA];   // per target row: (rn, 0), or (0, -inf) for padding
  __shared__ __align__(16) float2 s_sbB[TB];   // per candidate row
  __shared__ float s_cm[2][TB];                // column maxima of the two row halves
  __shared__ float s_colmax[4 * TB];           // running column maxima over target blocks
  __shared__ float s_red[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 1, wn = wave & 1;

  // ---- persistent work split: XCD x owns tiles [xs, xs + cnt); its workgroup l takes every
  // Gx-th of them starting at l.
  const int G = gridDim.x, wg = blockIdx.x, xcd = wg % NXCD, l = wg / NXCD;
  const int Gx = (G - xcd + NXCD - 1) / NXCD;
  const int64_t q8 = a.tiles / NXCD, r8 = a.tiles % NXCD;
  const int64_t xs = xcd * q8 + (xcd < r8 ? xcd : r8), cnt = q8 + (xcd < r8 ? 1 : 0);
  int64_t t = l;
  if (t >= cnt) return;

  const int nk = a.d / KC;
  uint32_t fa[4], fb[4];
  frag_offsets<SWZ_ROW>(fa, wm * 128, lane);
  frag_offsets<SWZ_ROW>(fb, wn * 64, lane);

  auto tile_unit = [&](int64_t tl) {
    Unit u;
    const int64_t L = xs + tl;
    u.b = L / a.pairs;
    decode_pair((int)(L % a.pairs), a.n_s, u.i, u.j);
    u.ua = 0;
    u.ub = 0;
    return u;
  };

  // Copy addressing: scalar state per unit plus lane terms recomputed at every copy (laundered
  // through an empty asm so they are not hoisted into long-lived registers). Wave w copies target
  // rows [64w, 64w + 64) and candidate rows [32w, 32w + 32), 8 rows per instruction; lane l lands
  // in chunk position (l & 7) of row (l >> 3) of the group, i.e. fetches the logical chunk
  // (l & 7) ^ swz(row) with swz(row) = (row >> 1) & 7.
  __amdgpu_buffer_rsrc_t xr;
  int64_t rowA0 = 0, rowB0 = 0;   // first token of the unit's target / candidate block
  int limA = 0, limB = 0;         // valid rows of those blocks
  auto set_unit = [&](const Unit& u) {
    xr = make_rsrc(a.x + u.b * a.N * a.ld_x, (uint32_t)(a.N * a.ld_x * 2));
    rowA0 = (int64_t)u.i * a.S + u.ua * TA;
    rowB0 = (int64_t)u.j * a.S + u.ub * TB;
    limA = (int)min((int64_t)min(a.S - u.ua * TA, TA), a.N - rowA0);
    limB = (int)min((int64_t)min(a.S - u.ub * TB, TB), a.N - rowB0);
  };
  // Copy chunk kc of the current copy unit; with valid == false every lane loads zeros.
  auto dma = [&](int kc, uint8_t* dA, uint8_t* dB, bool valid) {
    int sub = lane >> 3;
    asm volatile("" : "+v"(sub));
    const uint32_t kb = (uint32_t)kc * KC * 2;
    const uint32_t ldb = (uint32_t)a.ld_x * 2;
    const uint32_t c0 = 16u * (uint32_t)((lane & 7) ^ (sub >> 1));
    const uint32_t laneA = (uint32_t)sub * ldb + (uint32_t)(rowA0 * ldb);
    const uint32_t laneB = (uint32_t)sub * ldb + (uint32_t)(rowB0 * ldb);
    const int la = valid ? limA : 0, lb = valid ? limB : 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int r0 = wave * 64 + n * 8;
      const uint32_t c = (n & 1) ? (c0 ^ 64u) : c0;
      dma16(xr, dA + r0 * ROWB, r0 + sub < la ? laneA + (uint32_t)r0 * ldb + c : OOB, kb);
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int r0 = wave * 32 + n * 8;
      const uint32_t c = (n & 1) ? (c0 ^ 64u) : c0;
      dma16(xr, dB + r0 * ROWB, r0 + sub < lb ? laneB + (uint32_t)r0 * ldb + c : OOB, kb);
    }
  };

  f32x16 acc[4][2];
  // Fragments of k-step ks + 1 are read while the MFMAs of k-step ks run; scheduling barriers
  // keep the compiler from hoisting more reads (and registers) than that.
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
    uint4 ra[2][4], rb[2][2];
    auto fetch = [&](int ks, int slot) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) ra[slot][mb] = lds_read16(sa, fa[ks] + mb * 32 * ROWB);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) rb[slot][nb] = lds_read16(sb, fb[ks] + nb * 32 * ROWB);
    };
    fetch(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks < 3) fetch(ks + 1, cur ^ 1);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = mfma32(as_bf16x8(ra[cur][mb]), as_bf16x8(rb[cur][nb]), acc[mb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Row-max scratch in sA1: wave w owns [128 rows][16 lane pairs] fp32 (8 KB). After a pair-max
  // across lanes 2p and 2p+1, the even lane stores the rows with (v & 1) == 0, the odd one the rest.
  float* const scr = reinterpret_cast<float*>(sA1);

  // Per-thread partial scores of the current pair: thread tid owns target row tid of the target
  // block and (tid < 128) candidate column tid of the candidate block.
  float rmax = 0.f, sr = 0.f, sc = 0.f;

  Unit cur = tile_unit(t);
  set_unit(cur);
  dma(0, sA0, sB0, true);
  copy_sync();
  // An odd chunk count gets one zero chunk so that every unit starts on stage 0.
  const int nk2 = (nk + 1) & ~1;

  for (;;) {
    // ---- what comes after this unit: candidate blocks inner, target blocks outer, then tiles
    Unit nx = cur;
    bool has_next = true;
    if (cur.ub + 1 < a.qb) {
      nx.ub = cur.ub + 1;
    } else if (cur.ua + 1 < a.qa) {
      nx.ua = cur.ua + 1;
      nx.ub = 0;
    } else if (t + Gx < cnt) {
      nx = tile_unit(t + Gx);
    } else {
      has_next = false;
    }
    const int64_t cb = cur.b, cA0 = rowA0, cB0 = rowB0;
    const int cLimA = limA, cLimB = limB;

    // ---- K loop over the features, two stages. The last copy of the loop is the next unit's
    // first chunk, so no copy is in flight during the epilogue, and every copy is issued
    // unconditionally (control-flow joins would make the compiler wait for all copies before
    // the next LDS read).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
    for (int kc = 0; kc < nk2; kc += 2) {
      dma(kc + 1, sA1, sB1, kc + 1 < nk);
      compute(sA0, sB0);
      copy_sync();
      const bool last = kc + 2 >= nk2;
      if (last && has_next) set_unit(nx);
      dma(last ? 0 : kc + 2, sA0, sB0, !last || has_next);
      compute(sA1, sB1);
      copy_sync();
    }

    // ---- epilogue (no copies in flight)
    const bool vA = tid < cLimA;
    const bool vB = tid < cLimB;            // false for tid >= TB
    const float* rnb = a.rn + cb * a.N;
    const float rA = vA ? rnb[cA0 + tid] : 0.f;
    const float rB = vB ? rnb[cB0 + tid] : 0.f;
    const bool first_ub = cur.ub == 0, last_ub = cur.ub == a.qb - 1;
    const bool first_ua = cur.ua == 0, last_ua = cur.ua == a.qa - 1;
    const int ubc = cur.ub;
    s_sbA[tid] = make_float2(rA, vA ? 0.f : -INFINITY);
    if (tid < TB) s_sbB[tid] = make_float2(rB, vB ? 0.f : -INFINITY);
    lds_sync();

    // One pass over the accumulators, both directions:
    //   column u: max over this wave's rows t of C_tu * rn_t (padding rows -> -inf)
    //   row t:    max over this wave's 64 columns u of C_tu * rn_u -> scratch
    float csc[2], cbi[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float2 s = s_sbB[wn * 64 + nb * 32 + (lane & 31)];
      csc[nb] = s.x;
      cbi[nb] = s.y;
    }
    const float2* sbA_lane = s_sbA + wm * 128 + (lane >> 5) * 4;
    float* const wscr = scr + wave * (128 * 16) + ((lane & 31) >> 1);
    const int par = lane & 1;
    float cm[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 p01 = *reinterpret_cast<const float4*>(sbA_lane + mb * 32 + g * 8);
        const float4 p23 = *reinterpret_cast<const float4*>(sbA_lane + mb * 32 + g * 8 + 2);
        const float rsc[4] = {p01.x, p01.z, p23.x, p23.z};
        const float rbi[4] = {p01.y, p01.w, p23.y, p23.w};
        float m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c0 = acc[mb][0][g * 4 + e], c1 = acc[mb][1][g * 4 + e];
          m[e] = fmaxf(fmaf(c0, csc[0], cbi[0]), fmaf(c1, csc[1], cbi[1]));
          cm[0] = fmaxf(cm[0], fmaf(c0, rsc[e], rbi[e]));
          cm[1] = fmaxf(cm[1], fmaf(c1, rsc[e], rbi[e]));
          // pair-max with the neighbouring lane (DPP quad_perm [1, 0, 3, 2])
          m[e] = fmaxf(m[e], __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                 0, __builtin_bit_cast(int, m[e]), 0xB1, 0xF, 0xF, false)));
        }
        // rows of this g-group: mb*32 + 8g + 4h + e; even lane stores e = 0, 2, odd lane e = 1, 3
        const int rbase = mb * 32 + g * 8 + (lane >> 5) * 4;
        wscr[(rbase + par) * 16] = par ? m[1] : m[0];
        wscr[(rbase + 2 + par) * 16] = par ? m[3] : m[2];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float m = fmaxf(cm[nb], __shfl_xor(cm[nb], 32));
      if (lane < 32) s_cm[wm][wn * 64 + nb * 32 + lane] = m;
    }
    lds_sync();
    {
      // target row tid: the 16 + 16 pair maxima of waves (wr, 0) and (wr, 1)
      const int wr = tid >> 7, rl = tid & 127;
      const float* p0 = scr + (wr * 2 + 0) * (128 * 16) + rl * 16;
      const float* p1 = scr + (wr * 2 + 1) * (128 * 16) + rl * 16;
      float m = -INFINITY;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = ((c + rl) & 3) * 4;
        const float4 u = *reinterpret_cast<const float4*>(p0 + cc);
        const float4 w = *reinterpret_cast<const float4*>(p1 + cc);
        m = fmaxf(m, fmaxf(fmaxf(u.x, u.y), fmaxf(u.z, u.w)));
        m = fmaxf(m, fmaxf(fmaxf(w.x, w.y), fmaxf(w.z, w.w)));
      }
      rmax = first_ub ? m : fmaxf(rmax, m);
      if (last_ub && vA) sr += rA * rmax;
      if (tid < TB) {
        float cmv = fmaxf(s_cm[0][tid], s_cm[1][tid]);
        if (!first_ua) cmv = fmaxf(cmv, s_colmax[ubc * TB + tid]);
        if (!last_ua) s_colmax[ubc * TB + tid] = cmv;
        else if (vB) sc += rB * cmv;
      }
    }

    if (last_ua && last_ub) {
      // ---- scores of the pair; fixed reduction order (bitwise reproducible)
      float r = sr, c = sc;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        r += __shfl_xor(r, o);
        c += __shfl_xor(c, o);
      }
      if (lane == 0) {
        s_red[wave] = r;
        s_red[4 + wave] = c;
      }
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
      sr = 0.f;
      sc = 0.f;
    }

    if (!has_next) break;
    if (nx.ua == 0 && nx.ub == 0) t += Gx;
    cur = nx;
    lds_sync();   // this epilogue's LDS reads are done before stage 1 is refilled
  }
}

}  // namespace

hipError_t launch_maxsim_bf16(const uint16_t* x, const float* rn, int64_t B, int64_t N, int d, int64_t ld_x, int S,
                              float* scores, hipStream_t stream) {
  MaxsimParams p;
  p.x = x;
  p.rn = rn;
  p.N = N;
  p.ld_x = ld_x;
  p.d = d;
  p.S = S;
  p.n_s = (int)((N + S - 1) / S);
  p.qa = (S + TA - 1) / TA;
  p.qb = (S + TB - 1) / TB;
  p.pairs = (int)((int64_t)p.n_s * (p.n_s - 1) / 2);
  p.tiles = B * (int64_t)p.pairs;
  p.scores = scores;
  int dev = 0, cus = 0;
  hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  const int64_t grid = p.tiles < cus ? p.tiles : cus;
  hipLaunchKernelGGL(maxsim_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
