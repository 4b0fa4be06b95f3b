// All-pairs split MaxSim on bf16 MFMA (gfx950).
//
// MaxSim relevance of candidate split j to target split i is the sum over the tokens t of i of
// the largest cosine between x_t and any token u of j (paperlayer.ai "Avey-B" summary,
// section 3; papernotes.org Avey-B note, 方法详解/整体框架). Both directions of a split pair
// come from the same dot-product tile C = X_i X_j^T:
//   score(i <- j) = sum_t rn_t * max_u (C_tu * rn_u)      (row direction)
//   score(j <- i) = sum_u rn_u * max_t (C_tu * rn_t)      (column direction)
// with rn = 1 / |x| (0 for a zero vector), because rn_t > 0 factors out of the max. So one
// workgroup per unordered pair i < j computes the tile once and writes both scores; the tile
// never leaves the chip.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid, each wave owning 128 x 128 of the 256 x 256
// fp32 accumulator (16 MFMA 32x32x16 blocks). Features stream through LDS in chunks of 64
// (double-buffered, 2 x 64 KB). Splits longer than 256 tokens are covered by up to 2 x 2
// quadrants with running row / column maxima in LDS. Sums of squares for the token norms are
// accumulated from the same LDS fragments the MFMAs consume (dot2 instructions issued between
// the MFMAs).
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int TILE = 256;
constexpr int BAND = 4;
constexpr int RP_STRIDE = 36;   // floats per row of the transposed row-max scratch (144 B)

struct MaxsimParams {
  const uint16_t* x;
  int64_t N, ld_x;
  int d, S, n_s, q;
  int64_t pairs;   // unordered pairs per sequence
  int64_t tiles;   // B * pairs
  float* scores;
};

// Unordered pair p of one sequence -> (i, j), i < j. Pairs are grouped in bands of BAND
// target splits: first the pairs inside the band, then the band x later-splits rectangle in
// candidate-major order, so 32 consecutive pairs touch about 4 + 8 distinct splits.
__device__ void decode_pair(int64_t p, int n_s, int& i, int& j) {
  int i0 = 0;
  for (;;) {
    const int h = min(BAND, n_s - i0);
    const int64_t inband = (int64_t)h * (h - 1) / 2;
    const int64_t rect = (int64_t)h * (n_s - i0 - h);
    if (p < inband) {
      int a = 0;
      while (p >= h - 1 - a) { p -= h - 1 - a; ++a; }
      i = i0 + a;
      j = i + 1 + (int)p;
      return;
    }
    p -= inband;
    if (p < rect) {
      j = i0 + h + (int)(p / h);
      i = i0 + (int)(p % h);
      return;
    }
    p -= rect;
    i0 += h;
  }
}

struct Smem {
  float sq[2][1][TILE];               // [A|B][.][row]: sums of squares of the tile's rows
  float2 sbA[TILE], sbB[TILE];        // per row / column: (rn, 0) or (0, -inf) when padding
  float cm[2][TILE];                  // column maxima of the two row halves
  float rowmax[2 * TILE], colmax[2 * TILE], rnA[2 * TILE], rnB[2 * TILE];
  float red[8];
};

template <int Q>
__global__ void __launch_bounds__(256, 1) maxsim_bf16_kernel(MaxsimParams a) {
  // Two named stage buffers per operand: separate LDS objects let the compiler see that
  // reads of one stage do not depend on the in-flight copies into the other.
  __shared__ __align__(16) uint8_t sA0[TILE * ROWB], sB0[TILE * ROWB], sA1[TILE * ROWB], sB1[TILE * ROWB];
  __shared__ __align__(16) Smem sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 1, wn = wave & 1;

  const int64_t L = xcd_remap(blockIdx.x, a.tiles);
  const int64_t b = L / a.pairs;
  int i, j;
  decode_pair(L % a.pairs, a.n_s, i, j);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x + b * a.N * a.ld_x, (uint32_t)(a.N * a.ld_x * 2));
  const int nk = a.d / KC;
  const int64_t baseI = (int64_t)i * a.S, baseJ = (int64_t)j * a.S;

  // Copy role: wave w fills rows [64w, 64w + 64) of both operands, eight rows per instruction;
  // lane l lands in LDS chunk position (l & 7) of row (l >> 3) of that group, so it fetches the
  // logical chunk (l & 7) ^ swz(row).
  const int ld_sub = lane >> 3, ld_pos = lane & 7;
  // Fragment read offsets: A rows of this wave start at 128 wm, B rows at 128 wn.
  uint32_t fa[4], fb[4];
  frag_offsets<SWZ_ROW>(fa, wm * 128, lane);
  frag_offsets<SWZ_ROW>(fb, wn * 128, lane);

  for (int qi = 0; qi < Q; ++qi) {
    for (int qj = 0; qj < Q; ++qj) {
      // Byte offsets (within the sequence) of this lane's 8 A rows and 8 B rows; padding rows
      // point past the descriptor and read as zero.
      uint32_t offA[8], offB[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int row = wave * 64 + n * 8 + ld_sub;
        const uint32_t c = (uint32_t)(ld_pos ^ (int)swz<SWZ_ROW>(row));
        const int slotA = qi * TILE + row, slotB = qj * TILE + row;
        const bool vA = slotA < a.S && baseI + slotA < a.N;
        const bool vB = slotB < a.S && baseJ + slotB < a.N;
        offA[n] = vA ? (uint32_t)((baseI + slotA) * a.ld_x * 2) + 16u * c : OOB;
        offB[n] = vB ? (uint32_t)((baseJ + slotB) * a.ld_x * 2) + 16u * c : OOB;
      }

      f32x16 acc[4][4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
      float sqA[4] = {0.f, 0.f, 0.f, 0.f}, sqB[4] = {0.f, 0.f, 0.f, 0.f};

      auto dma = [&](int kc, uint8_t* dA, uint8_t* dB) {
        const uint32_t kb = (uint32_t)kc * KC * 2;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const uint32_t o = (uint32_t)(wave * 64 + n * 8) * ROWB;
          dma16(xr, dA + o, offA[n], kb);
          dma16(xr, dB + o, offB[n], kb);
        }
      };
      // Fragments of k-step ks + 1 are read while the MFMAs of k-step ks run; scheduling
      // barriers keep the compiler from hoisting more reads (and registers) than that.
      auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
        uint4 ra[2][4], rb[2][4];
        auto fetch = [&](int ks, int slot) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) ra[slot][mb] = lds_read16(sa, fa[ks] + mb * 32 * ROWB);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) rb[slot][nb] = lds_read16(sb, fb[ks] + nb * 32 * ROWB);
        };
        fetch(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int cur = ks & 1;
          if (ks < 3) fetch(ks + 1, cur ^ 1);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = mfma32(as_bf16x8(ra[cur][mb]), as_bf16x8(rb[cur][nb]), acc[mb][nb]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) sqA[mb] = sumsq8(ra[cur][mb], sqA[mb]);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) sqB[nb] = sumsq8(rb[cur][nb], sqB[nb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // Double-buffered K loop over the features, unrolled by two stages; an odd last chunk is
      // peeled so the accumulators flow through one straight path.
      dma(0, sA0, sB0);
      wait_vmem();
      __syncthreads();
      int kc = 0;
      for (; kc + 2 <= nk; kc += 2) {
        dma(kc + 1, sA1, sB1);
        compute(sA0, sB0);
        wait_vmem();
        __syncthreads();
        if (kc + 2 < nk) dma(kc + 2, sA0, sB0);
        compute(sA1, sB1);
        wait_vmem();
        __syncthreads();
      }
      if (kc < nk) {
        compute(sA0, sB0);
        __syncthreads();
      }

      // ---- token norms: lane halves hold the two k-halves; the two waves sharing a row block
      // summed the same rows, wave (wm, 0) publishes A rows and wave (0, wn) B rows.
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const float s = sqA[mb] + __shfl_xor(sqA[mb], 32);
        if (wn == 0 && lane < 32) sm.sq[0][0][wm * 128 + mb * 32 + lane] = s;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float s = sqB[nb] + __shfl_xor(sqB[nb], 32);
        if (wm == 0 && lane < 32) sm.sq[1][0][wn * 128 + nb * 32 + lane] = s;
      }
      __syncthreads();
      {
        const int r = tid;
        const int slotA = qi * TILE + r, slotB = qj * TILE + r;
        const bool vA = slotA < a.S && baseI + slotA < a.N;
        const bool vB = slotB < a.S && baseJ + slotB < a.N;
        const float ssA = sm.sq[0][0][r];
        const float ssB = sm.sq[1][0][r];
        const float rnA = (vA && ssA > 0.f) ? 1.0f / sqrtf(ssA) : 0.f;
        const float rnB = (vB && ssB > 0.f) ? 1.0f / sqrtf(ssB) : 0.f;
        sm.sbA[r] = make_float2(rnA, vA ? 0.f : -INFINITY);
        sm.sbB[r] = make_float2(rnB, vB ? 0.f : -INFINITY);
        sm.rnA[slotA] = rnA;
        sm.rnB[slotB] = rnB;
      }
      __syncthreads();

      // ---- one pass over the accumulators, both directions:
      //   column u: max over this wave's rows t of C_tu * rn_t (padding rows -> -inf)
      //   row t:    max over this wave's columns u of C_tu * rn_u (padding columns -> -inf),
      //             written transposed to LDS; wave w uses stage buffer w as scratch.
      auto rp_of = [&](int w) -> float* {
        return reinterpret_cast<float*>(w == 0 ? sA0 : w == 1 ? sB0 : w == 2 ? sA1 : sB1);
      };
      float* rp = rp_of(wave);
      float csc[4], cbi[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float2 t = sm.sbB[wn * 128 + nb * 32 + (lane & 31)];
        csc[nb] = t.x;
        cbi[nb] = t.y;
      }
      float cm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = wm * 128 + mb * 32 + g * 8 + (lane >> 5) * 4;
          const float4 p01 = *reinterpret_cast<const float4*>(&sm.sbA[r0]);
          const float4 p23 = *reinterpret_cast<const float4*>(&sm.sbA[r0 + 2]);
          const float rsc[4] = {p01.x, p01.z, p23.x, p23.z};
          const float rbi[4] = {p01.y, p01.w, p23.y, p23.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = g * 4 + e;
            float m = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const float c = acc[mb][nb][v];
              m = fmaxf(m, fmaf(c, csc[nb], cbi[nb]));
              cm[nb] = fmaxf(cm[nb], fmaf(c, rsc[e], rbi[e]));
            }
            rp[(mb * 32 + g * 8 + (lane >> 5) * 4 + e) * RP_STRIDE + (lane & 31)] = m;
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float m = fmaxf(cm[nb], __shfl_xor(cm[nb], 32));
        if (lane < 32) sm.cm[wm][wn * 128 + nb * 32 + lane] = m;
      }
      __syncthreads();
      {
        const int r = tid, wr = r >> 7, rl = r & 127;
        const float* p0 = rp_of(wr * 2 + 0) + rl * RP_STRIDE;
        const float* p1 = rp_of(wr * 2 + 1) + rl * RP_STRIDE;
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const float4 u = *reinterpret_cast<const float4*>(p0 + c);
          const float4 w = *reinterpret_cast<const float4*>(p1 + c);
          m = fmaxf(m, fmaxf(fmaxf(u.x, u.y), fmaxf(u.z, u.w)));
          m = fmaxf(m, fmaxf(fmaxf(w.x, w.y), fmaxf(w.z, w.w)));
        }
        const int sA = qi * TILE + r;
        sm.rowmax[sA] = (qj == 0) ? m : fmaxf(sm.rowmax[sA], m);
        const float cmv = fmaxf(sm.cm[0][r], sm.cm[1][r]);
        const int sB = qj * TILE + r;
        sm.colmax[sB] = (qi == 0) ? cmv : fmaxf(sm.colmax[sB], cmv);
      }
      __syncthreads();
    }
  }

  // ---- sums over valid tokens, fixed reduction order (bitwise reproducible)
  float sr = 0.f, sc = 0.f;
  for (int t = tid; t < Q * TILE; t += 256) {
    if (t < a.S && baseI + t < a.N) sr += sm.rnA[t] * sm.rowmax[t];
    if (t < a.S && baseJ + t < a.N) sc += sm.rnB[t] * sm.colmax[t];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sr += __shfl_xor(sr, o);
    sc += __shfl_xor(sc, o);
  }
  if (lane == 0) {
    sm.red[wave] = sr;
    sm.red[4 + wave] = sc;
  }
  __syncthreads();
  if (tid == 0) {
    const float tr = ((sm.red[0] + sm.red[1]) + sm.red[2]) + sm.red[3];
    const float tc = ((sm.red[4] + sm.red[5]) + sm.red[6]) + sm.red[7];
    float* sb = a.scores + b * (int64_t)a.n_s * a.n_s;
    sb[(int64_t)i * a.n_s + j] = tr;
    sb[(int64_t)j * a.n_s + i] = tc;
    if (j == i + 1) {
      sb[(int64_t)i * a.n_s + i] = -INFINITY;
      if (j == a.n_s - 1) sb[(int64_t)j * a.n_s + j] = -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_maxsim_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld_x, int S,
                              float* scores, hipStream_t stream) {
  MaxsimParams p;
  p.x = x;
  p.N = N;
  p.ld_x = ld_x;
  p.d = d;
  p.S = S;
  p.n_s = (int)((N + S - 1) / S);
  p.q = (S + TILE - 1) / TILE;
  p.pairs = (int64_t)p.n_s * (p.n_s - 1) / 2;
  p.tiles = B * p.pairs;
  p.scores = scores;
  if (p.q == 1)
    hipLaunchKernelGGL(maxsim_bf16_kernel<1>, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(maxsim_bf16_kernel<2>, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
