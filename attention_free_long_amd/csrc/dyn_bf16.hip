// Dynamic contextualizer core on bf16 MFMA (gfx950).
//
// Per split: G = N(Z_t) N(Z_t)^T over the split's valid tokens, r_p = sum_q G_pq and
// out_p = sum_q G_pq z_q / (r_p + eps) (papernotes.org Avey-B note, 关键设计 2 for the cosine
// mixing of the un-normalised tail, 关键设计 3 / eq. 6 for the row normalisation).
//
// Two GEMMs per workgroup, G never leaves the registers:
//  1. C1[q][p] = sum_k z_q[k] z_p[k] over k < m_t, for all q of the split and this wave's p.
//     In the MFMA result layout each lane owns one p (column) and 16 q (rows) per block, which
//     is exactly the B-operand layout the second GEMM needs along its K = q axis (up to a
//     fixed permutation of q inside each 16-row group, applied identically to both operands).
//     Token norms come from LDS fragments the waves read anyway where possible.
//  2. O[f][p] = sum_q Z^T[f][q] G[q][p]: Z^T tiles (128 features x 64 tokens) are staged
//     feature-major through a register transpose that also applies the q permutation; the
//     result lane owns token p and four consecutive features (8-byte stores), scaled by
//     1 / (r_p + eps). G is rounded to bf16 for this product and r_p is summed from the
//     rounded values, so the applied weights sum to r_p / (r_p + eps).
//
// Template: NQB = q blocks of 32 covering the split (8 for S <= 256, 16 for S <= 512); NPB = p
// blocks per wave (2 or 1), so one workgroup covers 4 * NPB * 32 tokens p.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

struct DynParams {
  const uint16_t* z;
  uint16_t* out;
  int64_t N, ld_z, ld_out, tiles;
  int m_t, S, n_s, pgroups;
  float eps;
};

template <int NQB, int NPB>
__global__ void __launch_bounds__(256, 1) dyn_bf16_kernel(DynParams a) {
  constexpr int QROWS = NQB * 32;
  constexpr int PWG = 4 * NPB * 32;
  constexpr int LROWS = QROWS / 4;       // Z rows copied per wave in GEMM 1
  constexpr int LN = LROWS / 8;          // copy instructions per wave per chunk
  // Norms of the q rows: when this workgroup's p rows are all the split's rows, each wave sums
  // its own p fragments; otherwise every wave also reads the fragments of 128 q rows of its own.
  constexpr bool kNormFromP = (PWG == QROWS);
  constexpr int NNB = kNormFromP ? NPB : 4;   // norm fragments per k-step
  __shared__ __align__(16) uint8_t sZ0[QROWS * ROWB], sZ1[QROWS * ROWB];
  __shared__ float s_sq[QROWS];
  __shared__ __align__(16) float s_rn[QROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);

  const int64_t L = xcd_remap(blockIdx.x, a.tiles);
  const int pg = (int)(L % a.pgroups);
  const int64_t split = L / a.pgroups;
  const int64_t b = split / a.n_s;
  const int i = (int)(split % a.n_s);
  const int64_t base = (int64_t)i * a.S;
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z + b * a.N * a.ld_z, (uint32_t)(a.N * a.ld_z * 2));
  const int nk = a.m_t / KC;

  // ------------------------------------------------------------------ GEMM 1
  const int ld_sub = lane >> 3, ld_pos = lane & 7;
  uint32_t offZ[LN];
#pragma unroll
  for (int n = 0; n < LN; ++n) {
    const int row = wave * LROWS + n * 8 + ld_sub;
    const uint32_t c = (uint32_t)(ld_pos ^ (int)swz<SWZ_ROW>(row));
    const bool v = row < a.S && base + row < a.N;
    offZ[n] = v ? (uint32_t)((base + row) * a.ld_z * 2) + 16u * c : OOB;
  }
  const int prow0 = pg * PWG + wave * NPB * 32;   // this wave's first p (split-local)
  const int nrow0 = kNormFromP ? prow0 : wave * 128;
  uint32_t fq[4], fp[4], fn[4];
  frag_offsets<SWZ_ROW>(fq, 0, lane);
  frag_offsets<SWZ_ROW>(fp, prow0, lane);
  frag_offsets<SWZ_ROW>(fn, nrow0, lane);

  f32x16 acc1[NQB][NPB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int nb = 0; nb < NPB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc1[qb][nb][v] = 0.f;
  float sq[NNB];
#pragma unroll
  for (int j = 0; j < NNB; ++j) sq[j] = 0.f;

  auto dma1 = [&](int kc, uint8_t* dst) {
#pragma unroll
    for (int n = 0; n < LN; ++n) dma16(zr, dst + (wave * LROWS + n * 8) * ROWB, offZ[n], (uint32_t)kc * KC * 2);
  };
  auto compute1 = [&](const uint8_t* s) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 rb[NPB];
#pragma unroll
      for (int nb = 0; nb < NPB; ++nb) rb[nb] = lds_read16(s, fp[ks] + nb * 32 * ROWB);
      if constexpr (kNormFromP) {
#pragma unroll
        for (int nb = 0; nb < NPB; ++nb) sq[nb] = sumsq8(rb[nb], sq[nb]);
      } else {
#pragma unroll
        for (int j = 0; j < NNB; ++j) sq[j] = sumsq8(lds_read16(s, fn[ks] + j * 32 * ROWB), sq[j]);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const uint4 ra = lds_read16(s, fq[ks] + qb * 32 * ROWB);
#pragma unroll
        for (int nb = 0; nb < NPB; ++nb) acc1[qb][nb] = mfma32(as_bf16x8(ra), as_bf16x8(rb[nb]), acc1[qb][nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  dma1(0, sZ0);
  wait_vmem();
  __syncthreads();
  int kc = 0;
  for (; kc + 2 <= nk; kc += 2) {
    dma1(kc + 1, sZ1);
    compute1(sZ0);
    wait_vmem();
    __syncthreads();
    if (kc + 2 < nk) dma1(kc + 2, sZ0);
    compute1(sZ1);
    wait_vmem();
    __syncthreads();
  }
  if (kc < nk) {
    compute1(sZ0);
    __syncthreads();
  }

  // token norms (lane halves hold the two k-halves)
#pragma unroll
  for (int j = 0; j < NNB; ++j) {
    const float t = sq[j] + __shfl_xor(sq[j], 32);
    if (lane < 32) s_sq[nrow0 + j * 32 + lane] = t;
  }
  __syncthreads();
  for (int q = tid; q < QROWS; q += 256) {
    const float ss = s_sq[q];
    const bool v = q < a.S && base + q < a.N;
    s_rn[q] = (v && ss > 0.f) ? 1.0f / sqrtf(ss) : 0.f;
  }
  __syncthreads();

  // G (bf16) as GEMM-2 B fragments, and r_p from the rounded values
  uint4 gfrag[NQB][2][NPB];
  float inv[NPB];
#pragma unroll
  for (int nb = 0; nb < NPB; ++nb) {
    const float rnp = s_rn[prow0 + nb * 32 + (lane & 31)];
    float r = 0.f;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q0 = qb * 32 + s2 * 16 + h * 8 + (lane >> 5) * 4;   // rows of v = 8*s2 + 4*h + 0..3
          const float4 rq = *reinterpret_cast<const float4*>(&s_rn[q0]);
          const int v0 = s2 * 8 + h * 4;
          const float g0 = acc1[qb][nb][v0 + 0] * rq.x * rnp;
          const float g1 = acc1[qb][nb][v0 + 1] * rq.y * rnp;
          const float g2 = acc1[qb][nb][v0 + 2] * rq.z * rnp;
          const float g3 = acc1[qb][nb][v0 + 3] * rq.w * rnp;
          pk[2 * h + 0] = pack_bf16(g0, g1);
          pk[2 * h + 1] = pack_bf16(g2, g3);
          r += (bf16lo(pk[2 * h]) + bf16hi(pk[2 * h])) + (bf16lo(pk[2 * h + 1]) + bf16hi(pk[2 * h + 1]));
        }
        gfrag[qb][s2][nb] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
    r += __shfl_xor(r, 32);
    inv[nb] = 1.0f / (r + a.eps);
  }

  // ------------------------------------------------------------------ GEMM 2
  constexpr int FT = 128;                 // features per output tile
  constexpr int NQC = QROWS / KC;         // 64-token chunks along K = q
  const int nft = (a.m_t + FT - 1) / FT;
  const int total = nft * NQC;
  // staging role: 4 features x 8 tokens; the 8 tokens are the ones a lane half feeds to
  // one k-step: 16g + 4h + {0..3} and 16g + 8 + 4h + {0..3} (g = tg >> 1, h = tg & 1)
  const int fg = tid & 31, tg = tid >> 5;
  const int qoff = 16 * (tg >> 1) + 4 * (tg & 1);
  uint32_t fz[4];
  frag_offsets<SWZ_DIAG>(fz, 0, lane);
  uint2 st2[8];
  auto gload2 = [&](int c) {
    const int ft = c / NQC, qc = c % NQC;
    const int f0 = ft * FT + fg * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = qc * KC + qoff + (e & 3) + ((e >> 2) << 3);
      const bool v = f0 < a.m_t && q < a.S && base + q < a.N;
      st2[e] = buf_load8(zr, v ? (uint32_t)(((base + q) * a.ld_z + f0) * 2) : OOB, 0);
    }
  };
  auto put2 = [&](uint8_t* dst) {
#pragma unroll
    for (int ff = 0; ff < 4; ++ff) {
      uint32_t o[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (ff >> 1) ? st2[2 * m].y : st2[2 * m].x;
        const uint32_t hi = (ff >> 1) ? st2[2 * m + 1].y : st2[2 * m + 1].x;
        o[m] = pick16(lo, hi, ff & 1);
      }
      lds_write16(dst, lds_off<SWZ_DIAG>(fg * 4 + ff, tg), make_uint4(o[0], o[1], o[2], o[3]));
    }
  };

  f32x16 acc2[4][NPB];
  auto zero2 = [&]() {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int nb = 0; nb < NPB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc2[fb][nb][v] = 0.f;
  };
  zero2();
  auto compute2 = [&](const uint8_t* s, auto qc_tag) {
    constexpr int qc = decltype(qc_tag)::value;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 ra[4];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) ra[fb] = lds_read16(s, fz[frag_ks<SWZ_DIAG>(ks, fb)] + fb * 32 * ROWB);
      const int qb = qc * 2 + (ks >> 1);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int nb = 0; nb < NPB; ++nb)
          acc2[fb][nb] = mfma32(as_bf16x8(ra[fb]), as_bf16x8(gfrag[qb][ks & 1][nb]), acc2[fb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  uint16_t* ob = a.out + b * a.N * a.ld_out;
  auto epilogue = [&](int ft) {
#pragma unroll
    for (int nb = 0; nb < NPB; ++nb) {
      const int p = prow0 + nb * 32 + (lane & 31);
      const int64_t tok = base + p;
      if (p >= a.S || tok >= a.N) continue;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = ft * FT + fb * 32 + g * 8 + (lane >> 5) * 4;
          if (f >= a.m_t) continue;
          const float sc = inv[nb];
          const uint32_t lo = pack_bf16(acc2[fb][nb][g * 4 + 0] * sc, acc2[fb][nb][g * 4 + 1] * sc);
          const uint32_t hi = pack_bf16(acc2[fb][nb][g * 4 + 2] * sc, acc2[fb][nb][g * 4 + 3] * sc);
          *reinterpret_cast<uint2*>(ob + tok * a.ld_out + f) = make_uint2(lo, hi);
        }
    }
  };

  // Chunk c = ft * NQC + qc; NQC is even, so chunk parity = qc parity and the stage buffer of
  // every chunk is known at compile time.
  static_assert(NQC % 2 == 0, "q chunks per feature tile must be even");
  gload2(0);
  put2(sZ0);
  __syncthreads();
  if (total > 1) gload2(1);
  for (int ft = 0; ft < nft; ++ft) {
    static_for<NQC>([&](auto qc_tag) {
      constexpr int qc = decltype(qc_tag)::value;
      const int c = ft * NQC + qc;
      compute2(qc % 2 == 0 ? sZ0 : sZ1, qc_tag);
      if (c + 1 < total) {
        put2(qc % 2 == 0 ? sZ1 : sZ0);
        if (c + 2 < total) gload2(c + 2);
      }
      __syncthreads();
    });
    epilogue(ft);
    zero2();
  }
}

template <int NQB, int NPB>
hipError_t launch_dyn_t(DynParams p, hipStream_t stream) {
  constexpr int PWG = 4 * NPB * 32;
  p.pgroups = (p.S + PWG - 1) / PWG;
  p.tiles = (int64_t)p.pgroups * p.tiles;   // tiles held B * n_s on entry
  hipLaunchKernelGGL((dyn_bf16_kernel<NQB, NPB>), dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dyn_bf16(const uint16_t* z, int64_t B, int64_t N, int m_t, int64_t ld_z, int S, float eps,
                           uint16_t* out, int64_t ld_out, hipStream_t stream) {
  DynParams p;
  p.z = z; p.out = out;
  p.N = N; p.ld_z = ld_z; p.ld_out = ld_out;
  p.m_t = m_t; p.S = S; p.eps = eps;
  p.n_s = (int)((N + S - 1) / S);
  p.tiles = B * p.n_s;
  p.pgroups = 1;
  if (S <= 256) return launch_dyn_t<8, 2>(p, stream);
  return launch_dyn_t<16, 1>(p, stream);
}

}  // namespace avey
