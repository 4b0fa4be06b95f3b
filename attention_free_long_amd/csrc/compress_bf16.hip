// Weighted gather + neural compression on bf16 MFMA (gfx950).
//
// For split i: Xhat_i = P X_cat + X_i with X_cat = [X_i; w_1 X_{j_1}; ...; w_k X_{j_k}]
// (papernotes.org Avey-B note, 关键设计 4, eq. 8; retrieved splits scaled by their normalised
// scores per 方法详解/整体框架; residual to the split's own tokens per the paperlayer.ai
// "Avey-B" summary, appendix H). X_cat is never materialised: the K dimension of the GEMM
// (k+1)S walks the gathered splits through idx, one 64-token chunk at a time.
//
// The product is computed transposed, C[f][s] = sum_kk X_cat[kk][f] P[s][kk], so that each lane
// of the result owns one output token and four consecutive features (8-byte stores). Both MFMA
// operands must be K-contiguous in LDS: P rows already are and are copied straight from
// global memory into LDS; X_cat is token-major, so each thread loads an 8 token x 8 feature
// block with 16-byte loads along the features, scales it by w in fp32 (bf16 round to nearest
// even), transposes it in registers and writes eight 16-byte rows of the feature-major tile.
// Tokens past N (zero padding of the last split) load as zero through the buffer descriptor.
//
// Workgroup: 256 threads, 256 features x 256 output tokens, 4 waves of 128 x 128.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int TILE = 256;

struct CompressParams {
  const uint16_t* x;
  const int32_t* idx;
  const float* w;
  const uint16_t* P;
  uint16_t* xhat;
  int64_t N, ld_x, ld_out, tiles;
  int d, S, k, n_s, s_tiles, f_tiles, residual;
};

__global__ void __launch_bounds__(256, 1) compress_bf16_kernel(CompressParams a) {
  // A: X_cat^T rows (features), SWZ_DIAG. B: P rows (output tokens), SWZ_ROW.
  __shared__ __align__(16) uint8_t sA0[TILE * ROWB], sB0[TILE * ROWB], sA1[TILE * ROWB], sB1[TILE * ROWB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 1, wn = wave & 1;

  const int64_t L = xcd_remap(blockIdx.x, a.tiles);
  const int ft = (int)(L % a.f_tiles);
  const int64_t rest = L / a.f_tiles;
  const int st = (int)(rest % a.s_tiles);
  const int64_t split = rest / a.s_tiles;
  const int64_t b = split / a.n_s;
  const int i = (int)(split % a.n_s);

  const uint16_t* xb = a.x + b * a.N * a.ld_x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(xb, (uint32_t)(a.N * a.ld_x * 2));
  const int KP = (a.k + 1) * a.S;          // row length of P
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P, (uint32_t)((int64_t)a.S * KP * 2));
  const int32_t* idx_i = a.idx + split * a.k;
  const float* w_i = a.w + split * a.k;
  const int nk = KP / KC;

  // A staging role: features f0..f0+7 of chunk tokens 8 tg .. 8 tg + 7.
  const int fg = tid & 31, tg = tid >> 5;
  const int f0 = ft * TILE + fg * 8;
  const bool f_ok = f0 < a.d;
  // B copy role: P rows, eight per instruction, lane -> (row, LDS chunk position).
  const int ld_sub = lane >> 3, ld_pos = lane & 7;
  uint32_t offB[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = wave * 64 + n * 8 + ld_sub;
    const uint32_t c = (uint32_t)(ld_pos ^ (int)swz<SWZ_ROW>(row));
    const int s = st * TILE + row;
    offB[n] = s < a.S ? (uint32_t)(s * KP * 2) + 16u * c : OOB;
  }
  uint32_t fa[4], fb[4];
  frag_offsets<SWZ_DIAG>(fa, wm * 128, lane);
  frag_offsets<SWZ_ROW>(fb, wn * 128, lane);

  uint4 stA[8];
  float wt = 1.f;
  // Issue the copies / loads of chunk kc: P rows straight into LDS (dB), X rows into registers.
  auto issue = [&](int kc, uint8_t* dB) {
    const int kk0 = kc * KC;
    const int blk = kk0 / a.S;
    int src = blk ? idx_i[blk - 1] : i;
    src = min(max(src, 0), a.n_s - 1);
    wt = blk ? w_i[blk - 1] : 1.f;
    const int64_t tok0 = (int64_t)src * a.S + (kk0 - blk * a.S) + tg * 8;
    const uint32_t kb = (uint32_t)kk0 * 2;
#pragma unroll
    for (int n = 0; n < 8; ++n) dma16(pr, dB + (wave * 64 + n * 8) * ROWB, offB[n], kb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = tok0 + e;
      const uint32_t off = (f_ok && t < a.N) ? (uint32_t)((t * a.ld_x + f0) * 2) : OOB;
      stA[e] = buf_load16(xr, off, 0);
    }
  };
  // Weight and transpose the staged 8 x 8 block into rows f0..f0+7 of the A tile. The current
  // split has weight 1, for which bf16 -> fp32 -> x1 -> bf16 is exact.
  auto put = [&](uint8_t* dA) {
    uint32_t in[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      in[e][0] = stA[e].x; in[e][1] = stA[e].y; in[e][2] = stA[e].z; in[e][3] = stA[e].w;
    }
#pragma unroll
    for (int ff = 0; ff < 8; ++ff) {
      uint32_t o[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = in[2 * m][ff >> 1], hi = in[2 * m + 1][ff >> 1];
        const float a0 = (ff & 1) ? bf16hi(lo) : bf16lo(lo);
        const float a1 = (ff & 1) ? bf16hi(hi) : bf16lo(hi);
        o[m] = pack_bf16(a0 * wt, a1 * wt);
      }
      lds_write16(dA, lds_off<SWZ_DIAG>(fg * 8 + ff, tg), make_uint4(o[0], o[1], o[2], o[3]));
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
    uint4 ra[2][4], rb[2][4];
    auto fetch = [&](int ks, int slot) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) ra[slot][mb] = lds_read16(sa, fa[frag_ks<SWZ_DIAG>(ks, mb)] + mb * 32 * ROWB);
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
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  issue(0, sB0);
  put(sA0);
  wait_vmem();
  __syncthreads();
  int kc = 0;
  for (; kc + 2 <= nk; kc += 2) {
    issue(kc + 1, sB1);
    compute(sA0, sB0);
    put(sA1);
    wait_vmem();
    __syncthreads();
    const bool more = kc + 2 < nk;
    if (more) issue(kc + 2, sB0);
    compute(sA1, sB1);
    if (more) put(sA0);
    wait_vmem();
    __syncthreads();
  }
  if (kc < nk) {
    compute(sA0, sB0);
    __syncthreads();
  }

  // Epilogue: lane owns token s, four consecutive features per (mb, g).
  uint16_t* ob = a.xhat + b * a.N * a.ld_out;
  const float rf = a.residual ? 1.f : 0.f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int s = st * TILE + wn * 128 + nb * 32 + (lane & 31);
    const int64_t tok = (int64_t)i * a.S + s;
    if (s >= a.S || tok >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = ft * TILE + wm * 128 + mb * 32 + g * 8 + (lane >> 5) * 4;
        if (f >= a.d) continue;
        float v0 = acc[mb][nb][g * 4 + 0], v1 = acc[mb][nb][g * 4 + 1];
        float v2 = acc[mb][nb][g * 4 + 2], v3 = acc[mb][nb][g * 4 + 3];
        const uint2 r = buf_load8(xr, (uint32_t)((tok * a.ld_x + f) * 2), 0);
        v0 = fmaf(rf, bf16lo(r.x), v0); v1 = fmaf(rf, bf16hi(r.x), v1);
        v2 = fmaf(rf, bf16lo(r.y), v2); v3 = fmaf(rf, bf16hi(r.y), v3);
        *reinterpret_cast<uint2*>(ob + tok * a.ld_out + f) = make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
      }
  }
}

}  // namespace

hipError_t launch_compress_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld_x, int S, int k,
                                const int32_t* idx, const float* w, const uint16_t* P, int residual, uint16_t* xhat,
                                int64_t ld_out, hipStream_t stream) {
  CompressParams p;
  p.x = x; p.idx = idx; p.w = w; p.P = P; p.xhat = xhat;
  p.N = N; p.ld_x = ld_x; p.ld_out = ld_out;
  p.d = d; p.S = S; p.k = k;
  p.n_s = (int)((N + S - 1) / S);
  p.s_tiles = (S + TILE - 1) / TILE;
  p.f_tiles = (d + TILE - 1) / TILE;
  p.residual = residual;
  p.tiles = B * p.n_s * p.s_tiles * p.f_tiles;
  hipLaunchKernelGGL(compress_bf16_kernel, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
